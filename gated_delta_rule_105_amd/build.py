"""Build the HIP library ``libkda.so`` in-tree for gfx950.

``python -m gated_delta_rule_105_amd.build`` compiles the KDA sources under
``csrc/`` with hipcc into ``gated_delta_rule_105_amd/libkda.so``, and the
device-peak microbenchmarks (``csrc/kda_peaks.hip``, a measurement aid for
bench.py) into ``libkda_peaks.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_prefill.hip", "kda_decode.hip", "kda_backward.hip"]
PEAKS_SOURCES = ["kda_peaks.hip"]
PEAKS_LIBRARY = os.path.join(HERE, "libkda_peaks.so")
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the KDA library needs ROCm to build")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        # packed fp32 VALU ops are kept out of generated code on purpose
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIBRARY, verbose)
    _compile(PEAKS_SOURCES, PEAKS_LIBRARY, verbose)
    return LIBRARY


def _compile(sources, library: str, verbose: bool) -> None:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = library + ".tmp"
    cmd = [hipcc(), *flags(), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)
    os.replace(tmp, library)


if __name__ == "__main__":
    print(build(verbose=True))
