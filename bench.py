"""Throughput of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one ``kda_chunk_forward`` over the prefill workload B=1, H=16,
T=4096, d_k=d_v=128, chunk 64, bf16 q/k/v/g/o, fp32 beta and state, nonzero
initial state (the workload the headline tokens/s figure is quoted on).  The
decode leg then times ``kda_decode_step`` on 256 sequences x 32 heads,
d=128, fp32 state [256, 32, 128, 128] updated in place, over consecutive steps
with fresh pre-staged inputs per step.  Inputs are seeded synthetic tensors
(package ``synth``) already resident in device memory when timing starts.

The prefill inputs are replicated over enough distinct buffer sets that their
total exceeds the 256 MB last-level cache several times; consecutive steps
cycle through them, so each step reads its inputs from HBM, not from cache.

Prints ONE JSON line.  ``roofline`` describes the dominant launch of the
chunked forward (the one with the largest mean duration, from HIP events
recorded on the launch stream between the call's launches): its share of the
algorithmic bytes (``LAUNCH_WORK``) divided by its mean duration, against HBM;
``call_roofline`` and ``mfma`` do the same for the whole call.
``cpu_baseline`` times the fp64 CPU oracle on the host cores (a baseline, not
a target).  ``other_workloads`` times the packed 8-sequence batch, the
1,048,576-token context and a serving-like batch (512 packed sequences of
64-512 tokens, H=32); ``states_workloads`` times the headline call with
prefix-cache states (kda_chunk_forward_states) beside plain calls;
``gate_workloads`` times Gated DeltaNet and DeltaNet gates beside KDA on the
prefill and decode workloads; ``mx_workload`` the headline workload with q,
k, v in MXFP8 (kda_chunk_forward_mx); ``backward_workload`` the backward pass
(kda_chunk_backward) on the headline workload, ``backward_long_workload``
at T = 65,536 with its default (windowed) workspace; ``cold`` the headline, packed
and million-token workloads as the median of calls each preceded by a 1 GiB
write that flushes L2 and the last-level cache; ``gpu_clock`` the graphics
clock under load; ``device_peaks`` the device's own measured peaks (dense
bf16 and fp32 MFMA loops, an HBM read sweep, a device copy) beside the
nominal ones; ``roofline_fraction`` the larger of the call's HBM and MFMA
fractions.  Other legs: ``--copy-calib MiB`` runs only a device copy of known
size (for scaling the HBM byte counters), ``--only
prefill|decode|backward|peaks`` runs one leg, ``--no-cpu`` skips the oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
LLC_BYTES = 256 << 20          # MI355X last-level (infinity) cache

# Algorithmic work and compulsory traffic of the chunked forward per (token,
# head) at d_k = d_v = 128, chunk 64 (multiply-adds counted over the needed
# triangles only, FLOP = 2 MAC):
#   3 d^2                     state products Wk S, Qt S, Kb^T U
#   d (C - 1) / 2             strict-lower key Gram
#   4 d (C + 1) / 2           Wk, Wv, P, P U (lower triangles incl. diagonal)
#   (C - 1)(C - 2) / 6        triangular inverse
FLOP_PER_TOKEN_HEAD = 2 * (3 * 128 * 128 + 128 * 63 // 2 + 4 * 128 * 65 // 2 + 63 * 62 // 6)
# The same products as full 64 x 64 tiles (what dense MFMA tiles issue for
# the key Gram, P, Wk, Wv and P U; the inverse not counted): per (token, head)
#   3 d^2 + 5 d C, FLOP = 2 MAC
ISSUED_FLOP_PER_TOKEN_HEAD = 2 * (3 * 128 * 128 + 5 * 128 * 64)
# bf16 q, k, v, g read + bf16 o written (2 B x 128 each) + fp32 beta
BYTES_PER_TOKEN_HEAD = 5 * 2 * 128 + 4
STATE_BYTES = 128 * 128 * 4    # one fp32 state matrix (h0 read, ht written)

# The same work per launch (per token and head).  The output sweep does the
# whole algorithmic work of the call: it reads every input, recomputes the
# chunk-local algebra, applies the state and writes o (plus ht per sequence
# and head).  The map sweep (composes each segment's affine state map from
# k, v, g, beta) and the segment scan are extra work of the segment
# decomposition: the map sweep's figures are its own compulsory reads and
# products (chunk-local key Gram, Wk, Wv, inverse; U = Wv - Wk B, Kh^T U,
# Wk M, Kh^T (Wk M) on the map), with no share of the call's algorithmic
# figures.
LAUNCH_WORK = {
    "kda_chunk_sweep_map": dict(bytes=3 * 2 * 128 + 4,
                                flop=2 * (128 * 63 // 2 + 2 * 128 * 65 // 2 + 63 * 62 // 6 + 4 * 128 * 128)),
    "kda_seg_scan": dict(bytes=0, flop=0),
    "kda_chunk_sweep_out": dict(bytes=BYTES_PER_TOKEN_HEAD, flop=FLOP_PER_TOKEN_HEAD),
}

# Backward pass (kda_chunk_backward) per (token, head) at d = 128, C = 64.
# Algorithmic multiply-adds beyond the forward replay (needed triangles only):
#   chunk-local recompute   d (C - 1) / 2 + 3 d (C + 1) / 2 + (C - 1)(C - 2) / 6
#   state products          7 d^2   (Wk S, Kh dH, Qt^T dO, Wk^T dU, dU S^T, dO S^T, U dH^T)
#   chunk-scaled products   6 d (C + 1) / 2 (P^T dO, dP, T^T dU, T^T dWk, dP Kh, dP^T Qt)
#                           + 4 d (C - 1) / 2 (dA: two products, dA Kh, dA^T Kt)
# plus the replay (FLOP_PER_TOKEN_HEAD).  Compulsory bytes: bf16 q, k, v, g,
# do read, bf16 dq, dk, dv, dg written (256 B each), fp32 beta read and dbeta
# written, plus h0 and dht read and dh0 written per (sequence, head).
BWD_MAC_PER_TOKEN_HEAD = (128 * 63 // 2 + 3 * 128 * 65 // 2 + 63 * 62 // 6 + 7 * 128 * 128
                          + 6 * 128 * 65 // 2 + 4 * 128 * 63 // 2)
BWD_FLOP_PER_TOKEN_HEAD = 2 * BWD_MAC_PER_TOKEN_HEAD + FLOP_PER_TOKEN_HEAD
BWD_BYTES_PER_TOKEN_HEAD = 9 * 2 * 128 + 2 * 4
PEAK_F32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix (the backward's products run on fp32 MFMA)

PREFILL = dict(B=1, T=4096, H=16, d=128, wid=1)
DECODE = dict(N=256, H=32, d=128, wid=4)
CPU_SAMPLE_SECONDS = 10.0

PREFILL_SOURCES = ("kda_prefill.hip", "kda_rows.h", "kda_device.h", "kda_api.cpp", "kda_launch.h")
MFMA_PROFILE = "kda_mfma_util_prefill_T4096_H16_backward.txt"
BWD_SOURCES = ("kda_backward.hip", "kda_prefill.hip", "kda_rows.h", "kda_device.h", "kda_api.cpp", "kda_launch.h")
# the kernel of a backward stage where it is not the stage's own name (d = 128)
BWD_STAGE_KERNEL = {"kda_bwd_chunk": "kda_bwd_chunk_fused", "kda_bwd_local": "kda_bwd_local_fused"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_105_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, digest: str, key: str = "hbm_bytes_per_call", digest_key: str = "source_digest"):
    """HBM bytes per call (or the value of `key`) from a committed counter
    summary, if it was taken on the current kernel source, whose digest the
    file records under `digest_key` (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            name_, _, val = line.partition("=")
            vals[name_.strip()] = val.strip()
    if vals.get(digest_key) != digest or key not in vals:
        return None
    return float(vals[key])


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed prefill calls")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000, help="timed decode steps")
    ap.add_argument("--only", choices=("prefill", "decode", "backward", "peaks", "both"), default="both")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the packed and long-context workloads")
    ap.add_argument("--bwd-sequential", action="store_true",
                    help="backward leg: only kda_chunk_backward (one launch per kernel and call, for counters)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MiB",
                    help="only run device copies of this size (counter calibration)")
    return ap.parse_args()


def copy_calib(mib: int) -> None:
    import torch
    n = mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n, "dispatches": 5}))


def bench_prefill(steps: int, warmup: int):
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    B, T, H, d, wid = (PREFILL[k] for k in ("B", "T", "H", "d", "wid"))
    log(f"prefill inputs B={B} T={T} H={H} d={d} bf16 (generated on the GPU)")
    base = synth.prefill_inputs(B, T, H, d, d, "bf16", wid=wid, h0=True, device="cuda")
    set_bytes = 4 * base["q"].numel() * 2 + base["beta"].numel() * 4 + base["q"].numel() * 2
    n_sets = max(2, math.ceil(3 * LLC_BYTES / set_bytes))
    sets = []
    for i in range(n_sets):
        s = {key: base[key].clone() for key in ("q", "k", "v", "g", "beta", "h0")}
        s["o"] = torch.empty_like(base["q"])
        s["ht"] = torch.empty_like(base["h0"])
        sets.append(s)
    del base
    ws = torch.empty(kda.workspace_bytes(B, T, H, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call(s, events=None):
        kda.chunk_forward(s["q"], s["k"], s["v"], s["g"], s["beta"], h0=s["h0"], o=s["o"], ht=s["ht"],
                          workspace=ws, events=events)

    log(f"prefill warmup {warmup} over {n_sets} buffer sets of {set_bytes / 1e6:.1f} MB")
    for i in range(warmup):
        call(sets[i % n_sets])
    torch.cuda.synchronize()
    # timed region 1: plain calls back to back (throughput), one event pair
    # around the whole loop (no instrumentation between the calls)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        call(sets[i % n_sets])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_call = e0.elapsed_time(e1) * 1e-3 / steps
    # timed region 2: the same calls through kda_chunk_forward_timed, which
    # records HIP events on the launch stream before each launch and after
    # the last (per-launch durations; the events add a little to each)
    n_ev = len(kda.CHUNK_LAUNCHES) + 1
    evl = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for row in evl:
        for e in row:
            e.record(stream)  # creates the event
    torch.cuda.synchronize()
    handles = [[e.cuda_event for e in row] for row in evl]
    for i in range(steps):
        call(sets[i % n_sets], handles[i])
    torch.cuda.synchronize()
    launch = {name: sum(row[j].elapsed_time(row[j + 1]) for row in evl) / steps * 1e-3
              for j, name in enumerate(kda.CHUNK_LAUNCHES)}
    log(f"prefill {steps} calls: wall {wall * 1e3:.3f} ms, GPU time per call {mean_call * 1e6:.2f} us; per launch "
        + ", ".join(f"{n} {t * 1e6:.2f} us" for n, t in launch.items()))
    token_heads = B * T * H
    bytes_call = token_heads * BYTES_PER_TOKEN_HEAD + 2 * B * H * STATE_BYTES
    flop_call = token_heads * FLOP_PER_TOKEN_HEAD
    return dict(wall=wall, mean_call=mean_call, tokens=B * T, token_heads=token_heads,
                bytes_call=bytes_call, flop_call=flop_call, n_sets=n_sets, launch=launch)


def bench_workload(wid: int, calls: int):
    """Secondary prefill workloads (packed batch, long context): tokens/s."""
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    w = synth.WORKLOADS[wid]
    log(f"workload {w.name}: inputs generated on the GPU")
    inp = synth.workload_inputs(w, device="cuda")
    T = inp["q"].shape[1]
    n_seqs = 0 if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    ws = torch.empty(kda.workspace_bytes(1, T, w.H, w.dk, torch.bfloat16, n_seqs), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["q"])
    ht = torch.empty((n_seqs or 1, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")

    def call():
        kda.chunk_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], o=o, ht=ht, workspace=ws, validate_cu=False)

    call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    mean = sum(a.elapsed_time(b) for a, b in ev) / calls * 1e-3
    token_heads = T * w.H
    bytes_call = token_heads * BYTES_PER_TOKEN_HEAD + 2 * (n_seqs or 1) * w.H * STATE_BYTES
    log(f"workload {w.name}: {calls} calls, mean {mean * 1e6:.1f} us")
    del inp, o, ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "tokens": T, "heads": w.H, "mean_call_us": mean * 1e6,
            "value": T / mean, "unit": "tokens/s", "hbm_frac": bytes_call / mean / 1e9 / PEAK_HBM_GBS,
            "mfma_frac": token_heads * FLOP_PER_TOKEN_HEAD / mean / 1e12 / PEAK_BF16_TFLOPS}


def bench_cold(wid: int, reps: int, warm: int = 3):
    """One workload the cold way: `warm` untimed calls, then `reps` calls,
    each after a 1 GiB device write that evicts the inputs from L2 and the
    last-level cache, each bracketed by its own HIP event pair; the median."""
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    w = synth.WORKLOADS[wid]
    log(f"cold {w.name}: {warm} warm-up calls, then {reps} calls each after a 1 GiB flush")
    inp = synth.workload_inputs(w, device="cuda")
    T = inp["q"].shape[1]
    n_seqs = 0 if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    ws = torch.empty(kda.workspace_bytes(1, T, w.H, w.dk, torch.bfloat16, n_seqs), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["q"])
    ht = torch.empty((n_seqs or 1, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def call():
        kda.chunk_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], o=o, ht=ht, workspace=ws, validate_cu=False)

    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    times.sort()
    med = times[len(times) // 2] if len(times) % 2 else 0.5 * (times[len(times) // 2 - 1] + times[len(times) // 2])
    token_heads = T * w.H
    bytes_call = token_heads * BYTES_PER_TOKEN_HEAD + (1 + (1 if inp["h0"] is not None else 0)) * (n_seqs or 1) \
        * w.H * STATE_BYTES
    hbm = bytes_call / med / 1e9 / PEAK_HBM_GBS
    mfma = token_heads * FLOP_PER_TOKEN_HEAD / med / 1e12 / PEAK_BF16_TFLOPS
    log(f"cold {w.name}: median {med * 1e6:.1f} us (min {times[0] * 1e6:.1f}, max {times[-1] * 1e6:.1f})")
    del inp, o, ws, flush
    torch.cuda.empty_cache()
    return {"workload": w.name, "reps": reps, "median_call_us": med * 1e6, "min_call_us": times[0] * 1e6,
            "max_call_us": times[-1] * 1e6, "value": T / med, "unit": "tokens/s", "hbm_frac": hbm,
            "mfma_frac": mfma, "roofline_fraction": max(hbm, mfma)}


def device_peaks():
    """The device's own peaks, measured beside the nominal ones the rooflines
    use: dense bf16 and fp32 MFMA throughput (libkda_peaks.so: eight
    independent accumulation chains per wave on register operands, four
    workgroups of four waves per CU), HBM read bandwidth (a 4 GiB sum with
    16-byte non-temporal loads) and a 2 GiB device copy (bytes read +
    written)."""
    import ctypes
    import torch

    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "gated_delta_rule_105_amd",
                                   "libkda_peaks.so"))
    lib.kda_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_peak_flop_per_mfma.restype = ctypes.c_longlong
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return statistics.median(ts)

    n_wg = 4 * n_cu
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    res = {"compute_units": n_cu}
    for kind, name, iters in ((0, "bf16_mfma_tflops", 20000), (1, "fp32_mfma_tflops", 10000)):
        def run(it=iters, k=kind):
            st = lib.kda_peak_mfma(k, n_wg, it, ctypes.c_void_p(out.data_ptr()), sp)
            if st != 0:
                raise RuntimeError(f"kda_peak_mfma: HIP error {st}")
        run(100)
        torch.cuda.synchronize()
        t = timed(run, 5)
        flop = n_wg * 4 * iters * lib.kda_peak_chains() * lib.kda_peak_flop_per_mfma(kind)
        res[name] = flop / t / 1e12
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda")  # 4 GiB
    src.fill_(1.0)
    rn_wg = 8 * n_cu
    rout = torch.empty(rn_wg * 256, dtype=torch.float32, device="cuda")

    def read():
        st = lib.kda_peak_read(ctypes.c_void_p(src.data_ptr()), src.numel() // 4, rn_wg, ctypes.c_void_p(rout.data_ptr()), sp)
        if st != 0:
            raise RuntimeError(f"kda_peak_read: HIP error {st}")
    read()
    res["hbm_read_gbs"] = src.numel() * 4 / timed(read, 5) / 1e9
    del src
    a = torch.empty(1 << 29, dtype=torch.float32, device="cuda")  # 2 GiB
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)
    res["copy_gbs"] = 2 * a.numel() * 4 / timed(lambda: b.copy_(a), 5) / 1e9
    del a, b, out, rout
    torch.cuda.empty_cache()
    res["nominal"] = {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "fp32_mfma_tflops": PEAK_F32_MFMA_TFLOPS,
                      "hbm_gbs": PEAK_HBM_GBS, "sclk_mhz": 2400.0}
    log("device peaks: " + ", ".join(f"{k} {v:.1f}" if isinstance(v, float) else f"{k} {v}"
                                     for k, v in res.items() if k != "nominal"))
    return res


def gpu_clock():
    """The graphics clock while a long call runs: the current level of the
    device's sysfs clock table (MHz), beside the nominal peak clock."""
    import glob
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    w = synth.WORKLOADS[3]
    inp = synth.workload_inputs(w, device="cuda")
    T = inp["q"].shape[1]
    ws = torch.empty(kda.workspace_bytes(1, T, w.H, w.dk, torch.bfloat16), dtype=torch.uint8, device="cuda")
    kda.chunk_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0=inp["h0"], workspace=ws)
    sysfs = None
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if "*" in line:
                    val = line.split(":", 1)[1].replace("*", "").strip().lower()
                    sysfs = float(val.replace("mhz", "").strip())
                    break
        except (OSError, ValueError):
            continue
        if sysfs is not None:
            break
    torch.cuda.synchronize()
    del inp, ws
    torch.cuda.empty_cache()
    return {"sysfs_sclk_mhz": sysfs, "nominal_mhz": 2400.0}


def bench_states(calls: int):
    """Prefix-cache states (kda_chunk_forward_states) on the headline workload:
    the same calls with a state every 16 chunks (1,024 tokens) and every
    chunk, timed beside plain calls on the same inputs, so that the
    difference is the cost of the emission."""
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    w = synth.WORKLOADS[1]
    inp = synth.workload_inputs(w, device="cuda")
    B, T, H, d = inp["q"].shape
    ws = torch.empty(kda.workspace_bytes(B, T, H, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["q"])
    ht = torch.empty_like(inp["h0"])
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    stream = torch.cuda.current_stream()

    def mean_of(call):
        call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / calls * 1e-3

    plain = mean_of(lambda: kda.chunk_forward(*args, h0=inp["h0"], o=o, ht=ht, workspace=ws))
    out = []
    for every in (16, 1):
        st = torch.empty((B * (T // (64 * every)), H, d, d), dtype=torch.float32, device="cuda")
        t = mean_of(lambda: kda.chunk_forward_states(*args, h0=inp["h0"], states_every=every, states=st, o=o,
                                                     ht=ht, workspace=ws))
        log(f"states every {every} chunks: {st.shape[0]} states, mean {t * 1e6:.1f} us (plain {plain * 1e6:.1f} us)")
        out.append({"workload": f"{w.name} + a state every {64 * every} tokens", "states_every_chunks": every,
                    "states": st.shape[0], "state_bytes": st.numel() * 4, "mean_call_us": t * 1e6,
                    "plain_call_us": plain * 1e6, "overhead_us": (t - plain) * 1e6, "value": T / t,
                    "unit": "tokens/s"})
        del st
    del inp, o, ws
    torch.cuda.empty_cache()
    return out


def bench_gates(calls: int, steps: int):
    """The gate variants beside KDA on the same inputs: Gated DeltaNet (one
    log-decay per token and head: channel 0 of the KDA gate) and DeltaNet (no
    decay), on the headline prefill workload and on the decode workload."""
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    stream = torch.cuda.current_stream()

    def mean_of(call, n):
        call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / n * 1e-3

    w = synth.WORKLOADS[1]
    inp = synth.workload_inputs(w, device="cuda")
    B, T, H, d = inp["q"].shape
    ws = torch.empty(kda.workspace_bytes(B, T, H, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["q"])
    ht = torch.empty_like(inp["h0"])
    gates = {"kda": inp["g"], "gated-deltanet": inp["g"][..., 0].contiguous(), "deltanet": None}
    out = []
    for name, g in gates.items():
        t = mean_of(lambda: kda.chunk_forward(inp["q"], inp["k"], inp["v"], g, inp["beta"], h0=inp["h0"], o=o,
                                              ht=ht, workspace=ws), calls)
        log(f"prefill gate {name}: mean {t * 1e6:.1f} us")
        out.append({"workload": f"{w.name} gate={name}", "mean_call_us": t * 1e6, "value": T / t,
                    "unit": "tokens/s"})
    del inp, o, ws, gates
    N, H, d, wid = (DECODE[k] for k in ("N", "H", "d", "wid"))
    dec = synth.decode_inputs(N, H, d, d, 1, "bf16", wid=wid, device="cuda")
    state = dec["state"]
    od = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda")
    gates = {"kda": dec["g"][0], "gated-deltanet": dec["g"][0][..., 0].contiguous(), "deltanet": None}
    for name, g in gates.items():
        t = mean_of(lambda: kda.decode_step(dec["q"][0], dec["k"][0], dec["v"][0], g, dec["beta"][0], state, o=od),
                    steps)
        bytes_step = 2 * N * H * d * d * 4
        log(f"decode gate {name}: mean step {t * 1e6:.1f} us")
        out.append({"workload": f"kda-decode-bf16-N{N}-H{H}-d{d} gate={name}", "mean_step_us": t * 1e6,
                    "value": 1.0 / t, "unit": "steps/s", "hbm_frac": bytes_step / t / 1e9 / PEAK_HBM_GBS})
    del dec, state
    torch.cuda.empty_cache()
    return out


def bench_mx(calls: int):
    """MXFP8 q, k, v (kda_chunk_forward_mx) beside bf16 on the headline
    workload: the same values (q, k, v encoded once, g bf16), buffer sets
    rotated as in the headline leg so that every call reads from HBM."""
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    w = synth.WORKLOADS[1]
    base = synth.mxfp8_inputs(synth.workload_inputs(w, device="cuda"))
    B, T, H, d = base["q"].shape
    keys = ("q8", "q_scale", "k8", "k_scale", "v8", "v_scale", "g", "beta", "h0")
    set_bytes = sum(base[k_].numel() * base[k_].element_size() for k_ in keys[:-1])
    n_sets = max(2, math.ceil(3 * LLC_BYTES / set_bytes))
    sets = [{k_: base[k_].clone() for k_ in keys} for _ in range(n_sets)]
    ws = torch.empty(kda.workspace_bytes(B, T, H, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty_like(base["h0"])
    del base
    stream = torch.cuda.current_stream()
    it = [0]

    def call():
        x = sets[it[0] % n_sets]
        it[0] += 1
        kda.chunk_forward_mx(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["v8"], x["v_scale"], x["g"], x["beta"],
                             h0=x["h0"], o=o, ht=ht, workspace=ws)

    for _ in range(n_sets):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    mean = sum(a.elapsed_time(b) for a, b in ev) / calls * 1e-3
    log(f"mxfp8 inputs: {calls} calls over {n_sets} buffer sets, mean {mean * 1e6:.1f} us")
    del sets, ws, o
    torch.cuda.empty_cache()
    th = T * H
    in_bytes = th * (3 * d + 3 * d // 32 + 2 * d + 4)  # e4m3 q, k, v + scales + bf16 g + fp32 beta
    return {"workload": f"{w.name} q,k,v MXFP8 (e4m3 + scale per 32 channels)", "mean_call_us": mean * 1e6,
            "value": T / mean, "unit": "tokens/s", "input_bytes": in_bytes,
            "hbm_frac": (in_bytes + th * 2 * d + 2 * H * STATE_BYTES) / mean / 1e9 / PEAK_HBM_GBS}


def bench_backward(calls: int, with_cpu: bool = True, overlap: bool = True):
    """Backward pass on the prefill workload with N(0, 1) upstream gradients
    for o and ht: mean call of kda_chunk_backward_overlapped (the value) and
    of kda_chunk_backward, and per-stage durations (HIP events on the launch
    stream, kda_chunk_backward_timed)."""
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    w = synth.WORKLOADS[1]
    inp = synth.workload_inputs(w, device="cuda")
    inp.update(synth.grad_inputs(inp, w.wid, device="cuda"))
    B, T, H, d = inp["q"].shape
    ws = torch.empty(kda.backward_workspace_bytes(B, T, H, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    out = {}
    stream = torch.cuda.current_stream()

    def call(events=None, overlap=False):
        return kda.chunk_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["do"], h0=inp["h0"],
                                  dht=inp["dht"], out=out, workspace=ws, events=events, overlap=overlap)

    out.update(call())
    if overlap:
        call(overlap=True)
    torch.cuda.synchronize()

    def timed(overlap):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for a, b in ev:
            a.record(stream)
            call(overlap=overlap)
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / calls * 1e-3

    mean_seq = timed(False)
    mean = timed(True) if overlap else mean_seq
    n_ev = len(kda.BWD_STAGES) + 1
    evl = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(calls)]
    for row in evl:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for row in evl:
        call([e.cuda_event for e in row])
    torch.cuda.synchronize()
    stage = {name: sum(row[j].elapsed_time(row[j + 1]) for row in evl) / calls * 1e-3
             for j, name in enumerate(kda.BWD_STAGES)}
    token_heads = B * T * H
    flop = token_heads * BWD_FLOP_PER_TOKEN_HEAD
    byts = token_heads * BWD_BYTES_PER_TOKEN_HEAD + 3 * B * H * STATE_BYTES
    log(f"backward {calls} calls: mean {mean * 1e6:.1f} us overlapped, {mean_seq * 1e6:.1f} us sequential; per stage "
        + ", ".join(f"{n} {t * 1e6:.1f} us" for n, t in stage.items()))
    # the dominant stage against the fp32 matrix peak: its share of the
    # algorithmic products (the local-gradient kernel does all but the
    # chunk-local recompute and the three state-gradient products)
    mac_chunk = 128 * 63 // 2 + 3 * 128 * 65 // 2 + 63 * 62 // 6
    mac_state = 3 * 128 * 128 + 128 * 65 // 2
    stage_flop = {"forward_replay": FLOP_PER_TOKEN_HEAD, "kda_bwd_chunk": 2 * mac_chunk,
                  "kda_bwd_state": 2 * mac_state,
                  "kda_bwd_local": 2 * (BWD_MAC_PER_TOKEN_HEAD - mac_chunk - mac_state)}
    dom = max(stage, key=stage.get)
    dom_tf = stage_flop[dom] * token_heads / stage[dom] / 1e12
    del ws, out
    torch.cuda.empty_cache()
    cpu = None
    if with_cpu:
        # the oracle's gradient on a bounded sample: heads 0 and 1 of the same
        # inputs (token-heads per second, scaled to tokens/s of 16 heads)
        import oracle
        cpu_inp = {key: (val[:, :, :2].cpu() if key in ("q", "k", "v", "g", "beta", "do") else val)
                   for key, val in inp.items()}
        t0 = time.perf_counter()
        oracle.backward(cpu_inp["q"], cpu_inp["k"], cpu_inp["v"], cpu_inp["g"], cpu_inp["beta"], cpu_inp["do"],
                        h0=inp["h0"][:, :2].cpu(), dht=inp["dht"][:, :2].cpu())
        el = time.perf_counter() - t0
        cpu = {"value": T * 2 / el / H, "unit": "tokens/s", "cores": 2, "kind": "oracle",
               "sample": f"fp64 token-by-token gradient of heads 0-1 of the T={T} workload, {el:.1f} s on 2 threads "
                         "(one per head), scaled to 16 heads"}
        log(f"cpu oracle backward: {el:.2f} s for 2 heads")
    del inp
    return {"workload": "kda-backward-bf16-B1-H16-T4096-d128 (do, dht ~ N(0,1))", "mean_call_us": mean * 1e6,
            "call": ("kda_chunk_backward_overlapped (replay and the later chunks' local gradients on a second stream)"
                     if overlap else "kda_chunk_backward"),
            "sequential_call_us": mean_seq * 1e6,
            "cpu_baseline": cpu,
            "value": B * T / mean, "unit": "tokens/s",
            "stage_us": {n: t * 1e6 for n, t in stage.items()},
            "call_roofline": {"bound": "mfma", "achieved": flop / mean / 1e12, "peak": PEAK_F32_MFMA_TFLOPS,
                              "unit": "TFLOP/s", "frac": flop / mean / 1e12 / PEAK_F32_MFMA_TFLOPS,
                              "algorithmic_flop": flop, "hbm_frac": byts / mean / 1e9 / PEAK_HBM_GBS},
            "roofline": {"bound": "mfma", "kernel": BWD_STAGE_KERNEL.get(dom, dom), "stage": dom, "achieved": dom_tf,
                         "peak": PEAK_F32_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": dom_tf / PEAK_F32_MFMA_TFLOPS,
                         "algorithmic_flop": stage_flop[dom] * token_heads, "mean_launch_us": stage[dom] * 1e6,
                         "traffic": read_traffic("kda_chunk_backward_T4096_H16_traffic.txt",
                                                 source_digest(BWD_SOURCES), f"{dom}_hbm_bytes"),
                         "mfma_util_counter_pct": read_traffic(MFMA_PROFILE, source_digest(BWD_SOURCES),
                                                               f"{dom}_mfma_util_pct", "backward_source_digest")}}


def bench_backward_long(calls: int, T: int = 65536):
    """Backward pass at a long context (B=1, H=16, the prefill recipe at T
    tokens) with the default workspace, which processes the chunks in windows:
    mean overlapped and sequential calls, and the workspace per (chunk, head)."""
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    H, d, wid = 16, 128, 360
    log(f"backward T={T} H={H}: inputs generated on the GPU")
    inp = synth.prefill_inputs(1, T, H, d, d, "bf16", wid=wid, h0=True, device="cuda")
    inp.update(synth.grad_inputs(inp, wid, device="cuda"))
    nbytes = kda.backward_workspace_bytes(1, T, H, d, torch.bfloat16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = {}
    stream = torch.cuda.current_stream()

    def call(overlap):
        return kda.chunk_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["do"], h0=inp["h0"],
                                  dht=inp["dht"], out=out, workspace=ws, overlap=overlap)

    out.update(call(False))
    call(True)
    torch.cuda.synchronize()
    res = {}
    for overlap in (False, True):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for a, b in ev:
            a.record(stream)
            call(overlap)
            b.record(stream)
        torch.cuda.synchronize()
        res[overlap] = sum(a.elapsed_time(b) for a, b in ev) / calls * 1e-3
    chunk_heads = (T + 63) // 64 * H
    log(f"backward T={T}: {res[True] * 1e3:.2f} ms overlapped, {res[False] * 1e3:.2f} ms sequential, "
        f"workspace {nbytes / 2 ** 20:.0f} MiB")
    del inp, ws, out
    torch.cuda.empty_cache()
    return {"workload": f"kda-backward-bf16-B1-H16-T{T}-d128 (default workspace: windows of chunks)",
            "mean_call_us": res[True] * 1e6, "sequential_call_us": res[False] * 1e6,
            "value": T / res[True], "unit": "tokens/s", "workspace_bytes": nbytes,
            "workspace_mib_per_chunk_head": nbytes / 2 ** 20 / chunk_heads}


def bench_decode(steps: int, warmup: int):
    import torch
    import gated_delta_rule_105_amd as kda
    import synth

    N, H, d, wid = (DECODE[k] for k in ("N", "H", "d", "wid"))
    n_in = steps + warmup
    log(f"decode inputs N={N} H={H} d={d} bf16, {n_in} pre-staged steps (generated on the GPU)")
    inp = synth.decode_inputs(N, H, d, d, n_in, "bf16", wid=wid, device="cuda")
    state = inp["state"]
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def call(i):
        kda.decode_step(inp["q"][i], inp["k"][i], inp["v"][i], inp["g"][i], inp["beta"][i], state, o=o)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # consecutive steps, one event pair around the loop
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        call(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_step = e0.elapsed_time(e1) * 1e-3 / steps
    log(f"decode {steps} steps: wall {wall * 1e3:.3f} ms, GPU time per step {mean_step * 1e6:.2f} us")
    # the same steps captured once in a HIP graph (no launch gaps between the
    # steps), replayed; one event pair around each replay
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                call(warmup + i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    reps = 3
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in gev:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    graph_step = min(a.elapsed_time(b) for a, b in gev) * 1e-3 / steps
    log(f"decode {steps} steps as one graph: best of {reps} replays, {graph_step * 1e6:.2f} us per step")
    del graph
    state_b = N * H * d * d * 4
    bytes_step = 2 * state_b + N * H * (5 * d * 2 + 4)
    return dict(wall=wall, mean_step=mean_step, steps=steps, bytes_step=bytes_step, graph_step=graph_step)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    import oracle
    import synth

    B, T, H, d, wid = (PREFILL[k] for k in ("B", "T", "H", "d", "wid"))
    inp = synth.prefill_inputs(B, T, H, d, d, "bf16", wid=wid, h0=True)
    orc = oracle.default()
    threads = min(orc.max_threads(), B * H)
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0=inp["h0"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= CPU_SAMPLE_SECONDS:
            break
    log(f"cpu oracle: {reps} full passes in {el:.2f} s on {threads} threads")
    return {"value": reps * B * T / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{reps} full passes of the prefill workload (B=1, H=16, T=4096, d=128), fp64 "
                      f"token-by-token recurrence, OpenMP over the 16 heads, {el:.1f} s"}


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the KDA path shards by sequence and head with no communication; see the design notes)",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calib:
        copy_calib(args.copy_calib)
        return 0
    out = {"metric": "KDA prefill tokens/s/GPU + % MFMA peak; decode steps/s + % HBM peak",
           "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                                    "beta sigmoid(N(0,1)), g max(-softplus(N(0,1)), -0.125))",
           "config": {"workload": "kda-prefill-bf16-B1-H16-T4096-d128-chunk64", "B": 1, "T": 4096,
                      "H": 16, "d_k": 128, "d_v": 128, "chunk": 64, "h0": "0.02 N(0,1)"}}
    if args.only in ("prefill", "both"):
        p = bench_prefill(args.steps, args.warmup)
        out["ms_per_step"] = p["wall"] / args.steps * 1e3
        out["value"] = p["tokens"] * args.steps / p["wall"]
        # roofline of the dominant launch: its share of the algorithmic work
        # (LAUNCH_WORK x token-heads) over its mean duration from the events
        dom = max(p["launch"], key=p["launch"].get)
        t_dom = p["launch"][dom]
        work = LAUNCH_WORK[dom]
        dom_bytes = work["bytes"] * p["token_heads"] + (PREFILL["B"] * PREFILL["H"] * STATE_BYTES
                                                         if dom == "kda_chunk_sweep_out" else 0)
        dom_flop = work["flop"] * p["token_heads"]
        gbs = dom_bytes / t_dom / 1e9
        traffic = read_traffic(f"{dom}_prefill_T4096_H16_traffic.txt", source_digest(PREFILL_SOURCES))
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": gbs / PEAK_HBM_GBS, "traffic": traffic, "kernel": dom,
                           "algorithmic_bytes": dom_bytes, "algorithmic_flop": dom_flop,
                           "mfma_frac": dom_flop / t_dom / 1e12 / PEAK_BF16_TFLOPS,
                           # MFMA busy cycles per SIMD from the counters (percent), when taken on this source
                           "mfma_util_counter_pct": read_traffic(MFMA_PROFILE, source_digest(PREFILL_SOURCES),
                                                                 f"{dom}_mfma_util_pct", "prefill_source_digest"),
                           "mean_launch_us": t_dom * 1e6,
                           "launch_us": {n: t * 1e6 for n, t in p["launch"].items()}}
        call_gbs = p["bytes_call"] / p["mean_call"] / 1e9
        out["call_roofline"] = {"bound": "hbm", "achieved": call_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": call_gbs / PEAK_HBM_GBS, "algorithmic_bytes": p["bytes_call"],
                                "mean_call_us": p["mean_call"] * 1e6}
        tf = p["flop_call"] / p["mean_call"] / 1e12
        issued = p["token_heads"] * ISSUED_FLOP_PER_TOKEN_HEAD
        out["mfma"] = {"achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": tf / PEAK_BF16_TFLOPS, "algorithmic_flop": p["flop_call"],
                       "issued_flop": issued,
                       "issued_frac": issued / p["mean_call"] / 1e12 / PEAK_BF16_TFLOPS}
        # the whole call's roofline fraction: the larger of its HBM and its
        # (algorithmic) MFMA fractions
        out["roofline_fraction"] = max(out["call_roofline"]["frac"], out["mfma"]["frac"])
        out["config"]["buffer_sets"] = p["n_sets"]
    if args.only in ("prefill", "both") and not args.no_extra:
        # the packed 8-sequence batch, the million-token context and the serving batch, timed the
        # same way (secondary lines: the headline value is the workload above)
        out["other_workloads"] = [bench_workload(2, 10), bench_workload(3, 3), bench_workload(5, 20)]
        # the cold protocol: a median over calls each after a cache flush
        out["cold"] = [bench_cold(1, 20), bench_cold(2, 20), bench_cold(3, 5)]
        out["gpu_clock"] = gpu_clock()
        out["device_peaks"] = device_peaks()
        out["states_workloads"] = bench_states(50)
        out["gate_workloads"] = bench_gates(50, 100)
        out["mx_workload"] = bench_mx(100)
        out["backward_workload"] = bench_backward(20, not args.no_cpu)
        out["backward_long_workload"] = bench_backward_long(3)
    if args.only == "backward":
        out["backward_workload"] = bench_backward(args.steps, not args.no_cpu, not args.bwd_sequential)
    if args.only == "peaks":
        out["device_peaks"] = device_peaks()
    if args.only in ("decode", "both"):
        dd = bench_decode(args.decode_steps, max(1, args.warmup))
        gbs = dd["bytes_step"] / dd["mean_step"] / 1e9
        out["decode"] = {"workload": "kda-decode-bf16-N256-H32-d128-fp32-state-in-place",
                         "value": dd["steps"] / dd["wall"], "unit": "steps/s",
                         "mean_step_us": dd["mean_step"] * 1e6,
                         "graph_step_us": dd["graph_step"] * 1e6,
                         "graph_hbm_frac": dd["bytes_step"] / dd["graph_step"] / 1e9 / PEAK_HBM_GBS,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": gbs / PEAK_HBM_GBS, "kernel": "kda_decode",
                                      "algorithmic_bytes": dd["bytes_step"],
                                      "traffic": read_traffic("kda_decode_N256_H32_traffic.txt",
                                                              source_digest(("kda_decode.hip",
                                                                             "kda_device.h")))}}
        if out["value"] is None:
            out["value"] = None
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
