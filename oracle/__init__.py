"""KDA oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct CPU implementations of what the HIP library
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import anything from this package; the product path
(``gated_delta_rule_105_amd``) never does, and shares no code with it.

Contents
--------
``kda_oracle.c`` / :func:`forward`
    The token-by-token fp64 recurrence (the oracle proper).  Pinned by the
    invariant, closed-form, brute-force and library checks in
    ``tests/test_oracle_pins.py``.
``kda_oracle_bwd.c`` / :func:`backward`
    Its reverse-mode derivative, token by token in fp64 (the chain rule on
    the forward's lines, last line first).  Pinned by central finite
    differences of the forward, by the homogeneity identities of the
    recurrence and by the floor's one-sided derivative in
    ``tests/test_oracle_bwd_pins.py``.
:mod:`oracle.chunked`
    The chunk-parallel (UT/WY) rewriting of the same recurrence, in fp64
    numpy.  Used only as a cross-formulation pin of :func:`forward`.
:mod:`oracle.chunked_bwd`
    The gradient of that chunk-parallel form, in fp64 numpy: a
    cross-formulation pin of :func:`backward`.
:mod:`oracle.unrolled`
    Explicit products of the per-token transition matrices, for tiny T.
:mod:`oracle.toy_delta`
    The ungated delta-rule loop exactly as the pages describe it.

Passages followed (page title, section):
  * "Kimi K3 深度拆解" (chenxutan.com), 4.2 "线性注意力与 Delta Rule":
    delta-rule update, erase before write, read after write, state [d, d_v].
  * "Kimi K3 技術報告：三個架構改動一次看懂" (akiraxclaw.com),
    "長度：KDA 為什麼還要搭配 Gated MLA？": channel-wise forget gate.
  * "3 分钟看懂 Kimi K3" (landx.limxdynamics.com), "第一条主线", Figure 3:
    lower bound on the per-step log-decay.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
SOURCE_BWD = os.path.join(_HERE, "kda_oracle_bwd.c")
# KDA_ORACLE_LIBRARY selects another build of the oracle (a sanitizer build);
# default: the in-tree build, compiled on first use.
LIBRARY = os.environ.get("KDA_ORACLE_LIBRARY") or os.path.join(_HERE, "libkda_oracle.so")

# No -ffast-math and no -march: IEEE semantics, no contraction into FMA.  -O3
# vectorises only the loops over the value index, whose sums are independent,
# so every sum over the key index keeps its written order.
CFLAGS = ["-O3", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall"]


def build(source: str = SOURCE, out: str = LIBRARY, extra=(SOURCE_BWD,)) -> str:
    """Compile the C oracle (forward and gradient) with gcc; returns the path
    of the shared object."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source, *extra, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _as_f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (any dtype, any device)
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


class Oracle:
    """ctypes binding of one build of ``kda_oracle.c``."""

    def __init__(self, lib_path: str = LIBRARY):
        if not os.path.exists(lib_path):
            if lib_path != LIBRARY:
                raise FileNotFoundError(lib_path)
            build()
        self._lib = ctypes.CDLL(lib_path)
        f = self._lib.kda_oracle_forward
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        f.argtypes = [i64, p, i64, i64, i64, ctypes.c_double, p, p, p, p, p, p,
                      p, p, ctypes.c_int]
        f.restype = ctypes.c_int
        self._lib.kda_oracle_max_threads.restype = ctypes.c_int

    def _bwd(self):
        # looked up on first use: a build of the forward source alone (the
        # mutant tests make such builds) has no gradient symbol
        f = self._lib.kda_oracle_backward
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        f.argtypes = [i64, p, i64, i64, i64, ctypes.c_double, p, p, p, p, p, p,
                      p, p, p, p, p, p, p, p, ctypes.c_int]
        f.restype = ctypes.c_int
        return f

    def max_threads(self) -> int:
        return int(self._lib.kda_oracle_max_threads())

    def forward(self, q, k, v, g, beta, h0=None, cu_seqlens=None,
                g_floor: float = -0.125,
                n_threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Run the recurrence.

        q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H].
        With ``cu_seqlens`` (int, [n+1]) the batch must be B == 1 and holds n
        packed sequences.  h0: [S, H, dk, dv] or None (zeros), where S is the
        number of sequences.  Returns (o [B, T, H, dv], ht [S, H, dk, dv]),
        both float64.
        """
        q, k, v, g, beta = (_as_f32(x) for x in (q, k, v, g, beta))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and g.shape == q.shape
        assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
        if cu_seqlens is None:
            cu = np.arange(B + 1, dtype=np.int64) * T
        else:
            assert B == 1, "packed sequences need B == 1"
            cu = np.ascontiguousarray(np.asarray(
                cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                dtype=np.int64))
            assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
        n_seqs = len(cu) - 1
        h0a = None if h0 is None else _as_f64(h0)
        if h0a is not None:
            assert h0a.shape == (n_seqs, H, dk, dv)
        o = np.empty((B, T, H, dv), dtype=np.float64)
        ht = np.empty((n_seqs, H, dk, dv), dtype=np.float64)
        ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
        rc = self._lib.kda_oracle_forward(
            n_seqs, ptr(cu), H, dk, dv, float(g_floor), ptr(q), ptr(k), ptr(v),
            ptr(g), ptr(beta), ptr(h0a), ptr(o), ptr(ht), int(n_threads))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_forward failed with status {rc}")
        return o, ht

    def decode_step(self, q, k, v, g, beta, state, g_floor: float = -0.125,
                    n_threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """One token for each of N sequences.

        q, k, g: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; state [N, H, dk, dv].
        Returns (o [N, H, dv], new state [N, H, dk, dv]) in float64.  This is
        the recurrence run over N sequences of length one, packed.
        """
        q, k, v, g, beta = (_as_f32(x) for x in (q, k, v, g, beta))
        N = q.shape[0]
        cu = np.arange(N + 1, dtype=np.int64)
        o, ht = self.forward(q[None], k[None], v[None], g[None], beta[None],
                             h0=state, cu_seqlens=cu, g_floor=g_floor,
                             n_threads=n_threads)
        return o[0], ht

    def backward(self, q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None,
                 g_floor: float = -0.125, n_threads: int = 0):
        """Gradients of L = <do, o> + <dht, ht> for the forward above.

        q, k, g: [B, T, H, dk]; v, do: [B, T, H, dv]; beta: [B, T, H];
        h0, dht: [S, H, dk, dv] or None (zeros).  Returns a dict of float64
        arrays dq, dk, dv, dg, dbeta (shapes of their inputs) and dh0
        [S, H, dk, dv].  Where g is below g_floor, dg is 0; at g == g_floor
        the gradient passes.
        """
        q, k, v, g, beta = (_as_f32(x) for x in (q, k, v, g, beta))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and g.shape == q.shape
        assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
        if cu_seqlens is None:
            cu = np.arange(B + 1, dtype=np.int64) * T
        else:
            assert B == 1, "packed sequences need B == 1"
            cu = np.ascontiguousarray(np.asarray(
                cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                dtype=np.int64))
            assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
        n_seqs = len(cu) - 1
        doa = _as_f64(do)
        assert doa.shape == (B, T, H, dv)
        h0a = None if h0 is None else _as_f64(h0)
        dhta = None if dht is None else _as_f64(dht)
        for a in (h0a, dhta):
            if a is not None:
                assert a.shape == (n_seqs, H, dk, dv)
        out = dict(dq=np.zeros((B, T, H, dk)), dk=np.zeros((B, T, H, dk)),
                   dv=np.zeros((B, T, H, dv)), dg=np.zeros((B, T, H, dk)),
                   dbeta=np.zeros((B, T, H)), dh0=np.zeros((n_seqs, H, dk, dv)))
        ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
        rc = self._bwd()(
            n_seqs, ptr(cu), H, dk, dv, float(g_floor), ptr(q), ptr(k), ptr(v),
            ptr(g), ptr(beta), ptr(h0a), ptr(doa), ptr(dhta), ptr(out["dq"]),
            ptr(out["dk"]), ptr(out["dv"]), ptr(out["dg"]), ptr(out["dbeta"]),
            ptr(out["dh0"]), int(n_threads))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_backward failed with status {rc}")
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def forward(*args, **kwargs):
    """Module-level shortcut for :meth:`Oracle.forward` on the default build."""
    return default().forward(*args, **kwargs)


def decode_step(*args, **kwargs):
    """Module-level shortcut for :meth:`Oracle.decode_step`."""
    return default().decode_step(*args, **kwargs)


def backward(*args, **kwargs):
    """Module-level shortcut for :meth:`Oracle.backward`."""
    return default().backward(*args, **kwargs)
