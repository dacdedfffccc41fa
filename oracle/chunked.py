"""Chunk-parallel (UT/WY) form of the KDA recurrence in fp64 numpy.

TEST INFRASTRUCTURE ONLY: a second, independent formulation used to pin the
token-by-token oracle (it must agree to ~1e-11).  It is also the algebra the
HIP kernels implement, so a mistake in that derivation shows up here first.

Derivation (per sequence and head; chunk rows r = 1..C', state S entering the
chunk, g already floored).  With Gamma_r = sum_{s<=r} g_s per channel:

    Kt = K * e^{Gamma}        Kh = K * e^{-Gamma}       Qt = Q * e^{Gamma}
    Kb = K * e^{Gamma_L - Gamma}   (Gamma_L = last row of Gamma)
    A  = strict_lower(diag(beta) Kt Kh^T)
    T  = (I + A)^{-1}
    Wk = T diag(beta) Kt      Wv = T diag(beta) V
    U  = Wv - Wk S                                  (the delta-rule errors)
    P  = lower_incl(Qt Kh^T)
    O  = Qt S + P U
    S  <- diag(e^{Gamma_L}) S + Kb^T U

Sources: the chunk-parallel, inter-chunk recurrence with blocked matmuls is
named in "Kimi K3 深度拆解" (chenxutan.com), 4.2 "线性注意力与 Delta Rule"
(closing paragraph); the lower bound on the log-decay that keeps e^{-Gamma}
finite so that the diagonal block is a dense product is in "3 分钟看懂 Kimi K3"
(landx.limxdynamics.com), "第一条主线", Figure 3.  The rest is derived from
the recurrence by unrolling it over one chunk.
"""
from __future__ import annotations

import numpy as np


def _chunk_pair(q, k, v, g, beta, S, chunk, g_floor):
    T = q.shape[0]
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        G = np.maximum(g[c0:c1], g_floor)
        b = beta[c0:c1]
        Gam = np.cumsum(G, axis=0)
        GL = Gam[-1]
        Kt = K * np.exp(Gam)
        Kh = K * np.exp(-Gam)
        Qt = Q * np.exp(Gam)
        Kb = K * np.exp(GL[None, :] - Gam)
        A = np.tril((b[:, None] * Kt) @ Kh.T, -1)
        Tm = np.linalg.inv(np.eye(c1 - c0) + A)
        Wk = Tm @ (b[:, None] * Kt)
        Wv = Tm @ (b[:, None] * V)
        U = Wv - Wk @ S
        P = np.tril(Qt @ Kh.T)
        o[c0:c1] = Qt @ S + P @ U
        S = np.exp(GL)[:, None] * S + Kb.T @ U
    return o, S


def chunked_forward(q, k, v, g, beta, h0=None, cu_seqlens=None,
                    g_floor=-0.125, chunk=64):
    """Same contract as :meth:`oracle.Oracle.forward` (numpy inputs)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, H, dv))
    ht = np.zeros((len(seqs), H, dk, dv))
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            if t1 > t0:
                o[b, t0:t1, h], S = _chunk_pair(
                    q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                    g[b, t0:t1, h], beta[b, t0:t1, h], S, chunk, g_floor)
            ht[n, h] = S
    return o, ht
