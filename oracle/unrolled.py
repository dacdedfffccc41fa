"""Brute-force unrolled products of the per-token transitions (tiny T only).

TEST INFRASTRUCTURE ONLY.  Each token's update is the affine map
S -> M_t S + beta_t k_t v_t^T with the explicit dk x dk matrix
M_t = (I - beta_t k_t k_t^T) diag(a_t), a_t = exp(max(g_t, floor)).
Unrolling gives

    S_t = M_t ... M_1 S_0 + sum_{s<=t} M_t ... M_{s+1} beta_s k_s v_s^T,
    o_t = S_t^T q_t,

which is evaluated here literally, forming every product of matrices
(O(T^2 dk^3) work), so that no loop structure is shared with the oracle.
Gated delta rule as in "Kimi K3 深度拆解" (chenxutan.com), 4.2, with the
channel-wise gate of "Kimi K3 技術報告" (akiraxclaw.com), "長度".
"""
from __future__ import annotations

import numpy as np


def unrolled_pair(q, k, v, g, beta, S0, g_floor=-0.125):
    """q, k, g: [T, dk]; v: [T, dv]; beta: [T]; S0: [dk, dv]. Returns o, S_T."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, dk = q.shape
    I = np.eye(dk)
    M = [(I - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(np.maximum(g[t], g_floor)))
         for t in range(T)]

    def prod(lo, hi):  # M_hi ... M_lo (inclusive, 0-based), identity if empty
        out = I.copy()
        for s in range(lo, hi + 1):
            out = M[s] @ out
        return out

    outs = []
    S_t = S0
    for t in range(T):
        S_t = prod(0, t) @ S0
        for s in range(t + 1):
            S_t = S_t + prod(s + 1, t) @ (beta[s] * np.outer(k[s], v[s]))
        outs.append(S_t.T @ q[t])
    return np.array(outs), S_t
