"""Gradient of the chunk-parallel (UT/WY) form, in fp64 numpy.

TEST INFRASTRUCTURE ONLY: a second formulation of the gradient that
``oracle.Oracle.backward`` computes token by token, used to pin one against
the other (they must agree to ~1e-12).  It is also the algebra of the
backward kernels, so a slip in that derivation shows up here first.

Forward per chunk (oracle/chunked.py; rows r of the chunk, S entering it,
Gamma = running sum of the floored log-decay, gamma = e^{Gamma_last}):

    Qt = Q e^{Gamma}, Kt = K e^{Gamma}, Kh = K e^{-Gamma}
    Abar = strict_lower(Kt Kh^T), T = (I + diag(beta) Abar)^{-1}
    Wk = T diag(beta) Kt, Wv = T diag(beta) V, P = lower_incl(Qt Kh^T)
    U = Wv - Wk S, O = Qt S + P U, S_next = diag(gamma) (S + Kh^T U)

Reverse, with dH = dL/dS_next and dO = dL/dO (the chain rule on those lines;
the pages give no gradient):

    dU = P^T dO + Kh diag(gamma) dH
    dS = Qt^T dO + diag(gamma) dH - Wk^T dU              (to the chunk before)
    dP = lower_incl(dO U^T);  dQt = dO S^T + dP Kh
    Dk = T^T (-dU S^T);  Dv = T^T dU
    dA = strict_lower(-Dk Wk^T - Dv Wv^T)
    dKt = diag(beta) (Dk + dA Kh)
    dKh = U dH^T diag(gamma) + dP^T Qt + dA^T diag(beta) Kt
    dV = diag(beta) Dv
    dbeta_r = <Dk_r, Kt_r> + <Dv_r, V_r> + sum_s dA_rs Abar_rs
    dGamma = dQt Qt + dKt Kt - dKh Kh (element-wise), and the last row also
             gets sum_j dH_cj S_next_cj (the chunk-end decay)
    dq = dQt e^{Gamma};  dk = dKt e^{Gamma} + dKh e^{-Gamma}
    dg_r = sum_{s >= r} dGamma_s where g_r >= floor, else 0

Sources for the forward lines: "Kimi K3 深度拆解" (chenxutan.com), 4.2
"线性注意力与 Delta Rule" (delta rule, chunk-parallel form); "Kimi K3 技術報告"
(akiraxclaw.com), "長度：KDA 為什麼還要搭配 Gated MLA？" (channel-wise gate);
"3 分钟看懂 Kimi K3" (landx.limxdynamics.com), "第一条主线", Figure 3 (floor).
"""
from __future__ import annotations

import numpy as np


def _pair(q, k, v, g, beta, S0, do, dST, chunk, g_floor):
    T = q.shape[0]
    starts = []
    S = S0.copy()
    bounds = [(c0, min(c0 + chunk, T)) for c0 in range(0, T, chunk)]
    for c0, c1 in bounds:  # forward: the state entering every chunk
        starts.append(S.copy())
        G = np.cumsum(np.maximum(g[c0:c1], g_floor), axis=0)
        Kt, Kh = k[c0:c1] * np.exp(G), k[c0:c1] * np.exp(-G)
        b = beta[c0:c1]
        Tm = np.linalg.inv(np.eye(c1 - c0) + np.tril(b[:, None] * Kt @ Kh.T, -1))
        U = Tm @ (b[:, None] * v[c0:c1]) - Tm @ (b[:, None] * Kt) @ S
        S = np.exp(G[-1])[:, None] * (S + Kh.T @ U)
    starts.append(S)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dg": np.zeros_like(g), "dbeta": np.zeros_like(beta)}
    dH = dST.copy()
    for j in reversed(range(len(bounds))):
        c0, c1 = bounds[j]
        S, Sn = starts[j], starts[j + 1]
        Q, K, V, dO, b = q[c0:c1], k[c0:c1], v[c0:c1], do[c0:c1], beta[c0:c1]
        graw = g[c0:c1]
        G = np.cumsum(np.maximum(graw, g_floor), axis=0)
        eG, eGi = np.exp(G), np.exp(-G)
        Qt, Kt, Kh, gam = Q * eG, K * eG, K * eGi, np.exp(G[-1])
        Abar = np.tril(Kt @ Kh.T, -1)
        Tm = np.linalg.inv(np.eye(c1 - c0) + b[:, None] * Abar)
        Wk, Wv = Tm @ (b[:, None] * Kt), Tm @ (b[:, None] * V)
        P = np.tril(Qt @ Kh.T)
        U = Wv - Wk @ S
        dU = P.T @ dO + Kh @ (gam[:, None] * dH)
        dP = np.tril(dO @ U.T)
        dQt = dO @ S.T + dP @ Kh
        Dk = Tm.T @ (-dU @ S.T)
        Dv = Tm.T @ dU
        dA = np.tril(-Dk @ Wk.T - Dv @ Wv.T, -1)
        dKt = b[:, None] * (Dk + dA @ Kh)
        dKh = (U @ dH.T) * gam[None, :] + dP.T @ Qt + dA.T @ (b[:, None] * Kt)
        dGam = dQt * Qt + dKt * Kt - dKh * Kh
        dGam[-1] += np.sum(dH * Sn, axis=1)
        acc = np.cumsum(dGam[::-1], axis=0)[::-1]
        out["dq"][c0:c1] = dQt * eG
        out["dk"][c0:c1] = dKt * eG + dKh * eGi
        out["dv"][c0:c1] = b[:, None] * Dv
        out["dbeta"][c0:c1] = np.sum(Dk * Kt, 1) + np.sum(Dv * V, 1) + np.sum(dA * Abar, 1)
        out["dg"][c0:c1] = np.where(graw >= g_floor, acc, 0.0)
        dH = gam[:, None] * dH + Qt.T @ dO - Wk.T @ dU
    out["dh0"] = dH
    return out


def chunked_backward(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None,
                     g_floor=-0.125, chunk=64):
    """Same contract as :meth:`oracle.Oracle.backward` (numpy inputs)."""
    q, k, v, g, beta, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    out = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, H, dk)), "dv": np.zeros((B, T, H, dv)),
           "dg": np.zeros((B, T, H, dk)), "dbeta": np.zeros((B, T, H)), "dh0": np.zeros((len(seqs), H, dk, dv))}
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S0 = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            dST = np.zeros((dk, dv)) if dht is None else np.array(dht[n, h], dtype=np.float64)
            if t1 == t0:
                out["dh0"][n, h] = dST
                continue
            r = _pair(q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h], g[b, t0:t1, h], beta[b, t0:t1, h],
                      S0, do[b, t0:t1, h], dST, chunk, g_floor)
            for key in ("dq", "dk", "dv", "dg"):
                out[key][b, t0:t1, h] = r[key]
            out["dbeta"][b, t0:t1, h] = r["dbeta"]
            out["dh0"][n, h] = r["dh0"]
    return out
