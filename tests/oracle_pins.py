"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function takes an oracle object (anything with the
``forward(q, k, v, g, beta, h0=None, cu_seqlens=None, g_floor=...)`` contract
of :class:`oracle.Oracle`) and raises AssertionError when the oracle is wrong.
They are run against the real oracle in ``test_oracle_pins.py`` and against
deliberately broken builds of it in ``test_oracle_mutants.py``, which must each
fail at least one pin.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

from oracle.chunked import chunked_forward
from oracle.toy_delta import delta_rule
from oracle.unrolled import unrolled_pair

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_inputs(rng, B, T, H, dk, dv, g_mode="floored", sigma_g=1.0, floor=-0.125,
                h0=True):
    """Small float32 inputs with the workloads' distributions (fp64 math after)."""
    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(rng.standard_normal((B, T, H, dk))).astype(np.float32)
    k = unit(rng.standard_normal((B, T, H, dk))).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    x = rng.standard_normal((B, T, H, dk))
    softplus = np.log1p(np.exp(sigma_g * x))
    if g_mode == "floored":
        g = np.maximum(-softplus, floor)
    elif g_mode == "raw":          # below the floor on purpose
        g = -softplus
    elif g_mode == "weak":
        g = np.full_like(x, -1e-3)
    elif g_mode == "zero":
        g = np.zeros_like(x)
    else:
        raise ValueError(g_mode)
    g = g.astype(np.float32)
    S0 = (0.02 * rng.standard_normal((B, H, dk, dv))) if h0 else None
    return q, k, v, g, beta, S0


def rel_err(x, ref):
    return float(np.max(np.abs(np.asarray(x) - np.asarray(ref))) / max(np.max(np.abs(ref)), 1e-300))


# --------------------------------------------------------------------------
# I1: beta = 0 leaves only the gate: S_t = diag(exp(sum_{s<=t} max(g_s, f))) S_0.
def pin_beta_zero_closed_form(orc):
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 37, 2, 8, 6, g_mode="raw")
    beta[:] = 0
    o, ht = orc.forward(q, k, v, g, beta, h0=S0, g_floor=-0.125)
    G = np.cumsum(np.maximum(g.astype(np.float64), -0.125), axis=1)  # [1,T,H,dk]
    for h in range(2):
        for t in range(37):
            St = np.exp(G[0, t, h])[:, None] * S0[0, h]
            assert rel_err(o[0, t, h], St.T @ q[0, t, h]) < 1e-13
        assert rel_err(ht[0, h], np.exp(G[0, -1, h])[:, None] * S0[0, h]) < 1e-13
    # zero state and beta = 0: everything vanishes
    o0, h00 = orc.forward(q, k, v, g, beta, h0=None)
    assert np.all(o0 == 0) and np.all(h00 == 0)


# I2: g = 0 (no forgetting) is the ungated delta rule of the toy loop.
def pin_gate_one_is_delta_rule(orc):
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 50, 3, 8, 5, g_mode="zero")
    o, ht = orc.forward(q, k, v, g, beta, h0=S0, g_floor=-0.125)
    for h in range(3):
        ot, St = delta_rule(q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], S0[0, h])
        assert rel_err(o[0, :, h], ot) < 1e-12
        assert rel_err(ht[0, h], St) < 1e-12
    # and from a zero state, the toy loop's own starting point
    o, ht = orc.forward(q, k, v, g, beta, h0=None)
    ot, St = delta_rule(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0])
    assert rel_err(o[0, :, 0], ot) < 1e-12


# I3: with beta_t = 1 and |k_t| = 1 the write is exact: S_t^T k_t = v_t.
def pin_full_write_then_read(orc):
    rng = np.random.default_rng(13)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 40, 2, 16, 7)
    beta[:] = 1.0
    k = (k / np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
    kk = np.sum(k.astype(np.float64) ** 2, axis=-1)
    o, _ = orc.forward(q, k, v, g, beta, h0=S0)
    ok, _ = orc.forward(k, k, v, g, beta, h0=S0)   # read with q = k
    # S_t^T k_t = (1 - |k|^2) S'^T k + |k|^2 v ; |k|^2 = 1 up to float32 rounding
    dev = np.max(np.abs(kk - 1.0))
    assert rel_err(ok, v) < 1e-5 + 10 * dev
    assert not np.allclose(o, v, atol=1e-3)


# I4: brute-force unrolled products on T <= 8.
def pin_unrolled_products(orc):
    rng = np.random.default_rng(14)
    for T, dk, dv in ((1, 4, 3), (5, 6, 4), (8, 5, 7)):
        q, k, v, g, beta, S0 = rand_inputs(rng, 1, T, 2, dk, dv, g_mode="raw")
        o, ht = orc.forward(q, k, v, g, beta, h0=S0, g_floor=-0.125)
        for h in range(2):
            ot, St = unrolled_pair(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h],
                                   beta[0, :, h], S0[0, h], g_floor=-0.125)
            assert rel_err(o[0, :, h], ot) < 1e-12
            assert rel_err(ht[0, h], St) < 1e-12


# I5: the chunked (UT/WY) form equals the recurrence, for several chunk sizes,
# ragged tails, a nonzero initial state and packed sequences.
def pin_chunked_form(orc):
    rng = np.random.default_rng(15)
    for g_mode in ("floored", "weak", "zero"):
        q, k, v, g, beta, S0 = rand_inputs(rng, 2, 70, 2, 12, 9, g_mode=g_mode)
        o, ht = orc.forward(q, k, v, g, beta, h0=S0)
        for C in (1, 2, 4, 16, 64):
            oc, hc = chunked_forward(q, k, v, g, beta, h0=S0, chunk=C)
            assert rel_err(oc, o) < 1e-10, (g_mode, C)
            assert rel_err(hc, ht) < 1e-10, (g_mode, C)
    lengths = [3, 64, 65, 1, 130]
    cu = np.cumsum([0] + lengths)
    q, k, v, g, beta, _ = rand_inputs(rng, 1, int(cu[-1]), 2, 8, 8)
    S0 = 0.02 * rng.standard_normal((len(lengths), 2, 8, 8))
    o, ht = orc.forward(q, k, v, g, beta, h0=S0, cu_seqlens=cu)
    oc, hc = chunked_forward(q, k, v, g, beta, h0=S0, cu_seqlens=cu, chunk=64)
    assert rel_err(oc, o) < 1e-10 and rel_err(hc, ht) < 1e-10


# I6: for fixed q, k, g, beta the map (V, S_0) -> (O, S_T) is linear.
def pin_linearity(orc):
    rng = np.random.default_rng(16)
    q, k, v1, g, beta, S1 = rand_inputs(rng, 1, 30, 2, 8, 8)
    v2 = rng.standard_normal(v1.shape).astype(np.float32)
    S2 = 0.02 * rng.standard_normal(S1.shape)
    a, b = 0.75, -1.5   # exact in float32, so a*v1 + b*v2 rounds once
    v3 = (a * v1.astype(np.float64) + b * v2).astype(np.float32)
    o1, h1 = orc.forward(q, k, v1, g, beta, h0=S1)
    o2, h2 = orc.forward(q, k, v2, g, beta, h0=S2)
    o3, h3 = orc.forward(q, k, v3, g, beta, h0=a * S1 + b * S2)
    v3err = v3.astype(np.float64) - (a * v1.astype(np.float64) + b * v2)
    # the rounding of v3 enters linearly; with 1e-6 relative rounding the
    # combination still matches to ~1e-6
    assert rel_err(o3, a * o1 + b * o2) < 1e-5
    assert rel_err(h3, a * h1 + b * h2) < 1e-5
    assert np.max(np.abs(v3err)) < 1e-6


# I7: splitting a sequence and resuming from the carried state changes nothing.
def pin_split_resume(orc):
    rng = np.random.default_rng(17)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 150, 2, 8, 8)
    o, ht = orc.forward(q, k, v, g, beta, h0=S0)
    for cut in (1, 64, 77, 149):
        oa, ha = orc.forward(q[:, :cut], k[:, :cut], v[:, :cut], g[:, :cut], beta[:, :cut], h0=S0)
        ob, hb = orc.forward(q[:, cut:], k[:, cut:], v[:, cut:], g[:, cut:], beta[:, cut:], h0=ha)
        assert rel_err(np.concatenate([oa, ob], axis=1), o) < 1e-13
        assert rel_err(hb, ht) < 1e-13


# I9: with v = 0 the state norm never grows (|(I - b k k^T) diag(a)|_2 <= 1).
def pin_contraction(orc):
    rng = np.random.default_rng(18)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 60, 2, 8, 8, g_mode="weak")
    v[:] = 0
    S0 = rng.standard_normal(S0.shape)
    prev = np.linalg.norm(S0, axis=(-2, -1))
    for t in range(1, 61, 7):
        _, ht = orc.forward(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], h0=S0)
        cur = np.linalg.norm(ht, axis=(-2, -1))
        assert np.all(cur <= prev * (1 + 1e-12))
        prev = cur
    assert np.all(cur < np.linalg.norm(S0, axis=(-2, -1)))


# I10: value columns are independent; permuting them permutes o and S.
def pin_value_columns(orc):
    rng = np.random.default_rng(19)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 45, 2, 8, 10)
    perm = rng.permutation(10)
    o, ht = orc.forward(q, k, v, g, beta, h0=S0)
    op, hp = orc.forward(q, k, v[..., perm], g, beta, h0=S0[..., perm])
    assert rel_err(op, o[..., perm]) < 1e-14 and rel_err(hp, ht[..., perm]) < 1e-14
    oh, hh = orc.forward(q, k, v[..., :4], g, beta, h0=S0[..., :4])
    assert rel_err(oh, o[..., :4]) < 1e-14 and rel_err(hh, ht[..., :4]) < 1e-14


# Scalar case: dk = dv = 1, k = q = 1 makes the recurrence a first-order
# linear filter S_t = a (1 - b) S_{t-1} + b v_t (an exponential moving average),
# which scipy's lfilter evaluates independently.
def pin_scalar_ema_lfilter(orc):
    from scipy.signal import lfilter
    rng = np.random.default_rng(20)
    T = 200
    a_log, b = -0.0625, 0.375          # exact binary fractions
    q = np.ones((1, T, 1, 1), np.float32)
    k = np.ones((1, T, 1, 1), np.float32)
    g = np.full((1, T, 1, 1), a_log, np.float32)
    beta = np.full((1, T, 1), b, np.float32)
    v = rng.standard_normal((1, T, 1, 1)).astype(np.float32)
    o, ht = orc.forward(q, k, v, g, beta, h0=None, g_floor=-0.125)
    a = math.exp(a_log)
    ref = lfilter([b], [1.0, -a * (1.0 - b)], v[0, :, 0, 0].astype(np.float64))
    assert rel_err(o[0, :, 0, 0], ref) < 1e-13
    assert abs(ht[0, 0, 0, 0] - ref[-1]) < 1e-13 * max(1, abs(ref[-1]))
    # the floor binds: a log-decay of -1 behaves as -0.125
    g2 = np.full_like(g, -1.0)
    o2, _ = orc.forward(q, k, v, g2, beta, h0=None, g_floor=-0.125)
    ref2 = lfilter([b], [1.0, -math.exp(-0.125) * (1.0 - b)], v[0, :, 0, 0].astype(np.float64))
    assert rel_err(o2[0, :, 0, 0], ref2) < 1e-13


# Exact rational arithmetic on a small example whose inputs are all exact
# binary fractions; the only rounding left on the reference side is the gate
# a = exp(g), taken as the exact rational value of the double the C library
# returns for the same float32 g.
def pin_exact_rational(orc):
    rng = np.random.default_rng(21)
    T, dk, dv = 6, 3, 2
    dy = lambda shape, den: rng.integers(-den, den + 1, size=shape) / den  # noqa: E731
    q, k, v = dy((T, dk), 8), dy((T, dk), 8), dy((T, dv), 4)
    beta = rng.integers(1, 8, size=T) / 8.0
    g = -rng.integers(0, 4, size=(T, dk)) / 32.0      # -0.09375 .. 0, above the floor
    S0 = dy((dk, dv), 16)
    F = Fraction
    S = [[F(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        a = [F(math.exp(float(np.float32(x)))) for x in g[t]]
        kt, qt, vt, bt = [F(x) for x in k[t]], [F(x) for x in q[t]], [F(x) for x in v[t]], F(beta[t])
        Sd = [[a[c] * S[c][j] for j in range(dv)] for c in range(dk)]
        u = [bt * (vt[j] - sum(Sd[c][j] * kt[c] for c in range(dk))) for j in range(dv)]
        S = [[Sd[c][j] + kt[c] * u[j] for j in range(dv)] for c in range(dk)]
        outs.append([sum(S[c][j] * qt[c] for c in range(dk)) for j in range(dv)])
    ref_o = np.array([[float(x) for x in r] for r in outs])
    ref_S = np.array([[float(x) for x in r] for r in S])
    f32 = lambda x: np.asarray(x, np.float32)[None, :, None]  # noqa: E731
    o, ht = orc.forward(f32(q), f32(k), f32(v), f32(g), f32(beta), h0=S0[None, None],
                        g_floor=-0.125)
    assert rel_err(o[0, :, 0], ref_o) < 1e-14
    assert rel_err(ht[0, 0], ref_S) < 1e-14


def load_golden(name):
    """Parse a golden text fixture: '# ...' comments and 'key: v v v' lines."""
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = np.array([float(x) for x in rest.split()], dtype=np.float64)
    return vals


# Hand-worked example, one channel (see the fixture's own derivation).
def pin_golden_scalar(orc):
    gd = load_golden("scalar_ema_hand.txt")
    T = len(gd["v"])
    shp = (1, T, 1, 1)
    o, ht = orc.forward(np.full(shp, gd["q"][0], np.float32),
                        np.full(shp, gd["k"][0], np.float32),
                        gd["v"].reshape(shp).astype(np.float32),
                        np.full(shp, gd["g"][0], np.float32),
                        np.full((1, T, 1), gd["beta"][0], np.float32),
                        h0=gd["S0"].reshape(1, 1, 1, 1), g_floor=float(gd["floor"][0]))
    # exp(-ln 2) is 0.5 to within one ulp
    assert rel_err(o[0, :, 0, 0], gd["o"]) < 1e-15 * 8
    assert abs(ht[0, 0, 0, 0] - gd["S_T"][0]) < 1e-14


# Hand-worked example, two orthogonal keys (see the fixture's derivation).
def pin_golden_orthogonal(orc):
    gd = load_golden("orthogonal_keys_hand.txt")
    T = 3
    q = gd["q"].reshape(1, T, 1, 2).astype(np.float32)
    k = gd["k"].reshape(1, T, 1, 2).astype(np.float32)
    v = gd["v"].reshape(1, T, 1, 2).astype(np.float32)
    g = gd["g"].reshape(1, T, 1, 2).astype(np.float32)
    beta = gd["beta"].reshape(1, T, 1).astype(np.float32)
    o, ht = orc.forward(q, k, v, g, beta, h0=gd["S0"].reshape(1, 1, 2, 2),
                        g_floor=float(gd["floor"][0]))
    assert rel_err(o[0, :, 0].reshape(-1), gd["o"]) < 1e-14
    assert rel_err(ht[0, 0].reshape(-1), gd["S_T"]) < 1e-14


ALL_PINS = [
    pin_beta_zero_closed_form, pin_gate_one_is_delta_rule, pin_full_write_then_read,
    pin_unrolled_products, pin_chunked_form, pin_linearity, pin_split_resume,
    pin_contraction, pin_value_columns, pin_scalar_ema_lfilter, pin_exact_rational,
    pin_golden_scalar, pin_golden_orthogonal,
]
