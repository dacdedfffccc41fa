"""Pins of the oracle's gradient (``oracle.Oracle.backward``).

Each ``pin_*`` takes an oracle object and raises AssertionError when its
gradient is wrong.  The pins rest on what mathematics fixes, not on a second
copy of the reverse pass:
  * central finite differences of the forward, evaluated in fp64 by the
    chunked form (``oracle.chunked``, itself pinned to the recurrence), for
    every element of every input, with log-decays both above and strictly
    below the floor;
  * the floor's one-sided derivative from above where g equals the floor;
  * homogeneity: (v, h0) -> (o, ht) is linear and o is linear in q, so by
    Euler's identity <dv, v> + <dh0, h0> = <do, o> + <dht, ht> and
    <dq, q> = <do, o>, at any size;
  * the chunk-parallel gradient (``oracle.chunked_bwd``, the algebra of the
    backward kernels), a second formulation that must agree to ~1e-12.
They run against the real oracle in ``test_oracle_bwd_pins.py`` and against
builds with planted mistakes, which must each fail at least one pin.
"""
from __future__ import annotations

import numpy as np

from oracle.chunked import chunked_forward

FLOOR = -0.125


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def tiny_case(seed=3, below_floor=True, ties=False):
    """Two packed sequences (5 and 4 tokens), H=2, dk=3, dv=2, all inputs
    exactly representable in fp32 (the oracle reads fp32)."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 9, 2, 3, 2
    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = _f32(unit(rng.standard_normal((1, T, H, dk))))
    k = _f32(unit(rng.standard_normal((1, T, H, dk))))
    v = _f32(rng.standard_normal((1, T, H, dv)))
    beta = _f32(1 / (1 + np.exp(-rng.standard_normal((1, T, H)))))
    g = _f32(rng.uniform(-0.11, -0.01, (1, T, H, dk)))
    if below_floor:  # strictly below the floor: flat there, gradient 0
        g[0, 1, 0, 2] = -0.3
        g[0, 6, 1, 0] = -0.5
    if ties:
        g[0, 2, 0, 1] = FLOOR
        g[0, 7, 1, 2] = FLOOR
    cu = np.array([0, 5, 9])
    h0 = _f32(0.3 * rng.standard_normal((2, H, dk, dv)))
    do = rng.standard_normal((1, T, H, dv))
    dht = rng.standard_normal((2, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, cu=cu, do=do, dht=dht)


def _loss(c, **over):
    x = dict(c, **over)
    o, ht = chunked_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"],
                            cu_seqlens=x["cu"], g_floor=FLOOR, chunk=4)
    return float(np.sum(o * c["do"]) + np.sum(ht * c["dht"]))


def _grads(orc, c):
    return orc.backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], h0=c["h0"],
                        dht=c["dht"], cu_seqlens=c["cu"], g_floor=FLOOR)


# every element of every input against central differences
def pin_bwd_finite_differences(orc):
    c = tiny_case()
    grads = _grads(orc, c)
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"),
                        ("beta", "dbeta"), ("h0", "dh0")):
        x = c[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd[idx] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * eps)
        err = np.max(np.abs(grads[gname] - fd)) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-7, f"d{name}: finite-difference error {err:.2e}"
    # the entries below the floor are flat
    assert grads["dg"][0, 1, 0, 2] == 0 and grads["dg"][0, 6, 1, 0] == 0


# where g sits on the floor the gradient is the derivative from above
def pin_bwd_floor_tie(orc):
    c = tiny_case(seed=5, below_floor=False, ties=True)
    grads = _grads(orc, c)
    h = 1e-7
    for idx in ((0, 2, 0, 1), (0, 7, 1, 2)):
        gp = c["g"].copy()
        gp[idx] += h
        right = (_loss(c, g=gp) - _loss(c)) / h
        gm = c["g"].copy()
        gm[idx] -= h
        left = (_loss(c) - _loss(c, g=gm)) / h
        assert abs(left) < 1e-12, "below the floor the forward must be flat"
        assert abs(grads["dg"][idx] - right) <= 1e-5 * max(1.0, abs(right)), (grads["dg"][idx], right)


# Euler's identity for the parts of the map that are linear
def pin_bwd_homogeneity(orc):
    rng = np.random.default_rng(7)
    T, H, dk, dv = 150, 3, 16, 12
    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = _f32(unit(rng.standard_normal((1, T, H, dk))))
    k = _f32(unit(rng.standard_normal((1, T, H, dk))))
    v = _f32(rng.standard_normal((1, T, H, dv)))
    beta = _f32(1 / (1 + np.exp(-rng.standard_normal((1, T, H)))))
    g = _f32(np.maximum(-np.log1p(np.exp(rng.standard_normal((1, T, H, dk)))), FLOOR) * 0.05)
    cu = np.array([0, 61, 150])
    h0 = _f32(0.5 * rng.standard_normal((2, H, dk, dv)))
    do = rng.standard_normal((1, T, H, dv))
    dht = rng.standard_normal((2, H, dk, dv))
    o, ht = orc.forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu, g_floor=FLOOR)
    gr = orc.backward(q, k, v, g, beta, do, h0=h0, dht=dht, cu_seqlens=cu, g_floor=FLOOR)
    lhs = np.sum(gr["dv"] * v) + np.sum(gr["dh0"] * h0)
    rhs = np.sum(do * o) + np.sum(dht * ht)
    assert abs(lhs - rhs) <= 1e-10 * (abs(rhs) + np.sum(np.abs(do * o))), (lhs, rhs)
    lq, rq = np.sum(gr["dq"] * q), np.sum(do * o)
    assert abs(lq - rq) <= 1e-10 * np.sum(np.abs(do * o)), (lq, rq)


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_floor_tie, pin_bwd_homogeneity]


# the chunk-parallel gradient (the algebra of the backward kernels) against
# the token-by-token one, for several chunk sizes, ragged and packed lengths,
# decays above, on and below the floor
def pin_bwd_chunked_form(orc):
    from oracle.chunked_bwd import chunked_backward
    from oracle_pins import rand_inputs
    rng = np.random.default_rng(21)
    for mode, chunk in (("floored", 64), ("raw", 16), ("weak", 4), ("zero", 1)):
        q, k, v, g, beta, S0 = rand_inputs(rng, 1, 150, 2, 8, 6, g_mode=mode)
        cu = np.array([0, 37, 37, 150])
        h0 = 0.3 * rng.standard_normal((3, 2, 8, 6))
        do = rng.standard_normal(v.shape)
        dht = rng.standard_normal((3, 2, 8, 6))
        ref = orc.backward(q, k, v, g, beta, do, h0=h0, dht=dht, cu_seqlens=cu, g_floor=FLOOR)
        got = chunked_backward(q, k, v, g, beta, do, h0=h0, dht=dht, cu_seqlens=cu, g_floor=FLOOR, chunk=chunk)
        for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
            err = np.max(np.abs(got[key] - ref[key])) / max(np.max(np.abs(ref[key])), 1e-300)
            assert err < 1e-10, f"{mode} chunk={chunk} {key}: {err:.2e}"


ALL_BWD_PINS.append(pin_bwd_chunked_form)
