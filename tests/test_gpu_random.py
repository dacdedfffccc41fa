"""Seeded random configurations: forward, backward and decode against the
oracle, element by element.

Each case draws its configuration from its own fixed seed: the path (bf16 at
d = 128 or 64, fp32 at d = 64), a batch of equal lengths or a packed batch
(lengths mixing empty sequences, exact chunk multiples and ragged tails), the
number of heads, the gate (per channel, per head, none), h0 and dht present
or not, the spread of the log-decays and whether they reach below the floor.
So the sweep covers combinations the hand-picked cases of the other files do
not, and every run covers the same ones (the test id names the configuration).

Tolerances as elsewhere: max|x - x_ref| / max|x_ref| <= 1e-4 (fp32 path),
<= 1e-2 (bf16 path), on o and the final state, on every gradient and on the
decode outputs and state.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_105_amd as kda
import oracle
import synth
from gpu_util import TOL, f64, note, rel_err, to_dev

pytestmark = pytest.mark.gpu

N_PREFILL, N_DECODE = 48, 12


def _lengths(rs, n):
    out = []
    for _ in range(n):
        u = rs.rand()
        if u < 0.15:
            out.append(0)
        elif u < 0.35:
            out.append(64 * int(rs.randint(1, 5)))
        else:
            out.append(int(rs.randint(1, 901)))
    return out


def draw_prefill(c):
    rs = np.random.RandomState(7000 + c)
    dtype, d = [("bf16", 128), ("bf16", 64), ("f32", 64)][rs.choice(3, p=[0.5, 0.25, 0.25])]
    cfg = dict(dtype=dtype, d=d, H=int(rs.randint(1, 5)), h0=bool(rs.rand() < 0.6), dht=bool(rs.rand() < 0.7),
               gate=str(rs.choice(["channel", "head", "none"], p=[0.6, 0.2, 0.2])),
               sigma=float(rs.choice([0.5, 1.0, 2.0])), raw=bool(rs.rand() < 0.25))
    if rs.rand() < 0.5:
        cfg.update(B=int(rs.randint(1, 4)), T=int(rs.randint(1, 3001)), lengths=None)
    else:
        cfg.update(B=1, T=0, lengths=_lengths(rs, int(rs.randint(1, 17))))
    return cfg


def _pid(c):
    x = draw_prefill(c)
    shape = f"B{x['B']}T{x['T']}" if x["lengths"] is None else f"packed{len(x['lengths'])}"
    return (f"{c}-{x['dtype']}-d{x['d']}-{shape}-H{x['H']}-{x['gate']}" + ("-h0" if x["h0"] else "")
            + ("-raw" if x["raw"] else "") + f"-s{x['sigma']:g}")


def make_prefill(c):
    x = draw_prefill(c)
    wid = 700 + c
    inp = synth.prefill_inputs(x["B"], x["T"], x["H"], x["d"], x["d"], x["dtype"], wid=wid, sigma_g=x["sigma"],
                               h0=x["h0"], lengths=x["lengths"])
    if x["raw"]:  # log-decays below the floor in places: the kernels floor them
        z = synth.normal(tuple(inp["g"].shape), wid, "g")
        inp["g"] = (-torch.nn.functional.softplus(x["sigma"] * z)).to(inp["g"].dtype)
    inp.update(synth.grad_inputs(inp, wid, dht=x["dht"]))
    # (g for the GPU, g for the oracle): the per-head gate is channel 0 of the
    # per-channel one, broadcast over the channels for the oracle
    if x["gate"] == "head":
        gh = inp["g"][..., 0].contiguous()
        gates = (gh, gh[..., None].expand(inp["g"].shape).contiguous())
    elif x["gate"] == "none":
        gates = (None, torch.zeros_like(inp["g"]))
    else:
        gates = (inp["g"], inp["g"])
    return x, inp, gates


@pytest.mark.parametrize("c", range(N_PREFILL), ids=_pid)
def test_random_forward_backward(c):
    x, inp, (g_gpu, g_ref) = make_prefill(c)
    tol = TOL[x["dtype"]]
    cu = inp["cu_seqlens"]
    note(f"random prefill case {_pid(c)} q{tuple(inp['q'].shape)}")
    d = to_dev(inp)
    gd = None if g_gpu is None else g_gpu.cuda()
    o, ht = kda.chunk_forward(d["q"], d["k"], d["v"], gd, d["beta"], h0=d["h0"], cu_seqlens=d["cu_seqlens"])
    out = kda.chunk_backward(d["q"], d["k"], d["v"], gd, d["beta"], d["do"], h0=d["h0"], dht=d["dht"],
                             cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    cu_np = None if cu is None else cu.numpy()
    ro, rht = oracle.forward(inp["q"], inp["k"], inp["v"], g_ref, inp["beta"], h0=inp["h0"], cu_seqlens=cu_np)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], g_ref, inp["beta"], inp["do"], h0=inp["h0"],
                          dht=inp["dht"], cu_seqlens=cu_np)
    errs = {"o": rel_err(f64(o), ro), "ht": rel_err(f64(ht), rht)}
    if x["gate"] == "head":
        ref["dg"] = ref["dg"].sum(axis=-1)
    if x["gate"] == "none":
        assert out["dg"] is None
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        if out.get(key) is not None:
            errs[key] = rel_err(f64(out[key]), ref[key])
    print(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


def draw_decode(c):
    rs = np.random.RandomState(8000 + c)
    dtype, d = [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)][rs.randint(4)]
    return dict(dtype=dtype, d=d, N=int(rs.randint(1, 40)), H=int(rs.randint(1, 5)), steps=int(rs.randint(1, 9)),
                gate=str(rs.choice(["channel", "head", "none"], p=[0.6, 0.2, 0.2])),
                sigma=float(rs.choice([0.5, 1.0, 2.0])))


def _did(c):
    x = draw_decode(c)
    return f"{c}-{x['dtype']}-d{x['d']}-N{x['N']}-H{x['H']}-x{x['steps']}-{x['gate']}-s{x['sigma']:g}"


@pytest.mark.parametrize("c", range(N_DECODE), ids=_did)
def test_random_decode(c):
    x = draw_decode(c)
    inp = synth.decode_inputs(x["N"], x["H"], x["d"], x["d"], x["steps"], x["dtype"], wid=800 + c,
                              sigma_g=x["sigma"])
    tol = TOL[x["dtype"]]
    note(f"random decode case {_did(c)}")
    state = inp["state"].cuda()
    ref_state = inp["state"].double().numpy()
    eo = 0.0
    for s in range(x["steps"]):
        g = inp["g"][s]
        if x["gate"] == "head":
            g_gpu = g[..., 0].contiguous()
            g_ref = g_gpu[..., None].expand(g.shape).contiguous()
        elif x["gate"] == "none":
            g_gpu, g_ref = None, torch.zeros_like(g)
        else:
            g_gpu, g_ref = g, g
        o = kda.decode_step(inp["q"][s].cuda(), inp["k"][s].cuda(), inp["v"][s].cuda(),
                            None if g_gpu is None else g_gpu.cuda(), inp["beta"][s].cuda(), state)
        torch.cuda.synchronize()
        ro, ref_state = oracle.decode_step(inp["q"][s], inp["k"][s], inp["v"][s], g_ref, inp["beta"][s], ref_state)
        eo = max(eo, rel_err(f64(o), ro))
    es = rel_err(f64(state), ref_state)
    print(f"err_o={eo:.2e} err_state={es:.2e}")
    assert eo <= tol and es <= tol, (eo, es)
