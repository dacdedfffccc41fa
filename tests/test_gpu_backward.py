"""Backward pass (kda_chunk_backward) vs the oracle's gradient, element by
element, on seeded inputs and seeded upstream gradients.

Tolerance, per gradient (dq, dk, dv, dg, dbeta, dh0): max|x - x_ref| /
max|x_ref| <= 1e-4 on the fp32 path and <= 1e-2 on the bf16 path, as for the
forward outputs.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_105_amd as kda
import oracle
import synth
from gpu_util import TOL, f64, note, rel_err, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _case(B, T, H, d, dtype, h0=True, lengths=None, g_mode="floored", wid=300, sigma_g=1.0, dht=True):
    inp = synth.prefill_inputs(B, T, H, d, d, dtype, wid=wid, sigma_g=sigma_g, h0=h0, lengths=lengths)
    if g_mode == "weak":
        inp["g"] = torch.full_like(inp["g"], -1e-3)
    elif g_mode == "zero":
        inp["g"] = torch.zeros_like(inp["g"])
    elif g_mode == "raw":  # below the floor in places: the kernel floors, the gradient is 0 there
        x = synth.normal(tuple(inp["g"].shape), wid, "g")
        inp["g"] = (-torch.nn.functional.softplus(x)).to(inp["g"].dtype)
    inp.update(synth.grad_inputs(inp, wid, dht=dht))
    return inp


def _gpu_backward(inp, g=None, gate_mode=None):
    d = to_dev(inp)
    gg = d["g"] if gate_mode is None else (None if g is None else g.cuda())
    out = kda.chunk_backward(d["q"], d["k"], d["v"], gg, d["beta"], d["do"], h0=d.get("h0"),
                             dht=d.get("dht"), cu_seqlens=d.get("cu_seqlens"))
    torch.cuda.synchronize()
    return out


def _oracle_backward(inp, g=None):
    cu = inp.get("cu_seqlens")
    return oracle.backward(inp["q"], inp["k"], inp["v"], inp["g"] if g is None else g, inp["beta"], inp["do"],
                           h0=inp.get("h0"), dht=inp.get("dht"),
                           cu_seqlens=None if cu is None else cu.cpu().numpy())


def _check(name, out, ref, dtype, skip=()):
    errs = {}
    for key in GRADS:
        if key in skip or out.get(key) is None:
            continue
        errs[key] = rel_err(f64(out[key]), ref[key])
    print(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"{name}: {bad}"


CASES = {
    "f32-d64-T256": lambda: _case(1, 256, 2, 64, "f32", h0=False, wid=300),
    "f32-d64-B2-T130": lambda: _case(2, 130, 3, 64, "f32", wid=301),
    "f32-d64-T1": lambda: _case(1, 1, 2, 64, "f32", wid=302),
    "f32-d64-varlen": lambda: _case(1, 0, 2, 64, "f32", lengths=[5, 0, 128, 70], wid=303),
    # many packed sequences (empty ones, exact multiples of the chunk and
    # ragged ones): each chunk finds its sequence by binary search
    "f32-d64-300-seqs": lambda: _case(1, 0, 2, 64, "f32", wid=316,
                                      lengths=[(37 * i) % 193 if i % 7 else 64 * (i % 3) for i in range(300)]),
    "f32-d64-weak-decay": lambda: _case(1, 300, 2, 64, "f32", g_mode="weak", wid=304),
    "f32-d64-no-decay": lambda: _case(1, 256, 2, 64, "f32", g_mode="zero", wid=305),
    "f32-d64-below-floor": lambda: _case(1, 200, 2, 64, "f32", g_mode="raw", wid=306),
    "f32-d64-no-dht": lambda: _case(1, 190, 2, 64, "f32", dht=False, wid=307),
    "bf16-d128-T300": lambda: _case(1, 300, 3, 128, "bf16", wid=308),
    "bf16-d128-varlen": lambda: _case(1, 0, 2, 128, "bf16", lengths=[1, 64, 65, 0, 100, 37], wid=309),
    "bf16-d64-B2-T129": lambda: _case(2, 129, 2, 64, "bf16", wid=310),
    "bf16-d128-weak-decay": lambda: _case(1, 700, 2, 128, "bf16", g_mode="weak", wid=311),
    "bf16-d128-sigma2": lambda: _case(1, 333, 2, 128, "bf16", sigma_g=2.0, wid=312),
    # long chains of chunks with weak or no decay: the state gradient is
    # carried across every chunk of the sequence
    "f32-d64-T4096-weak-decay": lambda: _case(1, 4096, 2, 64, "f32", g_mode="weak", wid=313),
    "bf16-d128-T16384-weak-decay": lambda: _case(1, 16384, 2, 128, "bf16", g_mode="weak", wid=314),
    "bf16-d128-T8192-no-decay": lambda: _case(1, 8192, 2, 128, "bf16", g_mode="zero", wid=315),
}


@pytest.mark.parametrize("name", list(CASES))
def test_chunk_backward(name):
    inp = CASES[name]()
    dtype = "bf16" if inp["q"].dtype == torch.bfloat16 else "f32"
    note(f"chunk_backward {name} q{tuple(inp['q'].shape)} {dtype}")
    out = _gpu_backward(inp)
    ref = _oracle_backward(inp)
    _check(name, out, ref, dtype)


GATE_CASES = {
    "head-bf16-d128-T300": (lambda: _case(1, 300, 2, 128, "bf16", wid=320), "head"),
    "head-f32-d64-varlen": (lambda: _case(1, 0, 2, 64, "f32", lengths=[5, 0, 128, 70], wid=321), "head"),
    "none-bf16-d128-T200": (lambda: _case(1, 200, 2, 128, "bf16", wid=322), "none"),
    "none-f32-d64-B2-T130": (lambda: _case(2, 130, 2, 64, "f32", wid=323), "none"),
}


@pytest.mark.parametrize("name", list(GATE_CASES))
def test_chunk_backward_gates(name):
    """Gated DeltaNet (per-head g) and DeltaNet (no g).  The oracle runs the
    per-head gate broadcast over the channels; its per-channel dg summed over
    the channels is the per-head dg (every channel carries the same g)."""
    make, mode = GATE_CASES[name]
    inp = make()
    dtype = "bf16" if inp["q"].dtype == torch.bfloat16 else "f32"
    if mode == "head":
        g_gpu = inp["g"][..., 0].contiguous()
        g_ref = g_gpu[..., None].expand(inp["g"].shape).contiguous()
    else:
        g_gpu, g_ref = None, torch.zeros_like(inp["g"])
    note(f"chunk_backward gate={mode} {name} q{tuple(inp['q'].shape)}")
    out = _gpu_backward(inp, g=g_gpu, gate_mode=mode)
    ref = _oracle_backward(inp, g=g_ref)
    if mode == "head":
        ref["dg"] = ref["dg"].sum(axis=-1)
        _check(name, out, ref, dtype)
    else:
        assert out["dg"] is None
        _check(name, out, ref, dtype, skip=("dg",))


def test_backward_full_workload_sampled_heads():
    """B=1, H=16, T=4096, d=128 bf16 (the prefill workload), all heads on the
    GPU: every gradient element of heads 0 and 11 against the oracle, and the
    homogeneity identities of the recurrence over all heads:
    <dv, v> + <dh0, h0> = <do, o> + <dht, ht> and <dq, q> = <do, o>."""
    inp = synth.workload_inputs(synth.WORKLOADS[1])
    inp.update(synth.grad_inputs(inp, 1))
    note("chunk_backward workload 1 (T=4096 H=16 d=128 bf16)")
    out = _gpu_backward(inp)
    d = to_dev(inp)
    o, ht = kda.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    torch.cuda.synchronize()
    heads = [0, 11]
    sub = {key: (val[:, :, heads].contiguous() if key in ("q", "k", "v", "g", "beta", "do") else val)
           for key, val in inp.items()}
    sub["h0"] = inp["h0"][:, heads].contiguous()
    sub["dht"] = inp["dht"][:, heads].contiguous()
    ref = _oracle_backward(sub)
    got = {key: (out[key][:, :, heads] if key != "dh0" else out[key][:, heads]) for key in GRADS}
    _check("workload1 heads 0, 11", got, ref, "bf16")
    # identities over all heads, in fp64 from the GPU's own outputs
    v, q, do = f64(d["v"]), f64(d["q"]), f64(d["do"])
    do_o = np.sum(do * f64(o))
    scale = np.sum(np.abs(do * f64(o)))
    lhs = np.sum(f64(out["dv"]) * v) + np.sum(f64(out["dh0"]) * f64(d["h0"]))
    rhs = do_o + np.sum(f64(d["dht"]) * f64(ht))
    print(f"identities: v/h0 {lhs:.6e} vs {rhs:.6e}; q {np.sum(f64(out['dq']) * q):.6e} vs {do_o:.6e}")
    assert abs(lhs - rhs) <= 1e-2 * scale
    assert abs(np.sum(f64(out["dq"]) * q) - do_o) <= 1e-2 * scale


def test_backward_long_context_two_heads():
    """B=1, H=16, T=65,536, d=128 bf16 (the prefill recipe at 16x the
    length, weak decay so the state gradient crosses many chunks): every
    gradient element of heads 2 and 13 against the oracle."""
    T, H, wid = 65536, 16, 360
    inp = synth.prefill_inputs(1, T, H, 128, 128, "bf16", wid=wid, h0=True)
    inp["g"] = torch.full_like(inp["g"], -1e-3)
    inp.update(synth.grad_inputs(inp, wid))
    note(f"chunk_backward T={T} H={H} d=128 bf16, weak decay")
    out = _gpu_backward(inp)
    heads = [2, 13]
    sub = {key: (val[:, :, heads].contiguous() if key in ("q", "k", "v", "g", "beta", "do") else val)
           for key, val in inp.items()}
    sub["h0"] = inp["h0"][:, heads].contiguous()
    sub["dht"] = inp["dht"][:, heads].contiguous()
    ref = _oracle_backward(sub)
    got = {key: (out[key][:, :, heads] if key != "dh0" else out[key][:, heads]) for key in GRADS}
    _check(f"T={T} heads 2, 13", got, ref, "bf16")


def test_backward_packed_workload_sampled_heads():
    """The packed batch (8 sequences, L ~ U[1024, 8192], H=32, d=128, bf16,
    log-decay spread 2): every gradient element of heads 3 and 30 against the
    oracle, and the homogeneity identities over all heads."""
    w = synth.WORKLOADS[2]
    inp = synth.workload_inputs(w)
    inp.update(synth.grad_inputs(inp, w.wid))
    note(f"chunk_backward workload 2 (packed, T={inp['q'].shape[1]} H=32 d=128 bf16)")
    out = _gpu_backward(inp)
    d = to_dev(inp)
    o, ht = kda.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    heads = [3, 30]
    sub = {key: (val[:, :, heads].contiguous() if key in ("q", "k", "v", "g", "beta", "do") else val)
           for key, val in inp.items()}
    sub["dht"] = inp["dht"][:, heads].contiguous()
    ref = _oracle_backward(sub)
    got = {key: (out[key][:, :, heads] if key != "dh0" else out[key][:, heads]) for key in GRADS}
    _check("workload2 heads 3, 30", got, ref, "bf16")
    v, q, do = f64(d["v"]), f64(d["q"]), f64(d["do"])
    do_o = np.sum(do * f64(o))
    scale = np.sum(np.abs(do * f64(o)))
    lhs = np.sum(f64(out["dv"]) * v)  # h0 = 0 here
    rhs = do_o + np.sum(f64(d["dht"]) * f64(ht))
    assert abs(lhs - rhs) <= 1e-2 * scale
    assert abs(np.sum(f64(out["dq"]) * q) - do_o) <= 1e-2 * scale


def test_backward_split_resume():
    """The gradient of a sequence equals that of its two halves run with the
    state and the state gradient handed across (split at a chunk boundary
    and inside a chunk)."""
    inp = _case(1, 400, 2, 64, "f32", wid=330)
    d = to_dev(inp)
    full = kda.chunk_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], h0=d["h0"], dht=d["dht"])
    for t1 in (128, 150):
        note(f"chunk_backward split at {t1}")
        sl = lambda x, a, b: x[:, a:b].contiguous()  # noqa: E731
        _, mid = kda.chunk_forward(sl(d["q"], 0, t1), sl(d["k"], 0, t1), sl(d["v"], 0, t1), sl(d["g"], 0, t1),
                                   sl(d["beta"], 0, t1), h0=d["h0"])
        tail = kda.chunk_backward(*(sl(d[x], t1, 400) for x in ("q", "k", "v", "g", "beta", "do")),
                                  h0=mid, dht=d["dht"])
        head = kda.chunk_backward(*(sl(d[x], 0, t1) for x in ("q", "k", "v", "g", "beta", "do")),
                                  h0=d["h0"], dht=tail["dh0"])
        torch.cuda.synchronize()
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            joined = torch.cat([head[key], tail[key]], dim=1)
            e = rel_err(f64(joined), f64(full[key]))
            assert e <= 1e-4, (t1, key, e)
        assert rel_err(f64(head["dh0"]), f64(full["dh0"])) <= 1e-4


def test_backward_no_tokens():
    """T = 0: nothing to differentiate through, dh0 = dht exactly."""
    inp = _case(1, 0, 2, 64, "f32", lengths=[0, 0], wid=332)
    note("chunk_backward T=0")
    out = _gpu_backward(inp)
    assert torch.equal(out["dh0"].cpu(), inp["dht"])
    assert out["dq"].numel() == 0 and out["dbeta"].numel() == 0


def test_backward_deterministic():
    inp = _case(1, 300, 2, 128, "bf16", wid=331)
    note("chunk_backward determinism")
    a = _gpu_backward(inp)
    b = _gpu_backward(inp)
    for key in GRADS:
        assert torch.equal(a[key], b[key]), key


def _both(d, g="same", **kw):
    """The sequential call, then two overlapped calls in a row (the second
    one's outputs copied on the calling stream straight after it, before any
    synchronisation: the copy must see the finished gradients).  g: the gate
    to pass instead of d["g"] (a per-head gate, or None)."""
    args = (d["q"], d["k"], d["v"], d["g"] if isinstance(g, str) else g, d["beta"], d["do"])
    kw = dict(h0=d.get("h0"), dht=d.get("dht"), cu_seqlens=d.get("cu_seqlens"), **kw)
    seq = kda.chunk_backward(*args, **kw)
    kda.chunk_backward(*args, overlap=True, **kw)
    ov = kda.chunk_backward(*args, overlap=True, **kw)
    copy = {key: None if ov[key] is None else ov[key].clone() for key in GRADS}
    torch.cuda.synchronize()
    return seq, copy


@pytest.mark.parametrize("name", ["f32_B2_T300_d64", "bf16_packed_ragged_d128", "bf16_T0"])
def test_backward_overlapped_matches_sequential(name):
    """kda_chunk_backward_overlapped (forward replay on a second stream) gives
    the sequential call's results bit for bit, and against the oracle."""
    if name == "f32_B2_T300_d64":
        inp = _case(2, 300, 2, 64, "f32", wid=340)
    elif name == "bf16_packed_ragged_d128":
        inp = _case(1, 0, 2, 128, "bf16", lengths=[130, 1, 64, 257], wid=341)
    else:
        inp = _case(1, 0, 2, 128, "bf16", lengths=[0, 0], wid=342)
    note(f"chunk_backward overlapped {name}")
    seq, ov = _both(to_dev(inp))
    for key in GRADS:
        assert (seq[key] is None) == (ov[key] is None), key
        if seq[key] is not None:
            assert torch.equal(seq[key], ov[key]), key
    if inp["q"].shape[1] > 0:
        _check(name + " overlapped", ov, _oracle_backward(inp), "f32" if name.startswith("f32") else "bf16")


def test_backward_overlapped_full_workload():
    """The overlapped call at the benchmarked size (B=1, H=16, T=4096, d=128,
    bf16) equals the sequential call bit for bit."""
    w = synth.WORKLOADS[1]
    note("chunk_backward overlapped, T=4096 H=16 workload")
    inp = synth.workload_inputs(w, device="cuda")
    inp.update(synth.grad_inputs(inp, w.wid, device="cuda"))
    seq, ov = _both(inp)
    for key in GRADS:
        if seq[key] is not None:
            assert torch.equal(seq[key], ov[key]), key


@pytest.mark.parametrize("name,mode", [("head-bf16-d64-T300", "head"), ("none-bf16-d128-varlen", "none")])
def test_backward_overlapped_gates(name, mode):
    """The overlapped call with a per-head gate (Gated DeltaNet) and with none
    (DeltaNet) equals the sequential call bit for bit."""
    if name.startswith("head"):
        inp = _case(1, 300, 2, 64, "bf16", wid=343)
    else:
        inp = _case(1, 0, 2, 128, "bf16", lengths=[200, 3, 129], wid=344)
    d = to_dev(inp)
    g = d["g"][..., 0].contiguous() if mode == "head" else None
    note(f"chunk_backward overlapped gate={mode} {name}")
    seq, ov = _both(d, g=g)
    for key in GRADS:
        assert (seq[key] is None) == (ov[key] is None), key
        if seq[key] is not None:
            assert torch.equal(seq[key], ov[key]), key


@pytest.mark.parametrize("name", ["f32_B2_T300_d64", "bf16_T4096_H16"])
def test_backward_timed_matches_sequential(name):
    """kda_chunk_backward_timed (HIP events recorded on the launch stream
    before each stage and after the last) returns the plain call's gradients
    bit for bit, and the stage times it brackets are non-negative and add up
    to the whole."""
    if name.startswith("f32"):
        d = to_dev(_case(2, 300, 2, 64, "f32", wid=350))
    else:
        w = synth.WORKLOADS[1]
        d = synth.workload_inputs(w, device="cuda")
        d.update(synth.grad_inputs(d, w.wid, device="cuda"))
    note(f"chunk_backward timed {name}")
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"])
    kw = dict(h0=d.get("h0"), dht=d.get("dht"), cu_seqlens=d.get("cu_seqlens"))
    seq = kda.chunk_backward(*args, **kw)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(kda.BWD_STAGES) + 1)]
    for e in ev:
        e.record()  # creates the event
    torch.cuda.synchronize()
    timed = kda.chunk_backward(*args, events=[e.cuda_event for e in ev], **kw)
    torch.cuda.synchronize()
    for key in GRADS:
        assert (seq[key] is None) == (timed[key] is None), key
        if seq[key] is not None:
            assert torch.equal(seq[key], timed[key]), key
    parts = [ev[j].elapsed_time(ev[j + 1]) for j in range(len(kda.BWD_STAGES))]
    total = ev[0].elapsed_time(ev[-1])
    print(f"{name}: stages " + " ".join(f"{s}={t * 1e3:.1f}us" for s, t in zip(kda.BWD_STAGES, parts)))
    assert all(t >= 0 for t in parts) and total > 0
    assert abs(sum(parts) - total) <= 1e-3 + 1e-3 * total


def _window_budget(inp, W):
    """Workspace bytes for windows of about W chunks: the default size less
    the per-chunk areas (fp32 record, scratch at d = 64, end-state gradient) of the
    chunks beyond n_rows W slots, plus the two carry states per (sequence,
    head) that windows add."""
    B, T, H, d = inp["q"].shape
    cu = inp.get("cu_seqlens")
    rows = B if cu is None else cu.numel() - 1
    chunks = (T + 63) // 64
    n_slots = rows * chunks if cu is None else chunks + rows
    # at d = 128 no copies of v, dO and Gamma in the record, and no scratch
    # (the local-gradient kernel keeps it on chip)
    blocks, scr = (5, 0) if d == 128 else (8, 5 * 64 * d + 2 * 64 * 64 + d)
    per_slot = H * ((blocks * 64 * d + 3 * 64 * 64 + d + 64 + scr) * 4 + d * d * 4)
    full = kda.backward_workspace_bytes(B, T, H, d, inp["q"].dtype, n_seqs=0 if cu is None else rows)
    return full - (n_slots - rows * W) * per_slot + 2 * rows * H * d * d * 4 + 4 * 256


@pytest.mark.parametrize("name", ["f32_B2_T1000_d64", "bf16_packed_d128"])
def test_backward_windows_match(name):
    """A workspace smaller than the default makes the call process the chunks
    in windows (the last window first, the state gradient carried across
    window edges): the gradients equal the one-window call's bit for bit,
    sequential and overlapped, and the oracle's."""
    if name.startswith("f32"):
        inp, widths, dt = _case(2, 1000, 2, 64, "f32", wid=370), (5, 1), "f32"
    else:
        inp, widths, dt = _case(1, 0, 2, 128, "bf16", lengths=[700, 0, 64, 1000, 130], wid=371), (6, 3), "bf16"
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"])
    kw = dict(h0=d.get("h0"), dht=d.get("dht"), cu_seqlens=d.get("cu_seqlens"))
    note(f"chunk_backward windows {name}: one window")
    one = kda.chunk_backward(*args, **kw)
    torch.cuda.synchronize()
    _check(name + " one window", one, _oracle_backward(inp), dt)
    for W in widths:
        ws = torch.empty(_window_budget(inp, W), dtype=torch.uint8, device="cuda")
        for overlap in (False, True):
            note(f"chunk_backward windows {name}: about {W} chunks, overlap={overlap}")
            got = kda.chunk_backward(*args, workspace=ws, overlap=overlap, **kw)
            torch.cuda.synchronize()
            for key in GRADS:
                assert torch.equal(one[key], got[key]), (W, overlap, key)


@pytest.mark.parametrize("name", ["f32_B2_T300_d64", "bf16_packed_d128", "bf16_deltanet_d128"])
def test_autograd_matches_chunk_backward(name):
    """kda_chunk under torch.autograd gives chunk_backward's gradients bit for
    bit, for a loss whose gradients with respect to o and ht are seeded
    tensors (o's cast to o's dtype, as autograd passes it)."""
    if name.startswith("f32"):
        inp = _case(2, 300, 2, 64, "f32", wid=380)
    else:
        inp = _case(1, 0, 2, 128, "bf16", lengths=[130, 1, 64, 257], wid=381)
    d = to_dev(inp)
    g = None if name.endswith("deltanet_d128") else d["g"]
    note(f"kda_chunk autograd {name}")
    leaves = {key: d[key].clone().requires_grad_(True) for key in ("q", "k", "v", "beta", "h0") if d.get(key) is not None}
    gl = None if g is None else g.clone().requires_grad_(True)
    o, ht = kda.kda_chunk(leaves["q"], leaves["k"], leaves["v"], gl, leaves["beta"], h0=leaves.get("h0"),
                          cu_seqlens=d.get("cu_seqlens"))
    r_o = torch.randn(o.shape, generator=torch.Generator().manual_seed(382)).cuda()
    r_h = torch.randn(ht.shape, generator=torch.Generator().manual_seed(383)).cuda()
    ((o.float() * r_o).sum() + (ht * r_h).sum()).backward()
    ref = kda.chunk_backward(d["q"], d["k"], d["v"], g, d["beta"], r_o.to(o.dtype), h0=d.get("h0"), dht=r_h,
                             cu_seqlens=d.get("cu_seqlens"))
    torch.cuda.synchronize()
    pairs = [("dq", leaves["q"]), ("dk", leaves["k"]), ("dv", leaves["v"]), ("dbeta", leaves["beta"])]
    if gl is not None:
        pairs.append(("dg", gl))
    if "h0" in leaves:
        pairs.append(("dh0", leaves["h0"]))
    for key, leaf in pairs:
        assert leaf.grad is not None and torch.equal(leaf.grad, ref[key]), key
