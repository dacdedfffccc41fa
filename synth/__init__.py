"""Seeded synthetic inputs for the KDA workloads.

This module only draws random tensors with the value distributions of the
workloads; it contains none of the KDA arithmetic.  Both sides of every
parity check (the HIP library and the CPU oracle) read the very same tensors
produced here: bf16 tensors are rounded once (round to nearest even) and the
oracle up-converts those exact values.

Distributions (per workload): q, k ~ N(0, 1) then L2-normalised over the key
dimension per (token, head); v ~ N(0, 1); beta = sigmoid(N(0, 1)) in fp32;
log-decay g = max(-softplus(sigma_g * N(0, 1)), floor) per key channel; initial
state 0.02 * N(0, 1) in fp32 where the workload has one.  N(mu, s) means a
standard deviation of s.  The L2 normalisation of q and k follows the toy loop
of "Kimi K3 深度拆解" (chenxutan.com), 4.2, which assumes normalised q and k;
beta in (0, 1) is the write strength given there.

Every tensor is drawn from its own torch generator seeded from
(workload id, tensor id, block id), blockwise over tokens (65,536 per block) so
that host memory stays bounded for the million-token workload.  Generation can
run on the CPU or on the GPU (``device="cuda"``); the two give different bits,
so a check must feed both sides from one call.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "beta": 3, "g": 4, "h0": 5,
              "lengths": 6, "positions": 7, "state": 8, "do": 9, "dht": 10}
BLOCK_TOKENS = 65536
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One seeded synthetic workload (shapes, dtype and distributions)."""
    wid: int
    name: str
    kind: str                  # "prefill" or "decode"
    H: int
    dk: int
    dv: int
    dtype: str                 # dtype of q, k, v, g and o
    B: int = 1
    T: int = 0                 # tokens per sequence (prefill, fixed length)
    n_seqs: int = 0            # > 0: packed variable-length batch
    len_range: tuple = ()      # (lo, hi) inclusive, for packed batches
    sigma_g: float = 1.0
    g_floor: float = -0.125
    chunk: int = 64
    h0: bool = False
    N: int = 0                 # decode: concurrent sequences
    steps: int = 0             # decode: consecutive steps
    extra: Dict = field(default_factory=dict)


WORKLOADS = {
    0: Workload(0, "kda-prefill-fp32-B1-H2-T256-d64", "prefill", H=2, dk=64, dv=64,
                dtype="f32", B=1, T=256, h0=False),
    1: Workload(1, "kda-prefill-bf16-B1-H16-T4096-d128", "prefill", H=16, dk=128,
                dv=128, dtype="bf16", B=1, T=4096, h0=True),
    2: Workload(2, "kda-prefill-varlen-bf16-8seq-L1024..8192-H32-d128", "prefill",
                H=32, dk=128, dv=128, dtype="bf16", n_seqs=8,
                len_range=(1024, 8192), sigma_g=2.0, h0=False),
    3: Workload(3, "kda-prefill-bf16-B1-H16-T1048576-d128", "prefill", H=16,
                dk=128, dv=128, dtype="bf16", B=1, T=1 << 20, h0=True),
    4: Workload(4, "kda-decode-bf16-N256-H32-d128-1000steps", "decode", H=32,
                dk=128, dv=128, dtype="bf16", N=256, steps=1000, h0=True),
    # a serving-like batch: many short requests packed into one call
    5: Workload(5, "kda-prefill-serving-bf16-512seq-L64..512-H32-d128", "prefill",
                H=32, dk=128, dv=128, dtype="bf16", n_seqs=512,
                len_range=(64, 512), h0=True),
}


def seed_of(wid: int, tensor: str, block: int = 0) -> int:
    return ((wid * 1009 + TENSOR_IDS[tensor]) * 1_000_003 + block) & 0x7FFF_FFFF_FFFF


def normal(shape, wid: int, tensor: str, block: int = 0, device="cpu") -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(wid, tensor, block))
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def packed_lengths(wid: int, n_seqs: int, lo: int, hi: int) -> list:
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed_of(wid, "lengths"))
    return [int(x) for x in torch.randint(lo, hi + 1, (n_seqs,), generator=gen)]


def prefill_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
                   wid: int = 100, sigma_g: float = 1.0, g_floor: float = -0.125,
                   h0: bool = False, lengths: Optional[list] = None,
                   device="cpu") -> dict:
    """Inputs for one chunked forward.

    With ``lengths`` the batch is packed: B must be 1, T = sum(lengths), and
    ``cu_seqlens`` (int32, [n+1]) is returned.  Layout is [B, T, H, d].
    """
    dt = DTYPES[dtype]
    if lengths is not None:
        assert B == 1
        T = int(sum(lengths))
    out = {k: torch.empty((B, T, H, d), dtype=dt, device=device)
           for k, d in (("q", dk), ("k", dk), ("v", dv), ("g", dk))}
    out["beta"] = torch.empty((B, T, H), dtype=torch.float32, device=device)
    nblk = max(1, math.ceil(T / BLOCK_TOKENS))
    for b in range(B):
        for blk in range(nblk):
            t0, t1 = blk * BLOCK_TOKENS, min(T, (blk + 1) * BLOCK_TOKENS)
            if t1 <= t0:
                continue
            n = t1 - t0
            bid = b * 4096 + blk
            out["q"][b, t0:t1] = _unit(normal((n, H, dk), wid, "q", bid, device)).to(dt)
            out["k"][b, t0:t1] = _unit(normal((n, H, dk), wid, "k", bid, device)).to(dt)
            out["v"][b, t0:t1] = normal((n, H, dv), wid, "v", bid, device).to(dt)
            out["beta"][b, t0:t1] = torch.sigmoid(normal((n, H), wid, "beta", bid, device))
            x = normal((n, H, dk), wid, "g", bid, device)
            out["g"][b, t0:t1] = (-torch.nn.functional.softplus(sigma_g * x)).clamp_min(g_floor).to(dt)
    n_states = len(lengths) if lengths is not None else B
    out["h0"] = (0.02 * normal((n_states, H, dk, dv), wid, "h0", 0, device)) if h0 else None
    if lengths is not None:
        cu = [0]
        for L in lengths:
            cu.append(cu[-1] + int(L))
        out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=device)
    else:
        out["cu_seqlens"] = None
    out["g_floor"] = g_floor
    return out


def grad_inputs(inp: dict, wid: int, dht: bool = True, device="cpu") -> dict:
    """Upstream gradients for a backward call on the inputs `inp` of
    prefill_inputs: do ~ N(0, 1) in the shape and dtype of v (drawn per
    65,536-token block like the inputs), dht ~ N(0, 1) fp32 in the shape of
    the final state, or None."""
    v = inp["v"]
    B, T, H, dv = v.shape
    dk = inp["q"].shape[-1]
    do = torch.empty_like(v, device=device)
    nblk = max(1, math.ceil(T / BLOCK_TOKENS))
    for b in range(B):
        for blk in range(nblk):
            t0, t1 = blk * BLOCK_TOKENS, min(T, (blk + 1) * BLOCK_TOKENS)
            if t1 > t0:
                do[b, t0:t1] = normal((t1 - t0, H, dv), wid, "do", b * 4096 + blk, device).to(v.dtype)
    cu = inp.get("cu_seqlens")
    n_states = B if cu is None else cu.numel() - 1
    out = {"do": do, "dht": None}
    if dht:
        out["dht"] = normal((n_states, H, dk, dv), wid, "dht", 0, device)
    return out


def workload_inputs(w: Workload, device="cpu") -> dict:
    """Inputs of a prefill workload, full size."""
    assert w.kind == "prefill"
    lengths = None
    if w.n_seqs:
        lengths = packed_lengths(w.wid, w.n_seqs, *w.len_range)
    return prefill_inputs(w.B, w.T, w.H, w.dk, w.dv, w.dtype, wid=w.wid,
                          sigma_g=w.sigma_g, g_floor=w.g_floor, h0=w.h0,
                          lengths=lengths, device=device)


def decode_inputs(N: int, H: int, dk: int, dv: int, steps: int, dtype: str = "bf16",
                  wid: int = 104, sigma_g: float = 1.0, g_floor: float = -0.125,
                  device="cpu") -> dict:
    """Pre-staged per-step inputs [steps, N, H, d] and the initial state."""
    dt = DTYPES[dtype]
    q = torch.empty((steps, N, H, dk), dtype=dt, device=device)
    k = torch.empty_like(q)
    g = torch.empty_like(q)
    v = torch.empty((steps, N, H, dv), dtype=dt, device=device)
    beta = torch.empty((steps, N, H), dtype=torch.float32, device=device)
    for s in range(steps):
        q[s] = _unit(normal((N, H, dk), wid, "q", s, device)).to(dt)
        k[s] = _unit(normal((N, H, dk), wid, "k", s, device)).to(dt)
        v[s] = normal((N, H, dv), wid, "v", s, device).to(dt)
        beta[s] = torch.sigmoid(normal((N, H), wid, "beta", s, device))
        x = normal((N, H, dk), wid, "g", s, device)
        g[s] = (-torch.nn.functional.softplus(sigma_g * x)).clamp_min(g_floor).to(dt)
    state = 0.02 * normal((N, H, dk, dv), wid, "state", 0, device)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "state": state,
            "g_floor": g_floor}


def to_mxfp8(x: torch.Tensor):
    """MXFP8 encoding of x along its last dimension (input preparation, no
    KDA arithmetic): blocks of 32 consecutive elements share one power-of-two
    scale 2^E with E = floor(log2 amax) - 8 (8 is the exponent of e4m3's
    largest power of two), clamped to [-127, 127]; each element is x / 2^E
    saturated to +-448 and rounded to nearest even in e4m3 (finite-only
    encoding, OCP MX).  Returns (e4m3 bytes as uint8, scale bytes E + 127 as
    uint8 [..., d / 32], the decoded values in fp32: exactly what the bytes
    mean, which both sides of a parity check use)."""
    shp = x.shape
    xb = x.float().reshape(*shp[:-1], shp[-1] // 32, 32)
    amax = xb.abs().amax(-1, keepdim=True)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)), torch.full_like(amax, -127.0)) - 8
    e = e.clamp(-127, 127)
    scale = torch.exp2(e)
    f8 = (xb / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    dec = f8.float() * scale
    return (f8.view(torch.uint8).reshape(shp), (e + 127).to(torch.uint8).squeeze(-1),
            dec.reshape(shp))


def mxfp8_inputs(inp: dict) -> dict:
    """The prefill inputs with q, k and v in MXFP8: adds q8/k8/v8 (bytes) and
    q_scale/k_scale/v_scale, and replaces q, k, v by their decoded values
    (fp32) for the oracle."""
    out = dict(inp)
    for name in ("q", "k", "v"):
        b, sc, dec = to_mxfp8(inp[name])
        out[name + "8"], out[name + "_scale"], out[name] = b, sc, dec
    return out


def sample_positions(wid: int, T: int, n: int) -> list:
    """n distinct token positions in [0, T), seeded."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed_of(wid, "positions"))
    return sorted(int(x) for x in torch.randperm(T, generator=gen)[:n])
