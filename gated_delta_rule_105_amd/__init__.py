"""MI355X-native Kimi Delta Attention (KDA): chunked prefill and decode step.

Thin PyTorch-facing layer over the C ABI of ``libkda.so`` (include/kda.h).
PyTorch supplies device memory and the current HIP stream; all arithmetic
runs in the library's HIP kernels.  There is no CPU fallback: calling into a
missing library raises.

    o, ht = chunk_forward(q, k, v, g, beta, h0=None, cu_seqlens=None)
    o, ht, states = chunk_forward_states(q, k, v, g, beta, states_every=16)
    o = decode_step(q, k, v, g, beta, state)          # state updated in place
    grads = chunk_backward(q, k, v, g, beta, do, h0=None, dht=None)

g selects the gate: [.., H, d] one log-decay per key channel (KDA), [.., H]
one per head (Gated DeltaNet), None no decay (DeltaNet).

KDA is the gated delta rule with a channel-wise forget gate,
S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
o_t = S_t^T q_t, alpha_t = exp(max(g_t, g_floor)) ("Kimi K3 深度拆解"
(chenxutan.com), 4.2 "线性注意力与 Delta Rule"; "Kimi K3 技術報告"
(akiraxclaw.com), "長度：KDA 為什麼還要搭配 Gated MLA？").
"""
from __future__ import annotations

from typing import Optional, Tuple

from ._lib import (BWD_STAGES, CHUNK_LAUNCHES, KDA_DTYPE_BF16, KDA_DTYPE_F32, KDA_GATE_CHANNEL, KDA_GATE_HEAD,
                   KDA_GATE_NONE, KDA_OK, ChunkDesc, ChunkDescEx, KdaError, status_string, version)
from . import _lib

__all__ = ["chunk_forward", "chunk_forward_noalloc", "chunk_forward_states", "chunk_forward_mx", "chunk_backward", "decode_step",
           "kda_chunk",
           "workspace_bytes", "backward_workspace_bytes", "make_desc", "make_desc_ex", "KdaError", "status_string",
           "version",
           "CHUNK_LAUNCHES", "BWD_STAGES"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t}; KDA takes bfloat16 or float32")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(name, t, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def make_desc(B: int, T: int, H: int, d: int, dtype, n_seqs: int = 0, chunk: int = 64,
              g_floor: float = -0.125) -> ChunkDesc:
    return ChunkDesc(B=B, T=T, H=H, d_k=d, d_v=d, chunk=chunk, n_seqs=n_seqs,
                     dtype=_dtype_code(dtype), g_floor=g_floor)


def make_desc_ex(B: int, T: int, H: int, d: int, dtype, n_seqs: int = 0, chunk: int = 64,
                 g_floor: float = -0.125, gate: int = KDA_GATE_CHANNEL) -> ChunkDescEx:
    return ChunkDescEx(shape=make_desc(B, T, H, d, dtype, n_seqs, chunk, g_floor), gate=gate)


class _on_stream:
    """Context in which torch allocates from the pool of the stream the
    library enqueues on, so that a tensor freed on return (a workspace) is
    not handed to other work while that stream still uses it."""

    def __init__(self, stream, device):
        self.ctx = None
        if stream is not None:
            torch = _torch()
            self.ctx = torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device))

    def __enter__(self):
        if self.ctx is not None:
            self.ctx.__enter__()

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)


def _gate_of(g, full_dims: int) -> int:
    """Gate layout from g: per channel (full_dims dims), per head (one fewer), none."""
    if g is None:
        return KDA_GATE_NONE
    if g.dim() == full_dims:
        return KDA_GATE_CHANNEL
    if g.dim() == full_dims - 1:
        return KDA_GATE_HEAD
    raise ValueError(f"g must have {full_dims} (per channel) or {full_dims - 1} (per head) dims, or be None")


def workspace_bytes(B: int, T: int, H: int, d: int, dtype, n_seqs: int = 0, chunk: int = 64,
                    g_floor: float = -0.125) -> int:
    """Device workspace one chunk_forward call of this shape needs."""
    return _lib.workspace_size(make_desc(B, T, H, d, dtype, n_seqs, chunk, g_floor))


def check_cu_seqlens(cu, T: int) -> None:
    """Host-side check of packed-sequence offsets (the library trusts them)."""
    c = [int(x) for x in (cu.tolist() if hasattr(cu, "tolist") else cu)]
    if len(c) < 2 or c[0] != 0 or c[-1] != T or any(b < a for a, b in zip(c, c[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")


def chunk_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 64,
                  g_floor: float = -0.125, *, o=None, ht=None, workspace=None,
                  output_final_state: bool = True, validate_cu: bool = True,
                  stream=None, events=None) -> Tuple[object, object]:
    """Chunked KDA forward over whole sequences.

    q, k: [B, T, H, d]; v: [B, T, H, d] (bf16 or fp32); beta: [B, T, H] fp32.
    g: [B, T, H, d] (KDA), [B, T, H] (Gated DeltaNet) or None (DeltaNet).
    cu_seqlens: int32 device tensor [n+1] for n packed sequences (B == 1).
    h0: fp32 [S, H, d, d] or None.  Returns (o [B, T, H, d], ht [S, H, d, d]
    fp32, or None when output_final_state is False).
    events: optional len(CHUNK_LAUNCHES) + 1 raw hipEvent_t handles recorded
    around the call's launches (kda_chunk_forward_timed), for measurement.
    """
    o, ht, _ = _forward(q, k, v, g, beta, h0, cu_seqlens, chunk, g_floor, o, ht, workspace,
                        output_final_state, validate_cu, stream, events, None, 0)
    return o, ht


def chunk_forward_noalloc(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 64,
                          g_floor: float = -0.125, *, o, ht=None, validate_cu: bool = True,
                          stream=None) -> None:
    """chunk_forward through kda_chunk_forward_noalloc, for callers that
    cannot allocate: no workspace (the library's fixed per-device scratch
    serves), and the outputs are the caller's: o [B, T, H, d] in q's dtype,
    ht fp32 [S, H, d, d] or None (final state not written).  KDA gate (g per
    key channel) only.  Calls on one device must not overlap (they share the
    scratch); calls ordered on one stream are safe."""
    torch = _torch()
    B, T, H, d = q.shape
    dt = q.dtype
    _check_dev("q", q, dt)
    for name, t in (("k", k), ("v", v), ("g", g)):
        _check_dev(name, t, dt, (B, T, H, d))
    _check_dev("beta", beta, torch.float32, (B, T, H))
    n_seqs = 0
    if cu_seqlens is not None:
        _check_dev("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        if validate_cu:
            check_cu_seqlens(cu_seqlens.cpu(), T)
    S = n_seqs if n_seqs else B
    _check_dev("h0", h0, torch.float32, (S, H, d, d))
    _check_dev("o", o, dt, (B, T, H, d))
    _check_dev("ht", ht, torch.float32, (S, H, d, d))
    desc = make_desc(B, T, H, d, dt, n_seqs, chunk, g_floor)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.chunk_forward_noalloc_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                        _ptr(cu_seqlens), _ptr(o), _ptr(ht), stream)
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_forward_noalloc")


def chunk_forward_states(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 64,
                         g_floor: float = -0.125, *, states_every: int = 1, states=None, o=None, ht=None,
                         workspace=None, output_final_state: bool = True, validate_cu: bool = True,
                         stream=None) -> Tuple[object, object, object]:
    """chunk_forward that also returns the state after every `states_every`
    full chunks of each sequence (kda_chunk_forward_states): states is fp32
    [count, H, d, d], the slots of each sequence consecutive and in order;
    slot m - 1 of sequence n holds the state after its first
    m * states_every * chunk tokens.  With packed sequences, count is an
    upper bound and the slots past the last one written are left as given
    (zeros when allocated here)."""
    torch = _torch()
    B, T, H, d = q.shape
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    count = _lib.states_count(make_desc(B, T, H, d, q.dtype, n_seqs, chunk, g_floor), states_every)
    if states is None:
        states = torch.zeros((count, H, d, d), dtype=torch.float32, device=q.device)
    _check_dev("states", states, torch.float32, (count, H, d, d))
    return _forward(q, k, v, g, beta, h0, cu_seqlens, chunk, g_floor, o, ht, workspace, output_final_state,
                    validate_cu, stream, None, states, states_every)


def chunk_forward_mx(q, q_scale, k, k_scale, v, v_scale, g, beta, h0=None, cu_seqlens=None, chunk: int = 64,
                     g_floor: float = -0.125, *, o=None, ht=None, workspace=None,
                     output_final_state: bool = True, validate_cu: bool = True,
                     stream=None) -> Tuple[object, object]:
    """chunk_forward with q, k, v in MXFP8 (kda_chunk_forward_mx): uint8
    tensors [B, T, H, d] of e4m3 bytes and uint8 scale tensors [B, T, H, d/32]
    (2^(s - 127) per block of 32 channels).  g (bf16, per channel or per
    head, or None) and o are bf16."""
    torch = _torch()
    B, T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.uint8, (B, T, H, d))
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check_dev(name, t, torch.uint8, (B, T, H, d // 32))
    o, ht, _ = _forward(q, k, v, g, beta, h0, cu_seqlens, chunk, g_floor, o, ht, workspace, output_final_state,
                        validate_cu, stream, None, None, 0, mx=(q_scale, k_scale, v_scale))
    return o, ht


def _forward(q, k, v, g, beta, h0, cu_seqlens, chunk, g_floor, o, ht, workspace, output_final_state,
             validate_cu, stream, events, states, states_every, mx=None):
    torch = _torch()
    B, T, H, d = q.shape
    dt = torch.bfloat16 if mx is not None else q.dtype  # dtype of g, o (and q, k, v without MXFP8)
    if mx is None:
        _check_dev("q", q, dt)
        for name, t in (("k", k), ("v", v)):
            _check_dev(name, t, dt, (B, T, H, d))
    gate = _gate_of(g, 4)
    _check_dev("g", g, dt, (B, T, H, d) if gate == KDA_GATE_CHANNEL else (B, T, H))
    _check_dev("beta", beta, torch.float32, (B, T, H))
    n_seqs = 0
    if cu_seqlens is not None:
        _check_dev("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        if validate_cu:
            check_cu_seqlens(cu_seqlens.cpu(), T)
    S = n_seqs if n_seqs else B
    _check_dev("h0", h0, torch.float32, (S, H, d, d))
    desc = make_desc(B, T, H, d, dt, n_seqs, chunk, g_floor)
    dx = ChunkDescEx(shape=desc, gate=gate)
    ws_bytes = _lib.workspace_size(desc)
    with _on_stream(stream, q.device):
        if o is None:
            o = torch.empty((B, T, H, d), dtype=dt, device=q.device)
        if ht is None and output_final_state:
            ht = torch.empty((S, H, d, d), dtype=torch.float32, device=q.device)
        if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _check_dev("o", o, dt, (B, T, H, d))
    _check_dev("ht", ht, torch.float32, (S, H, d, d))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), _ptr(o), _ptr(ht))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), stream)
    if mx is not None:
        st = _lib.chunk_forward_mx_raw(dx, _ptr(q), _ptr(mx[0]), _ptr(k), _ptr(mx[1]), _ptr(v), _ptr(mx[2]),
                                       *ptrs[3:], *tail)
        what = "kda_chunk_forward_mx"
    elif states is not None:
        st = _lib.chunk_forward_states_raw(dx, *ptrs, _ptr(states) if states.numel() else None, states_every,
                                           *tail)
        what = "kda_chunk_forward_states"
    elif events is not None:
        st = _lib.chunk_forward_timed_raw(dx, *ptrs, *tail, events)
        what = "kda_chunk_forward_timed"
    elif gate == KDA_GATE_CHANNEL:
        st = _lib.chunk_forward_raw(desc, *ptrs, *tail)
        what = "kda_chunk_forward"
    else:
        st = _lib.chunk_forward_gated_raw(dx, *ptrs, *tail)
        what = "kda_chunk_forward_gated"
    if st != KDA_OK:
        raise KdaError(st, what)
    return o, ht, states


def backward_workspace_bytes(B: int, T: int, H: int, d: int, dtype, n_seqs: int = 0, chunk: int = 64,
                             g_floor: float = -0.125) -> int:
    """Device workspace one chunk_backward call of this shape needs (any gate)."""
    return _lib.backward_workspace_size(make_desc(B, T, H, d, dtype, n_seqs, chunk, g_floor))


_AUX = {}


def _aux_stream(dev):
    """Second stream and fork/join events of `dev` for overlapped backward
    calls (created once per device; the events are recorded once so that
    their handles exist)."""
    torch = _torch()
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx not in _AUX:
        with torch.cuda.device(idx):
            side = torch.cuda.Stream()
            evs = [torch.cuda.Event(), torch.cuda.Event()]
            for e in evs:
                e.record()
            torch.cuda.current_stream().synchronize()
        _AUX[idx] = (side, evs)
    side, evs = _AUX[idx]
    return side.cuda_stream, evs[0].cuda_event, evs[1].cuda_event


def chunk_backward(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, chunk: int = 64,
                   g_floor: float = -0.125, *, want_dh0: bool = True, out=None, workspace=None,
                   validate_cu: bool = True, stream=None, events=None, overlap: bool = False) -> dict:
    """Gradients of L = <do, o> + <dht, ht> for chunk_forward with the same
    inputs (kda_chunk_backward).  do: [B, T, H, d] in the input dtype; dht:
    fp32 [S, H, d, d] or None (zero).  Returns a dict with dq, dk, dv (input
    dtype), dg (the layout of g, input dtype; None without a gate), dbeta
    (fp32 [B, T, H]) and dh0 (fp32 [S, H, d, d], or None when want_dh0 is
    False).  `out` may supply those tensors.  events: optional
    len(BWD_STAGES) + 1 raw hipEvent_t handles (kda_chunk_backward_timed).
    overlap: run the forward replay, and the local gradients of all but the
    first range of chunks, on a second stream of the device beside the
    state-gradient walk (it forks after the record stage;
    kda_chunk_backward_overlapped, the same results).  Overlapped calls on one device share that stream and its
    events, so they must be issued from one host thread.  workspace: a uint8
    device tensor used as it is; the call fits its windows of chunks to its
    size (smaller than backward_workspace_bytes(...) means narrower windows,
    too small raises KdaError).  None allocates the default size."""
    torch = _torch()
    B, T, H, d = q.shape
    dt = q.dtype
    _check_dev("q", q, dt)
    for name, t in (("k", k), ("v", v), ("do", do)):
        _check_dev(name, t, dt, (B, T, H, d))
    gate = _gate_of(g, 4)
    gshape = (B, T, H, d) if gate == KDA_GATE_CHANNEL else (B, T, H)
    _check_dev("g", g, dt, gshape)
    _check_dev("beta", beta, torch.float32, (B, T, H))
    n_seqs = 0
    if cu_seqlens is not None:
        _check_dev("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        if validate_cu:
            check_cu_seqlens(cu_seqlens.cpu(), T)
    S = n_seqs if n_seqs else B
    _check_dev("h0", h0, torch.float32, (S, H, d, d))
    _check_dev("dht", dht, torch.float32, (S, H, d, d))
    desc = make_desc(B, T, H, d, dt, n_seqs, chunk, g_floor)
    dx = ChunkDescEx(shape=desc, gate=gate)
    ws_bytes = _lib.backward_workspace_size(desc)
    out = dict(out or {})
    dev = q.device
    with _on_stream(stream, dev):
        for name, shape, odt in (("dq", (B, T, H, d), dt), ("dk", (B, T, H, d), dt), ("dv", (B, T, H, d), dt),
                                 ("dbeta", (B, T, H), torch.float32)):
            if out.get(name) is None:
                out[name] = torch.empty(shape, dtype=odt, device=dev)
        if gate != KDA_GATE_NONE and out.get("dg") is None:
            out["dg"] = torch.empty(gshape, dtype=dt, device=dev)
        if want_dh0 and out.get("dh0") is None:
            out["dh0"] = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    for name, shape, odt in (("dq", (B, T, H, d), dt), ("dk", (B, T, H, d), dt), ("dv", (B, T, H, d), dt),
                             ("dbeta", (B, T, H), torch.float32)):
        _check_dev(name, out[name], odt, shape)
    if gate == KDA_GATE_NONE:
        out["dg"] = None
    else:
        _check_dev("dg", out["dg"], dt, gshape)
    if want_dh0:
        _check_dev("dh0", out["dh0"], torch.float32, (S, H, d, d))
    else:
        out["dh0"] = None
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    aux = _aux_stream(dev) if overlap else None
    st = _lib.chunk_backward_raw(dx, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                 _ptr(cu_seqlens), _ptr(do), _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]),
                                 _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), stream, events,
                                 aux)
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_backward_timed" if events is not None else
                       "kda_chunk_backward_overlapped" if overlap else "kda_chunk_backward")
    return out


_KDA_FUNCTION = None


def _kda_function():
    """torch.autograd.Function over chunk_forward and chunk_backward (built
    on first use, so that importing the package does not import torch)."""
    global _KDA_FUNCTION
    if _KDA_FUNCTION is None:
        torch = _torch()

        class KDAChunk(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, g, beta, h0, cu_seqlens, g_floor):
                o, ht = chunk_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu_seqlens, g_floor=g_floor)
                ctx.save_for_backward(q, k, v, g, beta, h0, cu_seqlens)
                ctx.g_floor = g_floor
                return o, ht

            @staticmethod
            def backward(ctx, do, dht):
                q, k, v, g, beta, h0, cu_seqlens = ctx.saved_tensors
                out = chunk_backward(q, k, v, g, beta, do.contiguous(), h0=h0,
                                     dht=None if dht is None else dht.contiguous(), cu_seqlens=cu_seqlens,
                                     g_floor=ctx.g_floor, want_dh0=h0 is not None, validate_cu=False)
                return out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"], out["dh0"], None, None

        _KDA_FUNCTION = KDAChunk
    return _KDA_FUNCTION


def kda_chunk(q, k, v, g, beta, h0=None, cu_seqlens=None, g_floor: float = -0.125):
    """The chunked forward as a differentiable PyTorch operation: returns
    (o, ht) like chunk_forward, and its backward is chunk_backward (the
    gradients of q, k, v, g, beta and h0; o's gradient in o's dtype, ht's in
    fp32).  Arguments as chunk_forward."""
    return _kda_function().apply(q, k, v, g, beta, h0, cu_seqlens, g_floor)


def decode_step(q, k, v, g, beta, state, g_floor: float = -0.125, *, o=None, stream=None):
    """One decode step for N sequences; ``state`` [N, H, d, d] fp32 is updated
    in place.  q, k, v: [N, H, d]; g: [N, H, d] (KDA), [N, H] (Gated
    DeltaNet) or None (DeltaNet); beta: [N, H] fp32.  Returns o [N, H, d]."""
    torch = _torch()
    N, H, d = q.shape
    dt = q.dtype
    _check_dev("q", q, dt)
    for name, t in (("k", k), ("v", v)):
        _check_dev(name, t, dt, (N, H, d))
    gate = _gate_of(g, 3)
    _check_dev("g", g, dt, (N, H, d) if gate == KDA_GATE_CHANNEL else (N, H))
    _check_dev("beta", beta, torch.float32, (N, H))
    _check_dev("state", state, torch.float32, (N, H, d, d))
    if o is None:
        with _on_stream(stream, q.device):
            o = torch.empty((N, H, d), dtype=dt, device=q.device)
    _check_dev("o", o, dt, (N, H, d))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if gate == KDA_GATE_CHANNEL:
        st = _lib.decode_step_raw(N, H, d, d, _dtype_code(dt), g_floor, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(state), _ptr(o), stream)
    else:
        st = _lib.decode_step_gated_raw(N, H, d, d, _dtype_code(dt), gate, g_floor, _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(g), _ptr(beta), _ptr(state), _ptr(o), stream)
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step" if gate == KDA_GATE_CHANNEL else "kda_decode_step_gated")
    return o
