"""ctypes binding of ``libkda.so`` (the C ABI declared in include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Loading fails loudly when the library is missing;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY selects another build of the same library (the host-sanitizer
# build of the C front end, for instance); default: the in-tree build.
LIBRARY = os.environ.get("KDA_LIBRARY") or os.path.join(HERE, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE_TOO_SMALL = 3
KDA_ERR_HIP = 4
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
KDA_GATE_CHANNEL = 0   # g [.., H, d_k]: KDA
KDA_GATE_HEAD = 1      # g [.., H]: Gated DeltaNet
KDA_GATE_NONE = 2      # no g: DeltaNet

# Every symbol include/kda.h declares.
EXPORTS = ("kda_status_string", "kda_version", "kda_chunk_forward_workspace_size",
           "kda_chunk_forward", "kda_chunk_forward_gated", "kda_chunk_forward_timed",
           "kda_chunk_forward_states_count", "kda_chunk_forward_states", "kda_chunk_forward_mx",
           "kda_chunk_backward_workspace_size", "kda_chunk_backward", "kda_chunk_backward_overlapped",
           "kda_chunk_backward_timed", "kda_decode_step", "kda_decode_step_gated",
           "kda_chunk_forward_noalloc")

# Launches of one kda_chunk_forward call, in stream order (kda_chunk_forward_timed):
# the map sweep and the output sweep are the two instances of kda_chunk_sweep.
CHUNK_LAUNCHES = ("kda_chunk_sweep_map", "kda_seg_scan", "kda_chunk_sweep_out")
# Stages of one kda_chunk_backward call, in stream order (kda_chunk_backward_timed).
BWD_STAGES = ("forward_replay", "kda_bwd_chunk", "kda_bwd_state", "kda_bwd_local")


class KdaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class ChunkDesc(ctypes.Structure):
    """Mirror of kda_chunk_desc_t."""
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int), ("chunk", ctypes.c_int),
                ("n_seqs", ctypes.c_int), ("dtype", ctypes.c_int), ("g_floor", ctypes.c_float)]


class ChunkDescEx(ctypes.Structure):
    """Mirror of kda_chunk_desc_ex_t: the shape and the gate layout."""
    _fields_ = [("shape", ChunkDesc), ("gate", ctypes.c_int)]


_lib = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first with `python -m gated_delta_rule_105_amd.build` "
            "(the KDA path has no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    lib.kda_chunk_forward_workspace_size.argtypes = [ctypes.POINTER(ChunkDesc), ctypes.POINTER(sz)]
    lib.kda_chunk_forward_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_forward.argtypes = [ctypes.POINTER(ChunkDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.kda_chunk_forward.restype = ctypes.c_int
    lib.kda_chunk_forward_gated.argtypes = [ctypes.POINTER(ChunkDescEx), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]
    lib.kda_chunk_forward_gated.restype = ctypes.c_int
    lib.kda_chunk_forward_noalloc.argtypes = [ctypes.POINTER(ChunkDesc)] + [vp] * 10
    lib.kda_chunk_forward_noalloc.restype = ctypes.c_int
    lib.kda_chunk_forward_timed.argtypes = [ctypes.POINTER(ChunkDescEx), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp, ctypes.POINTER(vp)]
    lib.kda_chunk_forward_timed.restype = ctypes.c_int
    lib.kda_chunk_forward_states_count.argtypes = [ctypes.POINTER(ChunkDesc), ctypes.c_int, ctypes.POINTER(sz)]
    lib.kda_chunk_forward_states_count.restype = ctypes.c_int
    lib.kda_chunk_forward_states.argtypes = [ctypes.POINTER(ChunkDescEx), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             vp, ctypes.c_int, vp, sz, vp]
    lib.kda_chunk_forward_states.restype = ctypes.c_int
    lib.kda_chunk_forward_mx.argtypes = [ctypes.POINTER(ChunkDescEx), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp]
    lib.kda_chunk_forward_mx.restype = ctypes.c_int
    lib.kda_chunk_backward_workspace_size.argtypes = [ctypes.POINTER(ChunkDesc), ctypes.POINTER(sz)]
    lib.kda_chunk_backward_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_backward.argtypes = [ctypes.POINTER(ChunkDescEx)] + [vp] * 16 + [sz, vp]
    lib.kda_chunk_backward.restype = ctypes.c_int
    lib.kda_chunk_backward_overlapped.argtypes = [ctypes.POINTER(ChunkDescEx)] + [vp] * 16 + [sz, vp, vp, vp, vp]
    lib.kda_chunk_backward_overlapped.restype = ctypes.c_int
    lib.kda_chunk_backward_timed.argtypes = [ctypes.POINTER(ChunkDescEx)] + [vp] * 16 + [sz, vp,
                                                                                      ctypes.POINTER(vp)]
    lib.kda_chunk_backward_timed.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step_gated.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                          vp]
    lib.kda_decode_step_gated.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(int(status)).decode()


def version() -> int:
    return int(load().kda_version())


def workspace_size(desc: ChunkDesc) -> int:
    out = ctypes.c_size_t(0)
    st = load().kda_chunk_forward_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_forward_workspace_size")
    return int(out.value)


def chunk_forward_raw(desc: ChunkDesc, q, k, v, g, beta, h0, cu, o, ht, ws, ws_bytes, stream) -> int:
    """Call kda_chunk_forward with raw integer addresses; returns the status."""
    return int(load().kda_chunk_forward(ctypes.byref(desc), q, k, v, g, beta, h0, cu, o, ht, ws,
                                        ctypes.c_size_t(ws_bytes), stream))


def chunk_forward_gated_raw(dx: ChunkDescEx, q, k, v, g, beta, h0, cu, o, ht, ws, ws_bytes, stream) -> int:
    """Call kda_chunk_forward_gated with raw integer addresses; returns the status."""
    return int(load().kda_chunk_forward_gated(ctypes.byref(dx), q, k, v, g, beta, h0, cu, o, ht, ws,
                                              ctypes.c_size_t(ws_bytes), stream))


def chunk_forward_noalloc_raw(desc: ChunkDesc, q, k, v, g, beta, h0, cu, o, ht, stream) -> int:
    """Call kda_chunk_forward_noalloc with raw integer addresses; returns the status."""
    return int(load().kda_chunk_forward_noalloc(ctypes.byref(desc), q, k, v, g, beta, h0, cu, o, ht, stream))


def chunk_forward_timed_raw(dx: ChunkDescEx, q, k, v, g, beta, h0, cu, o, ht, ws, ws_bytes, stream,
                            events) -> int:
    """Call kda_chunk_forward_timed; `events` are len(CHUNK_LAUNCHES) + 1 raw hipEvent_t handles."""
    arr = (ctypes.c_void_p * (len(CHUNK_LAUNCHES) + 1))(*events)
    return int(load().kda_chunk_forward_timed(ctypes.byref(dx), q, k, v, g, beta, h0, cu, o, ht, ws,
                                              ctypes.c_size_t(ws_bytes), stream, arr))


def states_count(desc: ChunkDesc, states_every: int) -> int:
    out = ctypes.c_size_t(0)
    st = load().kda_chunk_forward_states_count(ctypes.byref(desc), int(states_every), ctypes.byref(out))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_forward_states_count")
    return int(out.value)


def chunk_forward_states_raw(dx: ChunkDescEx, q, k, v, g, beta, h0, cu, o, ht, states, states_every, ws,
                             ws_bytes, stream) -> int:
    """Call kda_chunk_forward_states with raw integer addresses; returns the status."""
    return int(load().kda_chunk_forward_states(ctypes.byref(dx), q, k, v, g, beta, h0, cu, o, ht, states,
                                               int(states_every), ws, ctypes.c_size_t(ws_bytes), stream))


def chunk_forward_mx_raw(dx: ChunkDescEx, q, qs, k, ks, v, vs, g, beta, h0, cu, o, ht, ws, ws_bytes, stream) -> int:
    """Call kda_chunk_forward_mx with raw integer addresses; returns the status."""
    return int(load().kda_chunk_forward_mx(ctypes.byref(dx), q, qs, k, ks, v, vs, g, beta, h0, cu, o, ht, ws,
                                           ctypes.c_size_t(ws_bytes), stream))


def backward_workspace_size(desc: ChunkDesc) -> int:
    out = ctypes.c_size_t(0)
    st = load().kda_chunk_backward_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_backward_workspace_size")
    return int(out.value)


def chunk_backward_raw(dx: ChunkDescEx, q, k, v, g, beta, h0, cu, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws,
                       ws_bytes, stream, events=None, aux=None) -> int:
    """Call kda_chunk_backward; its timed twin when `events` (len(BWD_STAGES)
    + 1 raw hipEvent_t handles) is given; kda_chunk_backward_overlapped when
    `aux` (raw second stream, fork event, join event) is given.  Returns the
    status."""
    args = (ctypes.byref(dx), q, k, v, g, beta, h0, cu, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws,
            ctypes.c_size_t(ws_bytes), stream)
    if aux is not None:
        if events is not None:
            raise ValueError("a call is either timed or overlapped")
        return int(load().kda_chunk_backward_overlapped(*args, *aux))
    if events is None:
        return int(load().kda_chunk_backward(*args))
    arr = (ctypes.c_void_p * (len(BWD_STAGES) + 1))(*events)
    return int(load().kda_chunk_backward_timed(*args, arr))


def decode_step_raw(N, H, d_k, d_v, dtype, g_floor, q, k, v, g, beta, state, o, stream) -> int:
    """Call kda_decode_step with raw integer addresses; returns the status."""
    return int(load().kda_decode_step(N, H, d_k, d_v, dtype, ctypes.c_float(g_floor), q, k, v, g, beta, state,
                                      o, stream))


def decode_step_gated_raw(N, H, d_k, d_v, dtype, gate, g_floor, q, k, v, g, beta, state, o, stream) -> int:
    """Call kda_decode_step_gated with raw integer addresses; returns the status."""
    return int(load().kda_decode_step_gated(N, H, d_k, d_v, dtype, gate, ctypes.c_float(g_floor), q, k, v, g,
                                            beta, state, o, stream))
