// C-ABI front end of the KDA library: argument validation and dispatch.
//
// Plain C++: every argument error is reported before any launch (and can be
// exercised on a machine without a GPU); the only HIP calls made here are the
// compute-unit query behind the forward's cut into segments
// (kda::device_compute_units) and, for kda_chunk_forward_noalloc, the lookup
// of the device scratch's address (kda::scratch_buffer), after every
// argument check.  The entry points and their contracts are
// declared in include/kda.h.
#include "kda.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "kda_launch.h"

static_assert(KDA_NOALLOC_SCRATCH_BYTES == kda::kScratchBytes, "scratch size of the header and the library agree");

static_assert(KDA_GATE_CHANNEL == kda::kGateChannel && KDA_GATE_HEAD == kda::kGateHead &&
                  KDA_GATE_NONE == kda::kGateNone,
              "gate codes of the C ABI and the kernels agree");

namespace {

constexpr size_t kAlign = 16;
constexpr size_t kWsAlign = 256;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Multiply non-negative sizes, flagging overflow of size_t.
bool mul(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

// Enum-typed arguments as their int representation: a C caller may store any
// int in them, and loading a value outside the enumerators through the enum
// type is undefined in C++, so they are only ever read this way.
template <typename E>
int as_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}
int dtype_of(const kda_chunk_desc_t* d) { return as_int(d->dtype); }

size_t elem_size(int t) { return t == KDA_DTYPE_BF16 ? 2 : 4; }

struct Sizes {
  size_t tokens;      // B * T
  size_t n_states;    // sequences
  size_t x_bytes;     // one of q, k, v, o (and g with channel gates)
  size_t g_bytes;     // g for the descriptor's gate (0 without one)
  size_t beta_bytes;
  size_t state_bytes; // h0 or ht
  int n_cu;           // compute units the plan was made for
  kda::SegPlan plan;  // segments and workspace
};

bool valid_gate(int gate) { return gate == KDA_GATE_CHANNEL || gate == KDA_GATE_HEAD || gate == KDA_GATE_NONE; }

// max_ws: the largest workspace the call can have (the plan keeps to it).
int check_desc(const kda_chunk_desc_t* d, int gate, Sizes* s, size_t max_ws = SIZE_MAX) {
  if (!d) return KDA_ERR_INVALID_ARGUMENT;
  if (d->B < 1 || d->T < 0 || d->H < 1 || d->d_k < 1 || d->d_v < 1 || d->chunk < 1 || d->n_seqs < 0)
    return KDA_ERR_INVALID_ARGUMENT;
  if (dtype_of(d) != KDA_DTYPE_F32 && dtype_of(d) != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (!valid_gate(gate)) return KDA_ERR_INVALID_ARGUMENT;
  if (d->n_seqs > 0 && d->B != 1) return KDA_ERR_INVALID_ARGUMENT;
  if (!(d->g_floor >= -1.0f && d->g_floor < 0.0f)) return KDA_ERR_INVALID_ARGUMENT;  // NaN fails too
  if ((double)d->chunk * -(double)d->g_floor > 16.0) return KDA_ERR_INVALID_ARGUMENT;
  if (d->d_k != d->d_v) return KDA_ERR_UNSUPPORTED;
  if (d->d_k != 64 && d->d_k != 128) return KDA_ERR_UNSUPPORTED;
  if (d->chunk != kda::kChunk) return KDA_ERR_UNSUPPORTED;
  if (dtype_of(d) == KDA_DTYPE_F32 && d->d_k != 64) return KDA_ERR_UNSUPPORTED;  // fp32 tiles fit LDS at d = 64

  const size_t B = (size_t)d->B, T = (size_t)d->T, H = (size_t)d->H, D = (size_t)d->d_k;
  s->n_states = d->n_seqs > 0 ? (size_t)d->n_seqs : B;
  if (!mul(B, T, &s->tokens)) return KDA_ERR_INVALID_ARGUMENT;
  size_t th, x;
  if (!mul(s->tokens, H, &th) || !mul(th, D, &x) || !mul(x, elem_size(dtype_of(d)), &s->x_bytes))
    return KDA_ERR_INVALID_ARGUMENT;
  if (!mul(th, 4, &s->beta_bytes)) return KDA_ERR_INVALID_ARGUMENT;
  s->g_bytes = gate == KDA_GATE_CHANNEL ? s->x_bytes : gate == KDA_GATE_HEAD ? th * elem_size(dtype_of(d)) : 0;
  size_t sh, sd;
  if (!mul(s->n_states, H, &sh) || !mul(sh, D * D, &sd) || !mul(sd, 4, &s->state_bytes))
    return KDA_ERR_INVALID_ARGUMENT;
  if (s->tokens > (size_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const int rows = d->n_seqs > 0 ? d->n_seqs : d->B;
  s->n_cu = kda::device_compute_units();
  if (!kda::plan_segments(d->d_k, (int)elem_size(dtype_of(d)), rows, (int64_t)d->T, d->H, d->n_seqs > 0, s->n_cu,
                          &s->plan, max_ws)) {
    // no cut fits max_ws (but one exists), or the sizes overflow
    kda::SegPlan any;
    const bool fits_unbounded = max_ws != SIZE_MAX &&
                                kda::plan_segments(d->d_k, (int)elem_size(dtype_of(d)), rows, (int64_t)d->T, d->H,
                                                   d->n_seqs > 0, s->n_cu, &any);
    return fits_unbounded ? KDA_ERR_WORKSPACE_TOO_SMALL : KDA_ERR_UNSUPPORTED;
  }
  if (s->plan.n_seg_bound > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

// Slots of kda_chunk_forward_states (see include/kda.h); false for a bad
// states_every.
bool state_slots(const kda_chunk_desc_t* d, int every, size_t* slots) {
  if (every < 1) return false;
  const int64_t per = (int64_t)every * d->chunk;
  const int64_t each = (int64_t)d->T / per;
  *slots = (size_t)(d->n_seqs > 0 ? each : (int64_t)d->B * each);
  return true;
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    default: return "KDA_ERR_UNKNOWN";
  }
}

int kda_version(void) { return KDA_VERSION; }

int kda_chunk_forward_workspace_size(const kda_chunk_desc_t* d, size_t* bytes) {
  if (!bytes) return KDA_ERR_INVALID_ARGUMENT;
  Sizes s;
  const int st = check_desc(d, KDA_GATE_CHANNEL, &s);
  if (st != KDA_OK) return st;
  *bytes = s.plan.ws_bytes;
  return KDA_OK;
}

int kda_chunk_forward_states_count(const kda_chunk_desc_t* d, int states_every, size_t* count) {
  if (!count) return KDA_ERR_INVALID_ARGUMENT;
  Sizes s;
  const int st = check_desc(d, KDA_GATE_CHANNEL, &s);
  if (st != KDA_OK) return st;
  if (!state_slots(d, states_every, count)) return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

// mx: MXFP8 q, k, v (e4m3 bytes) with their scale bytes, or NULL.
struct MxIn {
  const uint8_t* qs;
  const uint8_t* ks;
  const uint8_t* vs;
};

// states: NULL (no state emission) or the kda_chunk_forward_states buffer,
// with every >= 1.  scratch_ws: the workspace is the library's fixed device
// scratch (workspace must be NULL), taken after every argument check.
static int chunk_forward(const kda_chunk_desc_t* d, int gate, const void* q, const void* k, const void* v,
                         const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens, void* o,
                         float* ht, float* states, int every, const MxIn* mx, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events, bool scratch_ws = false) {
  Sizes s;
  const int st = check_desc(d, gate, &s, scratch_ws ? kda::kScratchBytes : SIZE_MAX);
  if (st != KDA_OK) return st;
  const bool has_tokens = s.tokens > 0;
  // bytes of q, k, v (MXFP8: one byte per element) and of each scale tensor
  size_t qkv_bytes = s.x_bytes, sc_bytes = 0;
  if (mx) {
    if (dtype_of(d) != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;  // MXFP8 inputs feed the bf16 path
    qkv_bytes = s.x_bytes / 2;
    sc_bytes = qkv_bytes / 32;
    if (has_tokens && (!mx->qs || !mx->ks || !mx->vs)) return KDA_ERR_INVALID_ARGUMENT;
  }
  const bool gated = gate != KDA_GATE_NONE;
  if (!gated) g = nullptr;  // not read
  if (has_tokens && (!q || !k || !v || (gated && !g) || !beta || !o)) return KDA_ERR_INVALID_ARGUMENT;
  if ((d->n_seqs > 0) != (cu_seqlens != nullptr)) return KDA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, g, beta, h0, o, ht};
  for (const void* p : ptrs)
    if (p && !aligned(p, kAlign)) return KDA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARGUMENT;
  const size_t ws_need = s.plan.ws_bytes;
  if (!scratch_ws && ws_need > 0) {
    if (!workspace || !aligned(workspace, kWsAlign)) return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE_TOO_SMALL;
  }
  // every input (read only; they may overlap one another)
  const Range ins[] = {range(q, qkv_bytes),
                       range(k, qkv_bytes),
                       range(v, qkv_bytes),
                       range(g, s.g_bytes),
                       range(beta, s.beta_bytes),
                       range(h0, s.state_bytes),
                       range(mx ? mx->qs : nullptr, sc_bytes),
                       range(mx ? mx->ks : nullptr, sc_bytes),
                       range(mx ? mx->vs : nullptr, sc_bytes)};
  const Range ro = range(o, s.x_bytes), rh = range(ht, s.state_bytes), rw = range(workspace, ws_need);
  size_t states_bytes = 0;
  if (states) {
    size_t slots, per;
    if (!state_slots(d, every, &slots)) return KDA_ERR_INVALID_ARGUMENT;
    if (!mul((size_t)d->H * d->d_k, (size_t)d->d_v * 4, &per) || !mul(slots, per, &states_bytes))
      return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned(states, kAlign)) return KDA_ERR_INVALID_ARGUMENT;
  }
  const Range rs = range(states, states_bytes);
  for (const Range& r : ins) {
    if (has_tokens && overlap(ro, r)) return KDA_ERR_INVALID_ARGUMENT;
    if (&r != &ins[5] && overlap(rh, r)) return KDA_ERR_INVALID_ARGUMENT;  // ht may alias h0 exactly
    if (overlap(rw, r) || overlap(rs, r)) return KDA_ERR_INVALID_ARGUMENT;
  }
  if (h0 && h0 != ht && overlap(rh, range(h0, s.state_bytes))) return KDA_ERR_INVALID_ARGUMENT;
  if (overlap(rh, ro) || overlap(rw, ro) || overlap(rw, rh) || overlap(rs, ro) || overlap(rs, rh) ||
      overlap(rs, rw))
    return KDA_ERR_INVALID_ARGUMENT;
  if (!ht && s.tokens == 0 && !events) return KDA_OK;  // nothing to write (no full chunk: no states either)
  if (scratch_ws && ws_need > 0 && kda::scratch_buffer(&workspace) != 0) return KDA_ERR_HIP;
  const int rows = d->n_seqs > 0 ? d->n_seqs : d->B;
  const kda::ChunkInputs in{q, k, v, g, beta, mx ? mx->qs : nullptr, mx ? mx->ks : nullptr, mx ? mx->vs : nullptr};
  const int e = kda::launch_chunk_forward(dtype_of(d) == KDA_DTYPE_BF16, d->d_k, rows, d->T, d->H, s.plan,
                                          d->g_floor, gate, in, h0, cu_seqlens, o, ht,
                                          states_bytes > 0 ? states : nullptr, every, workspace, stream,
                                          events);
  return e == 0 ? KDA_OK : KDA_ERR_HIP;
}

// the extended descriptor: its shape, and its gate (NULL: invalid)
static const kda_chunk_desc_t* shape_of(const kda_chunk_desc_ex_t* d) { return d ? &d->shape : nullptr; }
static int gate_of(const kda_chunk_desc_ex_t* d) { return d ? as_int(d->gate) : KDA_GATE_CHANNEL; }

int kda_chunk_forward(const kda_chunk_desc_t* d, const void* q, const void* k, const void* v,
                      const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                      void* o, float* ht, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_forward(d, KDA_GATE_CHANNEL, q, k, v, g, beta, h0, cu_seqlens, o, ht, nullptr, 0, nullptr, workspace,
                       workspace_bytes, stream, nullptr);
}

int kda_chunk_forward_gated(const kda_chunk_desc_ex_t* d, const void* q, const void* k, const void* v,
                            const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                            void* o, float* ht, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_forward(shape_of(d), gate_of(d), q, k, v, g, beta, h0, cu_seqlens, o, ht, nullptr, 0, nullptr,
                       workspace, workspace_bytes, stream, nullptr);
}

int kda_chunk_forward_noalloc(const kda_chunk_desc_t* d, const void* q, const void* k, const void* v,
                              const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                              void* o, float* ht, void* stream) {
  return chunk_forward(d, KDA_GATE_CHANNEL, q, k, v, g, beta, h0, cu_seqlens, o, ht, nullptr, 0, nullptr, nullptr,
                       0, stream, nullptr, true);
}

int kda_chunk_forward_timed(const kda_chunk_desc_ex_t* d, const void* q, const void* k, const void* v,
                            const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                            void* o, float* ht, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events) {
  if (!events) return KDA_ERR_INVALID_ARGUMENT;
  return chunk_forward(shape_of(d), gate_of(d), q, k, v, g, beta, h0, cu_seqlens, o, ht, nullptr, 0, nullptr,
                       workspace, workspace_bytes, stream, events);
}

int kda_chunk_forward_states(const kda_chunk_desc_ex_t* d, const void* q, const void* k, const void* v,
                             const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                             void* o, float* ht, float* states, int states_every, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Sizes s;
  const int st = check_desc(shape_of(d), gate_of(d), &s);  // before state_slots divides by the chunk
  if (st != KDA_OK) return st;
  size_t slots;
  if (!state_slots(shape_of(d), states_every, &slots)) return KDA_ERR_INVALID_ARGUMENT;
  if (!states && slots > 0) return KDA_ERR_INVALID_ARGUMENT;
  return chunk_forward(shape_of(d), gate_of(d), q, k, v, g, beta, h0, cu_seqlens, o, ht, states, states_every,
                       nullptr, workspace, workspace_bytes, stream, nullptr);
}

int kda_chunk_forward_mx(const kda_chunk_desc_ex_t* d, const void* q, const uint8_t* q_scale, const void* k,
                         const uint8_t* k_scale, const void* v, const uint8_t* v_scale, const void* g,
                         const float* beta, const float* h0, const int32_t* cu_seqlens, void* o, float* ht,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const MxIn mx{q_scale, k_scale, v_scale};
  return chunk_forward(shape_of(d), gate_of(d), q, k, v, g, beta, h0, cu_seqlens, o, ht, nullptr, 0, &mx,
                       workspace, workspace_bytes, stream, nullptr);
}

// ---- backward ------------------------------------------------------------

namespace {

// budget: SIZE_MAX for the default plan (the size query), else the
// workspace the caller gave (the widest window that fits).
bool plan_bwd(const kda_chunk_desc_t* d, const Sizes& s, size_t budget, kda::BwdPlan* bp) {
  size_t chunk_states;
  if (!state_slots(d, 1, &chunk_states)) return false;
  const int rows = d->n_seqs > 0 ? d->n_seqs : d->B;
  return kda::plan_backward(d->d_k, (int)elem_size(dtype_of(d)), rows, (int64_t)d->T, d->H, d->n_seqs > 0, s.n_cu,
                            s.tokens, chunk_states, budget, bp);
}

int chunk_backward(const kda_chunk_desc_ex_t* dx, const void* q, const void* k, const void* v, const void* g,
                   const float* beta, const float* h0, const int32_t* cu_seqlens, const void* dout, const float* dht,
                   void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0, void* workspace,
                   size_t workspace_bytes, void* stream, void* const* events,
                   const kda::AuxStream* aux = nullptr) {
  const kda_chunk_desc_t* d = shape_of(dx);
  const int gate = gate_of(dx);
  Sizes s;
  const int st = check_desc(d, gate, &s);
  if (st != KDA_OK) return st;
  kda::BwdPlan bp;
  if (!plan_bwd(d, s, SIZE_MAX, &bp)) return KDA_ERR_UNSUPPORTED;
  const bool has_tokens = s.tokens > 0;
  const bool gated = gate != KDA_GATE_NONE;
  if (!gated) {
    g = nullptr;  // neither read nor written
    dg = nullptr;
  }
  if (has_tokens && (!q || !k || !v || (gated && (!g || !dg)) || !beta || !dout || !dq || !dk || !dv || !dbeta))
    return KDA_ERR_INVALID_ARGUMENT;
  if ((d->n_seqs > 0) != (cu_seqlens != nullptr)) return KDA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, g, beta, h0, dout, dht, dq, dk, dv, dg, dbeta, dh0};
  for (const void* p : ptrs)
    if (p && !aligned(p, kAlign)) return KDA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARGUMENT;
  if (!workspace || !aligned(workspace, kWsAlign)) return KDA_ERR_INVALID_ARGUMENT;
  if (!plan_bwd(d, s, workspace_bytes, &bp)) return KDA_ERR_WORKSPACE_TOO_SMALL;
  // inputs may overlap one another; outputs overlap nothing
  const Range ins[] = {range(q, s.x_bytes),   range(k, s.x_bytes),    range(v, s.x_bytes),
                       range(g, s.g_bytes),   range(beta, s.beta_bytes), range(h0, s.state_bytes),
                       range(dout, s.x_bytes), range(dht, s.state_bytes)};
  const Range outs[] = {range(dq, s.x_bytes),      range(dk, s.x_bytes),         range(dv, s.x_bytes),
                        range(dg, s.g_bytes),      range(dbeta, s.beta_bytes),   range(dh0, s.state_bytes),
                        range(workspace, bp.ws_bytes)};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return KDA_ERR_INVALID_ARGUMENT;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j])) return KDA_ERR_INVALID_ARGUMENT;
  }
  const int rows = d->n_seqs > 0 ? d->n_seqs : d->B;
  const kda::ChunkInputs in{q, k, v, g, beta, nullptr, nullptr, nullptr};
  const int e = kda::launch_chunk_backward(dtype_of(d) == KDA_DTYPE_BF16, d->d_k, rows, d->T, d->H, bp, d->g_floor,
                                           gate, in, h0, cu_seqlens, dout, dht, dq, dk, dv, dg, dbeta, dh0,
                                           workspace, stream, events, aux);
  return e == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

int kda_chunk_backward_workspace_size(const kda_chunk_desc_t* d, size_t* bytes) {
  if (!bytes) return KDA_ERR_INVALID_ARGUMENT;
  Sizes s;
  const int st = check_desc(d, KDA_GATE_CHANNEL, &s);
  if (st != KDA_OK) return st;
  kda::BwdPlan bp;
  if (!plan_bwd(d, s, SIZE_MAX, &bp)) return KDA_ERR_UNSUPPORTED;
  *bytes = bp.ws_bytes;
  return KDA_OK;
}

int kda_chunk_backward(const kda_chunk_desc_ex_t* d, const void* q, const void* k, const void* v, const void* g,
                       const float* beta, const float* h0, const int32_t* cu_seqlens, const void* dout,
                       const float* dht, void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_backward(d, q, k, v, g, beta, h0, cu_seqlens, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace,
                        workspace_bytes, stream, nullptr);
}

int kda_chunk_backward_overlapped(const kda_chunk_desc_ex_t* d, const void* q, const void* k, const void* v,
                                  const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                                  const void* dout, const float* dht, void* dq, void* dk, void* dv, void* dg,
                                  float* dbeta, float* dh0, void* workspace, size_t workspace_bytes, void* stream,
                                  void* aux_stream, void* fork_event, void* join_event) {
  if (!fork_event || !join_event || fork_event == join_event) return KDA_ERR_INVALID_ARGUMENT;
  const kda::AuxStream aux{aux_stream, fork_event, join_event};
  return chunk_backward(d, q, k, v, g, beta, h0, cu_seqlens, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace,
                        workspace_bytes, stream, nullptr, &aux);
}

int kda_chunk_backward_timed(const kda_chunk_desc_ex_t* d, const void* q, const void* k, const void* v,
                             const void* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                             const void* dout, const float* dht, void* dq, void* dk, void* dv, void* dg,
                             float* dbeta, float* dh0, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events) {
  if (!events) return KDA_ERR_INVALID_ARGUMENT;
  return chunk_backward(d, q, k, v, g, beta, h0, cu_seqlens, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace,
                        workspace_bytes, stream, events);
}

int kda_decode_step(int N, int H, int d_k, int d_v, kda_dtype_t dtype, float g_floor, const void* q,
                    const void* k, const void* v, const void* g, const float* beta, float* state, void* o,
                    void* stream) {
  return kda_decode_step_gated(N, H, d_k, d_v, dtype, KDA_GATE_CHANNEL, g_floor, q, k, v, g, beta, state, o,
                               stream);
}

int kda_decode_step_gated(int N, int H, int d_k, int d_v, kda_dtype_t dtype, kda_gate_t gate, float g_floor,
                          const void* q, const void* k, const void* v, const void* g, const float* beta,
                          float* state, void* o, void* stream) {
  const int dt = as_int(dtype), gt = as_int(gate);
  if (N < 0 || H < 1 || d_k < 1 || d_v < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (dt != KDA_DTYPE_F32 && dt != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (!valid_gate(gt)) return KDA_ERR_INVALID_ARGUMENT;
  if (!(g_floor >= -1.0f && g_floor < 0.0f)) return KDA_ERR_INVALID_ARGUMENT;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  const bool gated = gt != KDA_GATE_NONE;
  if (!gated) g = nullptr;  // not read
  if (!q || !k || !v || (gated && !g) || !beta || !state || !o) return KDA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, g, beta, state, o};
  for (const void* p : ptrs)
    if (p && !aligned(p, kAlign)) return KDA_ERR_INVALID_ARGUMENT;
  size_t nh, x, xb, sb, bb;
  if (!mul((size_t)N, (size_t)H, &nh) || !mul(nh, (size_t)d_k, &x) || !mul(x, elem_size(dt), &xb) ||
      !mul(x, (size_t)d_k * 4, &sb) || !mul(nh, 4, &bb))
    return KDA_ERR_INVALID_ARGUMENT;
  if (nh > (size_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const size_t gb = gt == KDA_GATE_CHANNEL ? xb : gt == KDA_GATE_HEAD ? nh * elem_size(dt) : 0;
  const Range rs = range(state, sb), ro = range(o, xb);
  const Range ins[] = {range(q, xb), range(k, xb), range(v, xb), range(g, gb), range(beta, bb)};
  for (const Range& r : ins)
    if (overlap(rs, r) || overlap(ro, r)) return KDA_ERR_INVALID_ARGUMENT;
  if (overlap(rs, ro)) return KDA_ERR_INVALID_ARGUMENT;
  const int e = kda::launch_decode_step(dt == KDA_DTYPE_BF16, d_k, N, H, g_floor, gt, q, k, v, g,
                                        beta, state, o, stream);
  return e == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
