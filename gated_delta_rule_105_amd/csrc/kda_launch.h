// Internal interface between the C-ABI front end (kda_api.cpp, plain C++)
// and the HIP translation units that hold the kernels.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk

// Gate layouts (the values of kda_gate_t): g per key channel, per head, none.
constexpr int kGateChannel = 0, kGateHead = 1, kGateNone = 2;

// How a chunked forward is cut for the GPU.  Every sequence is cut into
// segments of `seg_chunks` chunks.  A chunk maps the state entering it
// affinely, and so does a segment: S_out = M S_in + B.
//  - With `maps`, a map sweep composes every segment's (M, B) from a zero
//    state, a scan chains them into each segment's incoming state S_in, and
//    the output sweep runs every segment from its S_in.  One record per
//    (segment, head) holds three d x d fp32 matrices: B, M and S_in.
//  - Without, every sequence is one segment: the output sweep alone, from h0.
// Both sweeps recompute the chunk-local algebra from the inputs; nothing per
// chunk goes through memory.
// Workspace: the segment records (with maps), then for a packed batch the
// per-sequence prefix sums of segments and of prefix-cache state slots.
struct SegPlan {
  int seg_chunks;        // chunks per segment (the longest sequence's chunks without maps)
  bool maps;             // map sweep + scan before the output sweep
  int64_t n_seg_bound;   // upper bound of segments over all sequences (grid of both sweeps)
  size_t rec_bytes;      // bytes of one (segment, head) record
  size_t seq_off;        // byte offset of the per-sequence prefix sums (packed batches)
  size_t ws_bytes;       // whole workspace
};

// Upper bound of groups of g chunks over the sequences: n_rows rows of T
// tokens, or (packed) n_rows sequences sharing T tokens.
inline int64_t group_bound(int64_t T, int n_rows, bool packed, int64_t g) {
  const int64_t chunks = (T + kChunk - 1) / kChunk;
  if (T == 0) return 0;
  if (packed) return (chunks + n_rows + g - 1) / g + n_rows;
  return (int64_t)n_rows * ((chunks + g - 1) / g);
}

// Compute units of the current device (0 when no device answers): the cost
// model below cuts sequences into segments for it.
int device_compute_units();

// Costs measured on MI355X at d = 128 (per-workgroup timestamps of the
// sweeps, B = 1, H = 16, T = 4096 and 65,536): per chunk of a sweep
// workgroup (one per CU; the map sweep 5.8 to 7.1 us, the output sweep 6.9
// to 8.4 us, inputs from cache or from HBM), per scan step, per launch
// (dispatch and drain beyond the workgroups' span) and per sweep workgroup
// outside its chunk loop.  The chunk and step times are scaled by
// (d / 128)^2 for d = 64.
constexpr double kMapChunkUs = 6.4, kOutChunkUs = 7.6, kScanStepUs = 1.13, kLaunchUs = 4.0, kSweepWgUs = 3.0;

// Chooses the cut from a cost model of the launches.  Either every sequence
// is one segment (the output sweep alone; one workgroup per (sequence, head)
// walks the sequence), or segments of L chunks (map sweep, scan of
// segments - 1 steps, output sweep; one workgroup per (segment, head) in
// both sweeps).  Host-only, deterministic in its arguments.  `packed`:
// n_rows sequences share T tokens (lengths unknown on the host; the mean
// length is used), else n_rows rows of T tokens each.  n_cu: compute units
// of the device.  max_ws: cuts whose workspace exceeds it are not taken.
// Returns false on overflow, or when no cut fits max_ws.
inline bool plan_segments(int d, int esz, int n_rows, int64_t T, int H, bool packed, int n_cu, SegPlan* p,
                          size_t max_ws = SIZE_MAX) {
  (void)esz;
  const double sc = (double)d * d / (128.0 * 128.0);
  const double t_map = kMapChunkUs * sc, t_out = kOutChunkUs * sc, t_scan = kScanStepUs * sc;
  const int64_t cus = n_cu > 0 ? n_cu : 256;
  const int64_t chunks_total = (T + kChunk - 1) / kChunk;
  const int rows = n_rows > 0 ? n_rows : 1;
  int64_t per_seq = packed ? (chunks_total + rows - 1) / rows : chunks_total;
  if (per_seq < 1) per_seq = 1;
  const int64_t pairs = (int64_t)n_rows * H;
  auto rounds = [&](int64_t wg) { return (double)((wg + cus - 1) / cus); };
  const size_t rec_bytes = (size_t)3 * d * d * sizeof(float);
  const size_t seq_bytes = packed ? (size_t)2 * ((size_t)n_rows + 1) * sizeof(int64_t) : 0;
  // workspace of a cut into segments of L chunks (0: one segment per sequence)
  auto ws_of = [&](int64_t L) -> double {
    const double recs = L > 0 ? (double)group_bound(T, n_rows, packed, L) * (double)H * (double)rec_bytes : 0.0;
    return ceil(recs / 256.0) * 256.0 + (double)seq_bytes;
  };
  if (ws_of(0) > (double)max_ws) return false;
  // one segment per sequence: the output sweep alone
  double best = rounds(pairs) * ((double)per_seq * t_out + kSweepWgUs) + kLaunchUs;
  int best_l = 0;
  for (int64_t L = 1; L < per_seq; L *= 2) {
    const int64_t segs = (per_seq + L - 1) / L;
    const double t = rounds(pairs * segs) * ((double)L * (t_map + t_out) + 2.0 * kSweepWgUs) +
                     (double)(segs - 1) * t_scan + 3.0 * kLaunchUs;
    if (t < best && ws_of(L) <= (double)max_ws) {
      best = t;
      best_l = (int)L;
    }
  }
  p->maps = best_l > 0;
  // without maps a packed batch needs its longest sequence to fit one segment
  p->seg_chunks = p->maps ? best_l : (int)(packed ? (chunks_total > 0 ? chunks_total : 1) : per_seq);
  p->n_seg_bound = group_bound(T, n_rows, packed, p->seg_chunks);
  p->rec_bytes = rec_bytes;
  const int64_t hh = H > 0 ? H : 1;
  if (p->n_seg_bound > ((int64_t)1 << 36) / hh || chunks_total > ((int64_t)1 << 36) / hh) return false;
  const size_t recs = p->maps ? (size_t)p->n_seg_bound * (size_t)H * p->rec_bytes : 0;
  p->seq_off = (recs + 255) / 256 * 256;
  p->ws_bytes = packed ? p->seq_off + seq_bytes : recs;
  return p->ws_bytes <= max_ws;
}

// Fixed device scratch of the allocation-free forward
// (kda_chunk_forward_noalloc): one array per device, in the library's code
// object, that every such call on the device shares.
constexpr size_t kScratchBytes = (size_t)64 << 20;

// Device address of the current device's scratch array (looked up once per
// device, then kept).  Returns a hipError_t.
int scratch_buffer(void** ptr);

// The inputs of one chunked forward.  q, k, v are in the operand type, or
// with MXFP8 inputs (qs != null) e4m3 bytes whose blocks of 32 channels
// share the power-of-two scale 2^(s - 127) of the scale byte s in qs, ks, vs
// ([.., H, d / 32]).  g: per the gate; null without one.
struct ChunkInputs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const float* beta;
  const uint8_t* qs;
  const uint8_t* ks;
  const uint8_t* vs;
};

// Launches of one chunked forward, in stream order.
constexpr int kLaunches = 3;  // map sweep, segment scan, output sweep

// Enqueue the chunked forward.  All arguments were validated by the caller.
// n_rows: number of sequences (n_seqs, or B when cu == nullptr).  gate: a
// kda_gate_t (g is null for KDA_GATE_NONE).  states:
// null, or the state slots of kda_chunk_forward_states, one every `every`
// chunks.  events: null, or kLaunches + 1 hipEvent_t handles (entries may be
// null) recorded on the stream before each launch and after the last.
// Returns a hipError_t.
int launch_chunk_forward(int is_bf16, int d, int n_rows, int T, int H, const SegPlan& plan,
                         float g_floor, int gate, const ChunkInputs& in, const float* h0,
                         const int32_t* cu, void* o, float* ht, float* states, int every,
                         void* ws, void* stream, void* const* events);

// ---- backward pass ------------------------------------------------------
// Floats of one (chunk, head) record of the backward pass at width d: five
// [64][d] blocks (Qt, Kt, Kh, Wk, Wv), three [64][64] (P, T, Abar), gamma [d]
// and beta [64], and at d = 64 three more [64][d] (copies of V and dO, and
// Gamma); and of one (chunk, head) scratch area of its local gradient
// kernel: five [64][d] blocks, two [64][64] and one [d] at d = 64, none at
// d = 128 (that kernel keeps its intermediates on chip).
constexpr size_t bwd_rec_floats(int d) {
  return (size_t)(d == 128 ? 5 : 8) * kChunk * d + (size_t)3 * kChunk * kChunk + (size_t)d + kChunk;
}
constexpr size_t bwd_scr_floats(int d) {
  return d == 128 ? 0 : (size_t)5 * kChunk * d + (size_t)2 * kChunk * kChunk + (size_t)d;
}

// Workspace of one backward call (byte offsets, each 256-byte aligned): the
// forward replay's own workspace first, then its o (discarded), its final
// states, the state after every full chunk, one zero state; then the area
// of the chunk records, the scratch areas and the end-state gradient of every
// chunk in flight, the per-sequence chunk and state-slot offsets of a packed
// batch, and with windows two carry states per (sequence, head).
//
// Windows: with width W > 0 the chunks are processed in windows of W chunk
// indices, [w W, (w + 1) W) of every sequence, from the last window to the
// first; chunk m of sequence n has area slot n W + (m - w W), so the area
// holds n_rows W slots, reused by every window.  The state gradient at a
// window's lower edge passes to the next window through a carry state.  With
// W = 0 the area has a slot for every chunk of the call (slots count the
// chunks of all sequences in order) and there is one window.
struct BwdPlan {
  SegPlan fwd;
  int64_t n_slots;  // upper bound of chunks over all sequences
  int64_t width;    // chunks per window, 0: one window
  int64_t span;     // upper bound of the chunks of one sequence
  int64_t n_area;   // slots of the record, scratch and gradient areas
  size_t o_off, ht_off, states_off, zero_off, rec_off, scr_off, dh_off, seq_off, carry_off, ws_bytes;
  size_t rec_floats, scr_floats;
  int64_t windows() const { return width > 0 ? (span + width - 1) / width : 1; }
};

// Chunk-heads of the area above which the default plan cuts sequences into
// windows: about 2.1 GiB of records and gradients at d = 128.
constexpr int64_t kBwdAreaChunkHeads = 8192;
// Narrowest window of the default plan.
constexpr int64_t kBwdMinWindow = 64;

// n_states: sequences; chunk_states: full chunks over all sequences (an
// upper bound for a packed batch).  budget: the workspace bytes available;
// SIZE_MAX gives the default plan (one window unless the area would pass
// kBwdAreaChunkHeads), otherwise the widest window that fits (one window
// when the whole area fits).  Returns false on overflow or when not even
// one-chunk windows fit the budget.
inline bool plan_backward(int d, int esz, int n_rows, int64_t T, int H, bool packed, int n_cu, size_t tokens,
                          size_t chunk_states, size_t budget, BwdPlan* p) {
  if (!plan_segments(d, esz, n_rows, T, H, packed, n_cu, &p->fwd)) return false;
  const size_t a = 256, hh = (size_t)H, dd = (size_t)d * d * sizeof(float);
  auto up = [&](size_t x) { return (x + a - 1) / a * a; };
  const int64_t chunks_total = (T + kChunk - 1) / kChunk;
  p->n_slots = T == 0 ? 0 : (packed ? chunks_total + n_rows : (int64_t)n_rows * chunks_total);
  p->span = chunks_total;  // a sequence of a packed batch has at most all of them
  p->rec_floats = bwd_rec_floats(d);
  p->scr_floats = bwd_scr_floats(d);
  const double per_slot = hh * ((p->rec_floats + p->scr_floats) * 4.0 + (double)dd);
  const double total = (double)p->fwd.ws_bytes + (double)tokens * hh * d * esz +
                       ((double)n_rows + (double)chunk_states + 1.0) * hh * dd + (double)p->n_slots * per_slot +
                       2.0 * (double)n_rows * hh * dd;
  if (total > 1.0e15) return false;
  auto layout = [&](int64_t width) {
    p->width = width;
    p->n_area = width > 0 ? (int64_t)n_rows * width : p->n_slots;
    size_t off = up(p->fwd.ws_bytes);
    p->o_off = off;
    off = up(off + tokens * hh * (size_t)d * esz);
    p->ht_off = off;
    off = up(off + (size_t)n_rows * hh * dd);
    p->states_off = off;
    off = up(off + chunk_states * hh * dd);
    p->zero_off = off;
    off = up(off + dd);
    p->rec_off = off;
    off = up(off + (size_t)p->n_area * hh * p->rec_floats * 4);
    p->scr_off = off;
    off = up(off + (size_t)p->n_area * hh * p->scr_floats * 4);
    p->dh_off = off;
    off = up(off + (size_t)p->n_area * hh * dd);
    p->seq_off = off;  // per-sequence prefix sums of a packed batch: 2 (n_rows + 1) int64
    off = up(off + (size_t)2 * ((size_t)n_rows + 1) * sizeof(int64_t));
    p->carry_off = off;
    if (width > 0) off = up(off + (size_t)2 * n_rows * hh * dd);
    p->ws_bytes = off;
    return off;
  };
  // windows narrower than a sequence whose area is smaller than one slot per chunk
  auto useful = [&](int64_t width) { return width >= 1 && width < p->span && (int64_t)n_rows * width < p->n_slots; };
  if (budget == SIZE_MAX) {
    int64_t width = 0;
    if (p->n_slots * (int64_t)H > kBwdAreaChunkHeads && n_rows > 0) {
      const int64_t w = kBwdAreaChunkHeads / ((int64_t)H * n_rows);
      width = w > kBwdMinWindow ? w : kBwdMinWindow;
      if (!useful(width) || 2 * (int64_t)n_rows * width > p->n_slots) width = 0;
    }
    layout(width);
    return true;
  }
  if (layout(0) <= budget) return true;
  if (n_rows == 0 || p->span < 2) return false;
  // the largest width that fits: the size grows with the width, so estimate
  // it, then step down past the alignment slack
  const size_t fixed = layout(1) - (size_t)n_rows * (size_t)per_slot;
  if (fixed >= budget) return false;
  int64_t width = (int64_t)((budget - fixed) / ((size_t)n_rows * (size_t)per_slot));
  if (width >= p->span) width = p->span - 1;
  while (width >= 1 && layout(width) > budget) --width;
  if (!useful(width)) return false;
  return true;
}

// Launches of one backward call, in stream order.
constexpr int kBwdLaunches = 4;  // forward replay (3 kernels), chunk records, state gradients, local gradients

// A second stream for the forward replay of a backward call, with the two
// caller-created events that fork it from the call's stream and join it back
// (hipStream_t, hipEvent_t, hipEvent_t).
struct AuxStream {
  void* stream;
  void* fork;
  void* join;
};

// Enqueue the backward pass.  All arguments were validated by the caller;
// dout is [.., H, d] in the operand type, dht may be null (zero), dg is null
// without a gate, dh0 may be null (not written).  events: null, or
// kBwdLaunches + 1 hipEvent_t handles recorded before each stage and after
// the last.  aux: null (every launch on `stream`), or a second stream for the
// forward replay and the local gradients of the later half of the chunks
// (then events must be null).  Returns a hipError_t.
int launch_chunk_backward(int is_bf16, int d, int n_rows, int T, int H, const BwdPlan& bp, float g_floor, int gate,
                          const ChunkInputs& in, const float* h0, const int32_t* cu, const void* dout,
                          const float* dht, void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0,
                          void* ws, void* stream, void* const* events, const AuxStream* aux = nullptr);

// Enqueue one decode step (gate: a kda_gate_t).  Returns a hipError_t.
int launch_decode_step(int is_bf16, int d, int N, int H, float g_floor, int gate,
                       const void* q, const void* k, const void* v,
                       const void* g, const float* beta, float* state, void* o,
                       void* stream);

}  // namespace kda
