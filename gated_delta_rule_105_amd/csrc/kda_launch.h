// Internal interface between the C-ABI front end (kda_api.cpp, plain C++)
// and the HIP translation units that hold the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk

// Gate layouts (the values of kda_gate_t): g per key channel, per head, none.
constexpr int kGateChannel = 0, kGateHead = 1, kGateNone = 2;

// How a chunked forward is cut for the GPU.
//  - The state passes cut every sequence into segments of `seg_chunks`
//    chunks.  One record per (segment, head) holds three d x d fp32 matrices:
//    the segment's affine state map S_out = M S_in + B (M and B) and its
//    incoming state S_in.
//  - The chunk pass writes one record per (chunk, head) with the chunk's
//    operands for the output pass.  With `maps_in_prep` its workgroups are
//    the (segment, head) pairs and also compose the segment maps; otherwise
//    every sequence is a single segment (no maps) and the chunk pass takes
//    groups of `prep_chunks` consecutive chunks of a sequence, one workgroup
//    per (group, head).
// Workspace: the segment records, then the chunk records.
struct SegPlan {
  int prep_chunks;       // chunks per chunk-pass workgroup
  int seg_chunks;        // chunks per segment of the state passes
  bool maps_in_prep;     // chunk-pass groups are the segments, and it writes their maps
  int64_t n_prep_bound;  // upper bound of chunk-pass groups over all sequences
  int64_t n_seg_bound;   // upper bound of segments over all sequences
  int64_t n_slots;       // upper bound of chunks over all sequences
  size_t rec_bytes;      // bytes of one (segment, head) record
  size_t crec_bytes;     // bytes of one (chunk, head) record
  size_t crec_off;       // byte offset of the chunk records
  size_t ws_bytes;       // crec_off + n_slots * H * crec_bytes
};

// Bytes of one chunk record for key/value width d and operand size esz.  The
// record starts with an image of the state passes' LDS: the MFMA A-operand
// fragments (1 KiB each, k-blocks of KB = 32 for bf16 and 16 for fp32) of
// Qt and Wk (4 row tiles x d / KB), Kh^T (d / 16 row tiles x 64 / KB) and P
// (4 x 64 / KB), then gamma (d fp32), padded to a multiple of 1 KiB; then
// Wv, 64 x d in the operand type.
inline size_t chunk_image_bytes(int d, int esz) {
  const size_t kb = esz == 2 ? 32 : 16;
  const size_t frags = 8 * (d / kb) + (size_t)(d / 16) * (kChunk / kb) + 4 * (kChunk / kb);
  return (frags * 1024 + (size_t)d * 4 + 1023) / 1024 * 1024;
}
inline size_t chunk_record_bytes(int d, int esz) {
  return chunk_image_bytes(d, esz) + (size_t)kChunk * d * esz;
}

// Upper bound of groups of g chunks over the sequences: n_rows rows of T
// tokens, or (packed) n_rows sequences sharing T tokens.
inline int64_t group_bound(int64_t T, int n_rows, bool packed, int64_t g) {
  const int64_t chunks = (T + kChunk - 1) / kChunk;
  if (T == 0) return 0;
  if (packed) return (chunks + n_rows + g - 1) / g + n_rows;
  return (int64_t)n_rows * ((chunks + g - 1) / g);
}

// Chooses the cut from a cost model of the launches (one workgroup per CU
// in the chunk and output passes; times per chunk and per scan step measured
// on the target).  Either every sequence is one segment (the chunk pass then
// balances its groups over the CUs on its own, and the output pass walks each
// sequence), or segments of L chunks: one workgroup per (segment, head) in
// both passes, the chunk pass composing the maps, and a scan of
// (segments - 1) steps between them.  Host-only, deterministic in its
// arguments.  `packed`: n_rows sequences share T tokens (lengths unknown on
// the host; the mean length is used), else n_rows rows of T tokens each.
// esz: operand bytes (2 bf16, 4 fp32).  Returns false on overflow.
inline bool plan_segments(int d, int esz, int n_rows, int64_t T, int H, bool packed, SegPlan* p) {
  const double t_prep = 9.0, t_map = 1.5, t_scan = 1.4, t_fwd = 4.7;  // us
  const int64_t n_cu = 256;
  const int64_t chunks_total = (T + kChunk - 1) / kChunk;
  const int rows = n_rows > 0 ? n_rows : 1;
  int64_t per_seq = packed ? (chunks_total + rows - 1) / rows : chunks_total;
  if (per_seq < 1) per_seq = 1;
  const int64_t pairs = (int64_t)n_rows * H;
  auto rounds = [&](int64_t wg) { return (double)((wg + n_cu - 1) / n_cu); };
  // one segment per sequence
  const int64_t share = (pairs * per_seq + n_cu - 1) / n_cu;  // chunks per CU
  double best = (double)share * t_prep + rounds(pairs) * (double)per_seq * t_fwd;
  int best_l = 0;  // 0: one segment per sequence
  for (int64_t L = 1; L < per_seq; L *= 2) {
    const int64_t segs = (per_seq + L - 1) / L;
    const double t = rounds(pairs * segs) * (double)L * (t_prep + t_map + t_fwd) + (double)(segs - 1) * t_scan;
    if (t < best) {
      best = t;
      best_l = (int)L;
    }
  }
  p->maps_in_prep = best_l > 0;
  if (p->maps_in_prep) {
    p->seg_chunks = best_l;
    p->prep_chunks = best_l;
  } else {
    // Whole sequences: a packed batch needs the longest sequence to fit, so
    // the segment is the bound of all chunks.  Chunk-pass groups: long enough
    // that the prefetch of the next chunk pays (at least 4 chunks where there
    // is work for it), short enough that the last round of workgroups stays
    // short: at most a quarter of one CU's share of all chunks, 64 at most.
    p->seg_chunks = (int)(packed ? (chunks_total > 0 ? chunks_total : 1) : per_seq);
    int64_t cap = share / 4 > 4 ? share / 4 : 4;
    if (cap > per_seq) cap = per_seq;
    int64_t pg = 1;
    while (pg < 64 && 2 * pg <= cap) pg *= 2;
    p->prep_chunks = (int)pg;
  }
  p->n_seg_bound = group_bound(T, n_rows, packed, p->seg_chunks);
  p->n_prep_bound = p->maps_in_prep ? p->n_seg_bound : group_bound(T, n_rows, packed, p->prep_chunks);
  p->n_slots = T == 0 ? 0 : (packed ? chunks_total + n_rows : (int64_t)n_rows * chunks_total);
  p->rec_bytes = (size_t)3 * d * d * sizeof(float);
  p->crec_bytes = chunk_record_bytes(d, esz);
  const int64_t hh = H > 0 ? H : 1;
  if (p->n_seg_bound > ((int64_t)1 << 36) / hh || p->n_slots > ((int64_t)1 << 36) / hh) return false;
  p->crec_off = (size_t)p->n_seg_bound * (size_t)H * p->rec_bytes;
  p->ws_bytes = p->crec_off + (size_t)p->n_slots * (size_t)H * p->crec_bytes;
  return true;
}

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
constexpr int kLaunches = 3;  // chunk pass (with the segment maps), segment scan, output pass

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
// Floats of one (chunk, head) record of the backward pass at width d: eight
// [64][d] blocks (Qt, Kt, Kh, V, dO, Wk, Wv, Gamma), three [64][64] (P, T, Abar),
// gamma [d] and beta [64]; and of one (chunk, head) scratch area of its local
// gradient kernel: five [64][d] blocks, two [64][64] and one [d].
constexpr size_t bwd_rec_floats(int d) {
  return (size_t)8 * kChunk * d + (size_t)3 * kChunk * kChunk + (size_t)d + kChunk;
}
constexpr size_t bwd_scr_floats(int d) { return (size_t)5 * kChunk * d + (size_t)2 * kChunk * kChunk + (size_t)d; }

// Workspace of one backward call (byte offsets, each 256-byte aligned): the
// forward replay's own workspace first, then its o (discarded), its final
// states, the state after every full chunk, one zero state, the chunk
// records, the scratch areas, the end-state gradient of every chunk and the
// per-sequence chunk and state-slot offsets of a packed batch.
struct BwdPlan {
  SegPlan fwd;
  int64_t n_slots;  // upper bound of chunks over all sequences
  size_t o_off, ht_off, states_off, zero_off, rec_off, scr_off, dh_off, seq_off, ws_bytes;
  size_t rec_floats, scr_floats;
};

// n_states: sequences; chunk_states: full chunks over all sequences (an
// upper bound for a packed batch).  Returns false on overflow.
inline bool plan_backward(int d, int esz, int n_rows, int64_t T, int H, bool packed, size_t tokens,
                          size_t chunk_states, BwdPlan* p) {
  if (!plan_segments(d, esz, n_rows, T, H, packed, &p->fwd)) return false;
  const size_t a = 256, hh = (size_t)H, dd = (size_t)d * d * sizeof(float);
  auto up = [&](size_t x) { return (x + a - 1) / a * a; };
  p->n_slots = p->fwd.n_slots;
  p->rec_floats = bwd_rec_floats(d);
  p->scr_floats = bwd_scr_floats(d);
  const double total = (double)p->fwd.ws_bytes + (double)tokens * hh * d * esz +
                       ((double)n_rows + (double)chunk_states + 1.0) * hh * dd +
                       (double)p->n_slots * hh * ((p->rec_floats + p->scr_floats) * 4.0 + (double)dd);
  if (total > 1.0e15) return false;
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
  off = up(off + (size_t)p->n_slots * hh * p->rec_floats * 4);
  p->scr_off = off;
  off = up(off + (size_t)p->n_slots * hh * p->scr_floats * 4);
  p->dh_off = off;
  off = up(off + (size_t)p->n_slots * hh * dd);
  p->seq_off = off;  // per-sequence prefix sums of a packed batch: 2 (n_rows + 1) int64
  off = up(off + (size_t)2 * ((size_t)n_rows + 1) * sizeof(int64_t));
  p->ws_bytes = off;
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
