// Internal interface between the C-ABI front end (kda_api.cpp, plain C++)
// and the HIP translation units that hold the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk

// How a chunked forward is cut for the GPU.
//  - The chunk pass takes groups of `prep_chunks` consecutive chunks of a
//    sequence, one workgroup per (group, head), and writes one record per
//    (chunk, head) with the chunk's operands for the state passes.
//  - The state passes cut every sequence into segments of `seg_chunks`
//    chunks.  One record per (segment, head) holds three d x d fp32 matrices:
//    the segment's affine state map S_out = M S_in + B (M and B) and its
//    incoming state S_in.
// Workspace: the segment records, then the chunk records.
struct SegPlan {
  int prep_chunks;       // chunks per chunk-pass workgroup
  int seg_chunks;        // chunks per segment of the state passes
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
// in every pass; times per chunk and per scan step measured on the target):
// longer segments mean fewer workgroups in the segment-map and output passes,
// shorter ones a longer chain in the segment scan.  Host-only, deterministic
// in its arguments.  `packed`: n_rows sequences share T tokens (lengths
// unknown on the host; the mean length is used), else n_rows rows of T
// tokens each.  esz: operand bytes (2 bf16, 4 fp32).  Returns false on
// overflow.
inline bool plan_segments(int d, int esz, int n_rows, int64_t T, int H, bool packed, SegPlan* p) {
  const double t_map = 3.0, t_scan = 1.4, t_fwd = 4.7;  // us
  const int64_t n_cu = 256;
  const int64_t chunks_total = (T + kChunk - 1) / kChunk;
  const int rows = n_rows > 0 ? n_rows : 1;
  int64_t per_seq = packed ? (chunks_total + rows - 1) / rows : chunks_total;
  if (per_seq < 1) per_seq = 1;
  const int64_t pairs = (int64_t)n_rows * H;
  auto rounds = [&](int64_t wg) { return (double)((wg + n_cu - 1) / n_cu); };
  double best = 1e300;
  int best_l = 1;
  for (int64_t L = 1;; L *= 2) {
    const int64_t Lc = L < per_seq ? L : per_seq;
    const int64_t segs = (per_seq + Lc - 1) / Lc;
    const double t = rounds(pairs * (segs - 1)) * Lc * t_map + (double)(segs - 1) * t_scan +
                     rounds(pairs * segs) * Lc * t_fwd;
    if (t < best) {
      best = t;
      best_l = (int)Lc;
    }
    if (L >= per_seq) break;
  }
  // A packed batch cut into whole sequences (one segment each) needs the
  // longest sequence to fit: use the bound of all chunks then.
  p->seg_chunks = (packed && best_l >= per_seq) ? (int)(chunks_total > 0 ? chunks_total : 1) : best_l;
  // chunk-pass groups (one workgroup each): long enough that the prefetch of
  // the next chunk pays (at least 4 chunks where there is work for it), short
  // enough that the last round of workgroups stays short: at most a quarter of
  // one CU's share of all chunks, 64 at most
  const int64_t share = (pairs * per_seq + n_cu - 1) / n_cu;
  int64_t cap = share / 4 > 4 ? share / 4 : 4;
  if (cap > per_seq) cap = per_seq;
  int64_t pg = 1;
  while (pg < 64 && 2 * pg <= cap) pg *= 2;
  p->prep_chunks = (int)pg;
  p->n_prep_bound = group_bound(T, n_rows, packed, pg);
  p->n_seg_bound = group_bound(T, n_rows, packed, p->seg_chunks);
  p->n_slots = T == 0 ? 0 : (packed ? chunks_total + n_rows : (int64_t)n_rows * chunks_total);
  p->rec_bytes = (size_t)3 * d * d * sizeof(float);
  p->crec_bytes = chunk_record_bytes(d, esz);
  const int64_t hh = H > 0 ? H : 1;
  if (p->n_seg_bound > ((int64_t)1 << 36) / hh || p->n_slots > ((int64_t)1 << 36) / hh) return false;
  p->crec_off = (size_t)p->n_seg_bound * (size_t)H * p->rec_bytes;
  p->ws_bytes = p->crec_off + (size_t)p->n_slots * (size_t)H * p->crec_bytes;
  return true;
}

// Launches of one chunked forward, in stream order.
constexpr int kLaunches = 4;  // chunk pass, segment maps, segment scan, output pass

// Enqueue the chunked forward.  All arguments were validated by the caller.
// n_rows: number of sequences (n_seqs, or B when cu == nullptr).  events:
// null, or kLaunches + 1 hipEvent_t handles (entries may be null) recorded
// on the stream before each launch and after the last.  Returns a hipError_t.
int launch_chunk_forward(int is_bf16, int d, int n_rows, int T, int H, const SegPlan& plan,
                         float g_floor, const void* q, const void* k, const void* v,
                         const void* g, const float* beta, const float* h0,
                         const int32_t* cu, void* o, float* ht, void* ws, void* stream,
                         void* const* events);

// Enqueue one decode step.  Returns a hipError_t.
int launch_decode_step(int is_bf16, int d, int N, int H, float g_floor,
                       const void* q, const void* k, const void* v,
                       const void* g, const float* beta, float* state, void* o,
                       void* stream);

}  // namespace kda
