// Internal interface between the C-ABI front end (kda_api.cpp, plain C++)
// and the HIP translation units that hold the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk

// How a chunked forward is cut for the GPU.  Every sequence is split into
// segments of `seg_chunks` consecutive chunks.  The workspace holds
//  - one record per (segment, head): three d x d fp32 matrices, the segment's
//    affine state map S_out = M S_in + B (M and B) and its incoming state S_in;
//  - one record per (chunk slot, head) with the chunk's operands for the
//    output pass (slot = segment * seg_chunks + chunk within the segment).
struct SegPlan {
  int seg_chunks;        // chunks per segment
  int64_t n_seg_bound;   // upper bound of segments over all sequences
  size_t rec_bytes;      // bytes of one (segment, head) record
  size_t crec_bytes;     // bytes of one (chunk slot, head) record
  size_t crec_off;       // byte offset of the chunk records
  size_t ws_bytes;       // crec_off + n_seg_bound * seg_chunks * H * crec_bytes
};

// Bytes of one chunk record for key/value width d and operand size esz.  The
// record starts with an image of the output pass's LDS: Qt and Wk as 64 rows
// of d + 16 / esz elements, Kh^T as d rows and P as 64 rows of 64 + 16 / esz
// elements (operand type), gamma (d fp32), padded to a multiple of 1 KiB;
// then Wv, 64 x d fp32.
inline size_t chunk_image_bytes(int d, int esz) {
  const size_t ldt = (size_t)d + 16 / esz, ldc = (size_t)kChunk + 16 / esz;
  const size_t img = (2 * kChunk * ldt + (size_t)d * ldc + kChunk * ldc) * esz + (size_t)d * 4;
  return (img + 1023) / 1024 * 1024;
}
inline size_t chunk_record_bytes(int d, int esz) {
  return chunk_image_bytes(d, esz) + (size_t)kChunk * d * 4;
}

// Chooses the segment length from a cost model of the three launches:
// longer segments mean fewer workgroups in the two chunk passes, shorter ones
// a longer sequential chain in the segment scan.  Host-only, deterministic in
// its arguments.  `packed`: n_rows sequences share T tokens (lengths unknown
// on the host), else n_rows rows of T tokens each.  esz: operand bytes (2 for
// bf16, 4 for fp32).  Returns false on overflow.
inline bool plan_segments(int d, int esz, int n_rows, int64_t T, int H, bool packed, SegPlan* p) {
  const double t_chunk = 3.0;   // us per chunk per workgroup (one workgroup per CU)
  const double t_step = 0.5;    // us per step of the segment scan
  const int64_t n_cu = 256;
  const int64_t chunks_total = (T + kChunk - 1) / kChunk;
  int64_t per_seq = packed ? (chunks_total + n_rows - 1) / (n_rows > 0 ? n_rows : 1) : chunks_total;
  if (per_seq < 1) per_seq = 1;
  const int64_t pairs = (int64_t)n_rows * H;
  double best = 1e300;
  int best_l = 1;
  for (int L = 1; L <= 64; L *= 2) {
    const int64_t segs = (per_seq + L - 1) / L;
    const int64_t wg2 = pairs * segs, wg1 = pairs * (segs - 1);
    const double t = (double)((wg1 + n_cu - 1) / n_cu + (wg2 + n_cu - 1) / n_cu) * L * t_chunk +
                     (double)(segs - 1) * t_step;
    if (t <= best) {
      best = t;
      best_l = L;
    }
    if (L >= per_seq) break;
  }
  p->seg_chunks = best_l;
  if (T == 0) {
    p->n_seg_bound = 0;
  } else if (packed) {
    p->n_seg_bound = (chunks_total + n_rows + best_l - 1) / best_l + n_rows;
  } else {
    p->n_seg_bound = (int64_t)n_rows * ((chunks_total + best_l - 1) / best_l);
  }
  p->rec_bytes = (size_t)3 * d * d * sizeof(float);
  p->crec_bytes = chunk_record_bytes(d, esz);
  if (p->n_seg_bound > ((int64_t)1 << 36) / (H > 0 ? H : 1)) return false;
  p->crec_off = (size_t)p->n_seg_bound * (size_t)H * p->rec_bytes;
  p->ws_bytes = p->crec_off + (size_t)p->n_seg_bound * (size_t)best_l * (size_t)H * p->crec_bytes;
  return true;
}

// Enqueue the chunked forward.  All arguments were validated by the caller.
// n_rows: number of sequences (n_seqs, or B when cu == nullptr).
// Returns a hipError_t.
int launch_chunk_forward(int is_bf16, int d, int n_rows, int T, int H, const SegPlan& plan,
                         float g_floor, const void* q, const void* k, const void* v,
                         const void* g, const float* beta, const float* h0,
                         const int32_t* cu, void* o, float* ht, void* ws, void* stream);

// Enqueue one decode step.  Returns a hipError_t.
int launch_decode_step(int is_bf16, int d, int N, int H, float g_floor,
                       const void* q, const void* k, const void* v,
                       const void* g, const float* beta, float* state, void* o,
                       void* stream);

}  // namespace kda
