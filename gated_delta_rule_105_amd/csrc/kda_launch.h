// Internal interface between the C-ABI front end (kda_api.cpp, plain C++)
// and the HIP translation units that hold the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk

// How a chunked forward is cut for the GPU.  Every sequence is split into
// segments of `seg_chunks` consecutive chunks.  Each (segment, head) has one
// workspace record of three d x d fp32 matrices: the segment's affine state
// map S_out = M S_in + B (M and B) and its incoming state S_in.
struct SegPlan {
  int seg_chunks;        // chunks per segment
  int64_t n_seg_bound;   // upper bound of segments over all sequences
  size_t rec_bytes;      // bytes of one (segment, head) record
  size_t ws_bytes;       // n_seg_bound * H * rec_bytes
};

// Chooses the segment length from a cost model of the three launches:
// longer segments mean fewer workgroups in the two chunk passes, shorter ones
// a longer sequential chain in the segment scan.  Host-only, deterministic in
// its arguments.  `packed`: n_rows sequences share T tokens (lengths unknown
// on the host), else n_rows rows of T tokens each.  Returns false on overflow.
inline bool plan_segments(int d, int n_rows, int64_t T, int H, bool packed, SegPlan* p) {
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
  if (p->n_seg_bound > ((int64_t)1 << 40) / (H > 0 ? H : 1)) return false;
  p->ws_bytes = (size_t)p->n_seg_bound * (size_t)H * p->rec_bytes;
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
