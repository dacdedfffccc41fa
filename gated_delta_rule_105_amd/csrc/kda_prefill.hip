// Chunked KDA forward for gfx950: two sweeps over the inputs around a
// segment scan.
//
// Chunk algebra (per sequence and head; chunk rows r = 0..63, S the state
// entering the chunk, g floored, G = running sum of g over the chunk's rows,
// G_L its last row, gamma = e^{G_L} per key channel):
//   Qt = Q e^{G},  Kt = K e^{G},  Kh = K e^{-G}
//   A  = diag(beta) strict_lower(Kt Kh^T),   (I + A) W = diag(beta) [Kt | V]
//   Wk, Wv = the two halves of W,   P = lower_incl(Qt Kh^T)
//   U  = Wv - Wk S,   O = Qt S + P U,   S <- diag(gamma) (S + Kh^T U)
// which is the recurrence S_t = (I - b k k^T) diag(a) S_{t-1} + b k v^T,
// o_t = S_t^T q_t unrolled over one chunk (K e^{G_L - G} = diag(gamma) Kh
// folds the chunk-end decay into one row scaling).  Sources: chunk-parallel
// computation with an inter-chunk recurrence built from blocked matrix
// products, "Kimi K3 深度拆解" (chenxutan.com), 4.2; the lower bound on the
// log-decay, which keeps e^{-G} finite so that the diagonal block is a dense
// product too, "3 分钟看懂 Kimi K3" (landx.limxdynamics.com), "第一条主线",
// Figure 3, and "Kimi K3 发布 47 页技术报告" (163.com), 01.
//
// One chunk maps the state affinely, S -> M_j S + B_j.  Every sequence is cut
// into segments of L chunks; a segment's composition is again affine,
// S_out = M S_in + B.  Up to three launches:
//   1. map sweep (kda_chunk_sweep<MAP>, one workgroup per (segment, head)):
//      the chunk-local algebra of each chunk from the inputs, then one state
//      step on B (from 0) and on M (from I, value part of U off); writes the
//      segment's (M, B).  The last segment of a sequence has none.
//   2. kda_seg_scan (one workgroup per (sequence, head, 16 state columns)):
//      S_0 = h0, S_{s+1} = M_s S_s + B_s, writing every segment's S_in.
//      M S is three bf16 products of a hi/lo split of both factors.
//   3. output sweep (kda_chunk_sweep<OUT>, one workgroup per (segment,
//      head)): the chunk-local algebra again, and the state step with the
//      outputs from S_in; writes o, the final state and prefix-cache states.
// With one segment per sequence only the output sweep runs, from h0.
//
// Within a chunk (one workgroup of D / 16 waves): the inputs arrive in
// registers (fetched during the previous chunk); the element-wise stage
// writes Qt, Kt, Kh and V token-major to LDS.  Operands whose contraction
// runs over tokens (Kt, V, Kh^T, Wk) are read from token- or channel-major
// arrays with the gfx950 transpose read, so no array is stored twice.  The
// triangular system is solved by 16-row blocks: the diagonal blocks'
// inverses by substitution, the rest by MFMA block products.  Wave w owns
// 16 value columns: columns of W, U, O and S never mix.
#include <mutex>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"
#include "kda_rows.h"

// Scratch of the allocation-free forward: segment records and packed prefix
// sums of kda_chunk_forward_noalloc, one copy per device, held from the
// library's load until the process ends.  Host code never uses this name as
// an address (on the host it is a stand-in, not device memory): the device
// address comes from kda::scratch_buffer.  Every word a call reads is
// written earlier in the same call, so nothing is cleared between calls.
static __device__ __align__(256) unsigned char scratch[kda::kScratchBytes];

namespace kda {
namespace {

constexpr int C = kChunk;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---- LDS arrays -------------------------------------------------------------
// A [rows][W] array is stored with rows of W + 16 elements and in units of 4
// elements; unit u of row t sits at unit u ^ ((t >> 2) & 3).  The padding
// puts consecutive rows 8 banks apart; the swizzle touches only the two low
// bits of the unit, which hold the lane-dependent part of every access, so
// each lane's addresses into an array differ by immediates only.  Both
// access patterns used here hit distinct banks within 16 lanes: 16 rows at
// one unit (row fragments) and 4 rows x 4 units (transpose reads).
// sidx is the layout's definition (element (t, c) of a [rows][W] array); the
// accessors (LaneOff, the element-wise stage) form the same offsets as a
// lane register plus immediates.
template <int W>
__device__ __forceinline__ int sidx(int t, int c) {
  return t * (W + 16) + ((((c >> 2) ^ ((t >> 2) & 3))) << 2) + (c & 3);
}
// Workgroup barrier that orders LDS accesses only: it waits for this wave's
// LDS operations, not for its global loads, so that the next chunk's inputs
// stay in flight across it (__syncthreads() would wait for them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, int W> struct Arr {
  static constexpr int BYTES = C * (W + 16) * (int)sizeof(T);  // 64 rows
};

// Lane-dependent part of an array access, in elements.  For a tile whose
// first row r0 and first column c0 (or k-block start k0) are multiples of 16,
// the swizzle's XOR acts on lane bits only, so an access is this part plus
// r0 (W + 16) + c0: one register per array width and access pattern, the
// rest immediates.
//   row: row fragment, lane (g, i) at row r0 + i, elements k0 + 4 g ...
//   col: column piece (bf16: lane (g, L) addressing row r0 + 4 g + L / 4 at
//        elements c0 + 4 (L % 4) ..; fp32: row r0 + 4 g, element c0 + i)
template <typename T, int W> struct LaneOff {
  int row, col;
  __device__ __forceinline__ explicit LaneOff(int lane) {
    const int g = lane >> 4, i = lane & 15;
    row = i * (W + 16) + ((g ^ ((i >> 2) & 3)) << 2);
    if constexpr (sizeof(T) == 2) col = (4 * g + (i >> 2)) * (W + 16) + (((i & 3) ^ g) << 2);
    else col = 4 * g * (W + 16) + (((i >> 2) ^ g) << 2) + (i & 3);
  }
};

// A lane's index and its offsets into the [64][D] and [D][64] arrays.
template <typename T, int D> struct Lanes {
  int lane;
  LaneOff<T, D> d;
  LaneOff<T, kChunk> c;
  __device__ __forceinline__ explicit Lanes(int l) : lane(l), d(l), c(l) {}
};

// Row fragment (A- or B-operand whose k runs along a row): row r0 + i,
// elements k0 + 4g .. k0 + 4g + 3 and, for bf16 (k-blocks of 32), k0 + 16 + 4g ...
template <int W>
__device__ __forceinline__ bf16x8 rowfrag(const bf16_t* X, const LaneOff<bf16_t, W>& lo_, int r0, int k0) {
  const bf16_t* p = X + lo_.row + r0 * (W + 16) + k0;
  const bf16x4 lo = *(const bf16x4*)p;
  const bf16x4 hi = *(const bf16x4*)(p + 16);
  return (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <int W>
__device__ __forceinline__ f32x4 rowfrag(const float* X, const LaneOff<float, W>& lo_, int r0, int k0) {
  return *(const f32x4*)(X + lo_.row + r0 * (W + 16) + k0);
}
// Column piece: lane (g, i) gets X[r0 + 4g + e][c0 + i], e = 0..3 (the
// accumulator layout of a 16 x 16 tile, and an operand fragment whose k runs
// down a column).  bf16: one transpose read; fp32: four scalar reads.
template <int W>
__device__ __forceinline__ s16x4 colpiece(const bf16_t* X, const LaneOff<bf16_t, W>& lo_, int r0, int c0) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + lo_.col + r0 * (W + 16) + c0));
}
template <int W>
__device__ __forceinline__ f32x4 colpiece(const float* X, const LaneOff<float, W>& lo_, int r0, int c0) {
  f32x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = X[lo_.col + (r0 + e) * (W + 16) + c0];
  return x;
}
__device__ __forceinline__ f32x4 widen4(const s16x4& h) {
  const uint2 w = __builtin_bit_cast(uint2, h);
  return (f32x4){__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 widen4(const f32x4& x) { return x; }
// Column fragment over a k-block (bf16: 32 rows as two pieces; fp32: 16)
template <int W>
__device__ __forceinline__ bf16x8 colfrag(const bf16_t* X, const LaneOff<bf16_t, W>& lo_, int r0, int c0) {
  const s16x4 a = colpiece<W>(X, lo_, r0, c0), b = colpiece<W>(X, lo_, r0 + 16, c0);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <int W>
__device__ __forceinline__ f32x4 colfrag(const float* X, const LaneOff<float, W>& lo_, int r0, int c0) {
  return colpiece<W>(X, lo_, r0, c0);
}

// ---- LDS layout of a sweep workgroup --------------------------------------
// Token-major [64][D]: Qt (output sweep only) and Kh in two buffer sets (a
// chunk's state step reads them while the next chunk's element-wise stage
// writes the other set), Kt, V.  Channel-major [D][64]: Wk^T.  Fragment
// images in lane order: P tiles (rt, sb), sb <= rt (output sweep), 4
// elements a lane; coefficient images of 16 bytes a lane (Blk): the
// off-diagonal blocks of -A (i, m), m < i, and the diagonal blocks' inverses
// T_bb.  fp32: partial sums of g [8][D], beta [64], gamma [D] in two buffer
// sets.
// After the last chunk the map sweep stages M [D][D + 4] fp32 from offset 0.
template <typename T, int D, bool OUT> struct Lay {
  static constexpr int ES = (int)sizeof(T);
  // two buffer sets (state step overlapped with the next element-wise stage)
  // on the bf16 path; the fp32 path, whose arrays are twice as large, runs
  // the state step in an interval of its own with one set
  static constexpr bool OVL = ES == 2;
  static constexpr int NBUF = OVL ? 2 : 1;
  static constexpr int ARR = Arr<T, D>::BYTES;       // token-major [64][D]
  static constexpr int ARRT = D * (C + 16) * ES;     // channel-major [D][64]
  static constexpr int IMG = 64 * 4 * ES;            // one fragment image (P tiles)
  static constexpr int CIMG = 64 * 16;               // one coefficient image (16 bytes a lane)
  static constexpr int QT0 = 0;                      // Qt, two buffer sets (output sweep)
  static constexpr int KH0 = QT0 + (OUT ? NBUF * ARR : 0);  // Kh, two buffer sets
  static constexpr int KT = KH0 + NBUF * ARR;
  static constexpr int VV = KT + ARR;
  static constexpr int WKT = VV + ARR;
  static constexpr int PIMG = WKT + ARRT;
  static constexpr int AIMG = PIMG + (OUT ? 10 * IMG : 0);
  static constexpr int TIMG = AIMG + 6 * CIMG;
  static constexpr int PART = TIMG + 4 * (ES == 2 ? 2 : 1) * CIMG;
  static constexpr int BETA = PART + 8 * D * 4;
  static constexpr int GAM0 = BETA + C * 4;          // gamma, two buffer sets
  static constexpr int STAGE_M = D * (D + 4) * 4;
  static constexpr int END = GAM0 + NBUF * D * 4;
  static constexpr int BYTES = OUT || END >= STAGE_M ? END : STAGE_M;
  __device__ static __forceinline__ int qt(int buf) { return QT0 + (OVL ? buf : 0) * ARR; }
  __device__ static __forceinline__ int kh(int buf) { return KH0 + (OVL ? buf : 0) * ARR; }
  __device__ static __forceinline__ int gam(int buf) { return GAM0 + (OVL ? buf : 0) * D * 4; }
  __device__ static __forceinline__ int pimg(int rt, int sb) { return PIMG + (rt * (rt + 1) / 2 + sb) * IMG; }
  __device__ static __forceinline__ int aimg(int i, int m) { return AIMG + (i * (i - 1) / 2 + m) * CIMG; }
  __device__ static __forceinline__ int timg(int b) { return TIMG + b * (ES == 2 ? 2 : 1) * CIMG; }
};

// ---- sequences and segments -----------------------------------------------
struct Seg {
  int64_t tok0;   // first packed token of the sequence
  int64_t slot0;  // first prefix-cache state slot of the sequence
  int len;        // tokens of the sequence
  int n;          // sequence
  int s;          // segment within the sequence
  int nseg;       // segments of the sequence
};
__device__ __forceinline__ int n_segments(int64_t len, int L) { return (int)(((len + C - 1) / C + L - 1) / L); }

// Packed batches: seqs[n] = segments of sequences 0 .. n - 1, seqs[n_rows +
// 1 + n] = prefix-cache state slots of sequences 0 .. n - 1 (kda_fwd_seqs).
// Global segment gs -> its sequence (binary search); false past the last.
__device__ __forceinline__ bool locate(const int32_t* cu, const int64_t* seqs, int n_rows, int T_per, int L,
                                       int64_t period, int64_t gs, Seg& r) {
  if (!cu) {
    const int per = n_segments(T_per, L);
    if (per == 0) return false;
    const int64_t n = gs / per;
    if (n >= n_rows) return false;
    r.n = (int)n;
    r.s = (int)(gs % per);
    r.nseg = per;
    r.tok0 = n * (int64_t)T_per;
    r.len = T_per;
    r.slot0 = period > 0 ? n * (T_per / period) : 0;
    return true;
  }
  if (n_rows == 0 || gs >= seqs[n_rows]) return false;
  int lo = 0, hi = n_rows - 1;  // the largest n with seqs[n] <= gs: not an empty sequence
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (seqs[mid] <= gs) lo = mid;
    else hi = mid - 1;
  }
  r.n = lo;
  r.s = (int)(gs - seqs[lo]);
  r.tok0 = cu[lo];
  r.len = cu[lo + 1] - cu[lo];
  r.nseg = n_segments(r.len, L);
  r.slot0 = seqs[n_rows + 1 + lo];
  return true;
}

// The prefix sums above for n_rows packed sequences: one workgroup, each
// thread summing a contiguous range of sequences, then the ranges' offsets.
// period = tokens per prefix-cache state (0: none).
__global__ void __launch_bounds__(256) kda_fwd_seqs(const int32_t* __restrict__ cu, int n_rows, int L,
                                                    int64_t period, int64_t* __restrict__ seqs) {
  __shared__ int64_t part[2][256];
  const int tid = threadIdx.x, per = (n_rows + 255) / 256;
  const int n0 = min(n_rows, tid * per), n1 = min(n_rows, n0 + per);
  int64_t a = 0, f = 0;
  for (int n = n0; n < n1; ++n) {
    const int64_t len = (int64_t)cu[n + 1] - cu[n];
    a += n_segments(len, L);
    f += period > 0 ? len / period : 0;
  }
  part[0][tid] = a;
  part[1][tid] = f;
  __syncthreads();
  int64_t oa = 0, of = 0;
  for (int t = 0; t < tid; ++t) {
    oa += part[0][t];
    of += part[1][t];
  }
  for (int n = n0; n < n1; ++n) {
    seqs[n] = oa;
    seqs[n_rows + 1 + n] = of;
    const int64_t len = (int64_t)cu[n + 1] - cu[n];
    oa += n_segments(len, L);
    of += period > 0 ? len / period : 0;
  }
  if (tid == 255) {
    seqs[n_rows] = oa;
    seqs[2 * n_rows + 1] = of;
  }
}

// ---- segment record: three d x d blocks of fp32 size per (segment, head)
//   B    : [d/16 row tiles][d/16 column tiles][64 lanes][4] fp32, accumulator
//          tile order (lane 16 g + i holds rows 4 g .. 4 g + 3 of column i)
//   M    : A-operand fragments of M for the scan, [d/16 row tiles][k-blocks]
//          [64 lanes][16 bytes]; bf16 keeps a hi and a lo fragment per slot
//          (M = hi + lo to about 2^-17), fp32 keeps M itself
//   S_in : incoming state of the segment, accumulator tile order like B
template <typename T, int D> struct Rec {
  static constexpr int NRT = D / 16, KB = Elem<T>::KB, NKB = D / KB;
  static constexpr size_t B = 0, M = (size_t)D * D, SIN = 2 * (size_t)D * D, FLOATS = 3 * (size_t)D * D;
  __device__ static __forceinline__ size_t tile(int rr, int ct, int lane) {
    return (((size_t)rr * NRT + ct) * 64 + lane) * 4;
  }
  __device__ static __forceinline__ size_t frag(int rr, int kb, int part, int lane) {
    return ((((size_t)rr * NKB + kb) * (sizeof(T) == 2 ? 2 : 1) + part) * 64 + lane) * 16;
  }
};

// ---- chunk inputs: Raw (kda_rows.h) ------------------------------------------

// ---- element-wise stage -----------------------------------------------------
// Floored log-decays in log2 units (every factor is one exp2); their partial
// sums over the thread's 8 rows go to PART (estage1); after a barrier each
// thread adds the parts before its own and forms Qt, Kt, Kh row by row, stored
// with V, beta and gamma into the chunk's buffer set `buf` (estage2).
template <typename T, int D, bool OUT, bool MX, bool NT>
__device__ __forceinline__ void estage1(unsigned char* smem, const Raw<T, D, OUT, MX, NT>& raw, float g_floor,
                                        int gate, int tid, float (&g0)[8], float (&g1)[8]) {
  typedef Lay<T, D, OUT> Y;
  typedef PairT<T> PW;
  constexpr float kLog2e = 1.4426950408889634f;
  const int cp = tid % (D / 2), part = tid / (D / 2), c = 2 * cp;
  typename PW::word w[8];
  if (gate == kGateHead) {
#pragma unroll
    for (int s = 0; s < 8; ++s) w[s] = PW::splat(raw.g[s]);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) w[s] = raw.g[s];
  }
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float x0 = PW::lo(w[s]), x1 = PW::hi(w[s]);
    g0[s] = __builtin_elementwise_maximum(x0, g_floor) * kLog2e;  // NaN-propagating: NaN stays NaN
    g1[s] = __builtin_elementwise_maximum(x1, g_floor) * kLog2e;
    p0 += g0[s];
    p1 += g1[s];
  }
  *(f32x2*)((float*)(smem + Y::PART) + part * D + c) = (f32x2){p0, p1};
}
template <typename T, int D, bool OUT, bool MX, bool NT>
__device__ __forceinline__ void estage2(unsigned char* smem, int buf, const Raw<T, D, OUT, MX, NT>& raw, int tid,
                                        const float (&g0)[8], const float (&g1)[8]) {
  typedef Lay<T, D, OUT> Y;
  typedef PairT<T> PW;
  typedef typename PW::word word;
  const int cp = tid % (D / 2), part = tid / (D / 2), c = 2 * cp;
  // element of row 8 part + s, channel c in the swizzled arrays: the row's
  // swizzle flips unit bit 0 from s = 4 on (the rest is the thread's)
  const int eb0 = 8 * part * (D + 16) + (((cp >> 1) ^ (2 * (part & 1))) << 2) + 2 * (cp & 1), eb1 = eb0 ^ 4;
  const float* sPart = (const float*)(smem + Y::PART);
  float gam0 = 0.f, gam1 = 0.f, gl0 = 0.f, gl1 = 0.f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const f32x2 x = *(const f32x2*)(sPart + p * D + c);
    gam0 += p < part ? x[0] : 0.f;
    gam1 += p < part ? x[1] : 0.f;
    gl0 += x[0];
    gl1 += x[1];
  }
  if (part == 0)
    *(f32x2*)((float*)(smem + Y::gam(buf)) + c) = (f32x2){__builtin_amdgcn_exp2f(gl0), __builtin_amdgcn_exp2f(gl1)};
  T* sQ = (T*)(smem + Y::qt(buf));
  T* sK = (T*)(smem + Y::KT);
  T* sH = (T*)(smem + Y::kh(buf));
  T* sV = (T*)(smem + Y::VV);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int e = (s < 4 ? eb0 : eb1) + s * (D + 16);
    gam0 += g0[s];
    gam1 += g1[s];
    const float e0 = __builtin_amdgcn_exp2f(gam0), e1 = __builtin_amdgcn_exp2f(gam1);
    const float ei0 = __builtin_amdgcn_exp2f(-gam0), ei1 = __builtin_amdgcn_exp2f(-gam1);
    const word kw = raw.kw(s);
    const float k0 = PW::lo(kw), k1 = PW::hi(kw);
    *(word*)(sK + e) = PW::pack(k0 * e0, k1 * e1);
    *(word*)(sH + e) = PW::pack(k0 * ei0, k1 * ei1);
    *(word*)(sV + e) = raw.vw(s);
    if (OUT) {
      const word qw = raw.qw(s);
      *(word*)(sQ + e) = PW::pack(PW::lo(qw) * e0, PW::hi(qw) * e1);
    }
  }
  if (tid < C) ((float*)(smem + Y::BETA))[tid] = raw.beta;
}

// ---- fragment images and 16 x 16 x 16 block products ----------------------
__device__ __forceinline__ s16x4 to_bf16x4(const f32x4& x) {
  const uint32_t a = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[0], x[1]));
  const uint32_t b = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[2], x[3]));
  return __builtin_bit_cast(s16x4, (uint2){a, b});
}
// Blk<T>: 16 x 16 x 16 block products of the triangular solve.  Coefficient
// fragments (A operand: lane (g, i) holds row i, k = 4 g .. 4 g + 3) are kept
// as images of 16 bytes per lane; right operands come from accumulator
// tiles.  bf16: a right operand is split hi + lo so that the product keeps
// about fp32 accuracy in it, and the two halves go down the k dimension of
// one 16 x 16 x 32 product against a coefficient image stored twice,
// [a | a]: a (hi + lo) in one instruction.  The diagonal inverses are split
// too, stored as two images [lo | hi] and [hi | 0]: tri forms lo r_hi + hi
// r_lo, then hi r_hi, in two 16 x 16 x 32 products.  (Every accumulation
// chain stays on one MFMA shape: a 16 x 16 x 16 product reading a 16 x 16 x
// 32 product's result as its accumulator, issued back to back, gave wrong
// sums.)  fp32: fp32 MFMA throughout.
__device__ __forceinline__ bf16x8 cat4(const s16x4& x, const s16x4& y) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <typename T> struct Blk;
template <> struct Blk<bf16_t> {
  typedef bf16x8 Coef;  // [a | a], or [lo | hi] and [hi | 0]
  typedef bf16x8 Opnd;  // [hi | lo]
  __device__ static __forceinline__ Coef load(const unsigned char* p) { return *(const bf16x8*)p; }
  // a plain 4-element image (P tiles)
  __device__ static __forceinline__ void store(unsigned char* p, const f32x4& x) { *(s16x4*)p = to_bf16x4(x); }
  __device__ static __forceinline__ void store_coef(unsigned char* p, const f32x4& x) {
    const s16x4 h = to_bf16x4(x);
    *(bf16x8*)p = cat4(h, h);
  }
  // the two images of a diagonal inverse, p and p + TRI2
  static constexpr int TRI2 = 64 * 16;
  __device__ static __forceinline__ void store_tri(unsigned char* p, const f32x4& x) {
    const s16x4 h = to_bf16x4(x);
    *(bf16x8*)p = cat4(to_bf16x4(x - widen4(h)), h);
    *(bf16x8*)(p + TRI2) = cat4(h, (s16x4){0, 0, 0, 0});
  }
  __device__ static __forceinline__ Opnd opnd(const f32x4& b) {
    const s16x4 h = to_bf16x4(b);
    return cat4(h, to_bf16x4(b - widen4(h)));
  }
  __device__ static __forceinline__ f32x4 apply(const Coef& a, const Opnd& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 tri(const Coef& t1, const Coef& t2, const Opnd& r) {
    const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t1, r, (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(t2, r, c, 0, 0, 0);
  }
};
template <> struct Blk<float> {
  typedef f32x4 Coef;
  typedef f32x4 Opnd;
  __device__ static __forceinline__ Coef load(const unsigned char* p) { return *(const f32x4*)p; }
  __device__ static __forceinline__ void store(unsigned char* p, const f32x4& x) { *(f32x4*)p = x; }
  __device__ static __forceinline__ void store_coef(unsigned char* p, const f32x4& x) { *(f32x4*)p = x; }
  static constexpr int TRI2 = 0;  // one image
  __device__ static __forceinline__ void store_tri(unsigned char* p, const f32x4& x) { *(f32x4*)p = x; }
  __device__ static __forceinline__ Opnd opnd(const f32x4& b) { return b; }
  __device__ static __forceinline__ f32x4 apply(const Coef& a, const Opnd& b, f32x4 c) { return mma(a, b, c); }
  __device__ static __forceinline__ f32x4 tri(const Coef& t, const Coef&, const Opnd& r) {
    return mma(t, r, (f32x4){0.f, 0.f, 0.f, 0.f});
  }
};

// ---- Gram tiles ---------------------------------------------------------------
// lane (g, i) = sum_c XA[ra + 4 g + e][c] XB[rb + i][c]: with XA = Kh and
// XB = Kt or Qt, element (row rb + i, k = ra + 4 g + e) of Kt Kh^T or Qt Kh^T,
// i.e. directly the coefficient fragment of that block.
template <typename T, int D>
__device__ __forceinline__ f32x4 gram_tile(const T* XA, int ra, const T* XB, int rb, const Lanes<T, D>& ln) {
  constexpr int KB = Elem<T>::KB;
  typename Frag<T>::type fa[D / KB], fb[D / KB];
#pragma unroll
  for (int kb = 0; kb < D / KB; ++kb) {
    fa[kb] = rowfrag<D>(XA, ln.d, ra, kb * KB);
    fb[kb] = rowfrag<D>(XB, ln.d, rb, kb * KB);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < D / KB; ++kb) acc = mma(fa[kb], fb[kb], acc);
  return acc;
}
// Off-diagonal block (i, m), m < i, of -A = -diag(beta) Kt Kh^T, as an image.
template <typename T, int D, bool OUT>
__device__ __forceinline__ void a_block(unsigned char* smem, int buf, int i, int m, const Lanes<T, D>& ln) {
  typedef Lay<T, D, OUT> Y;
  const f32x4 t = gram_tile<T, D>((const T*)(smem + Y::kh(buf)), 16 * m, (const T*)(smem + Y::KT), 16 * i, ln);
  const float nb = -((const float*)(smem + Y::BETA))[16 * i + (ln.lane & 15)];
  Blk<T>::store_coef(smem + Y::aimg(i, m) + ln.lane * 16, nb * t);
}
// Tile (rt, sb), sb <= rt, of P = lower_incl(Qt Kh^T), as an image.
template <typename T, int D>
__device__ __forceinline__ void p_block(unsigned char* smem, int buf, int rt, int sb, const Lanes<T, D>& ln) {
  typedef Lay<T, D, true> Y;
  const int lane = ln.lane;
  f32x4 t = gram_tile<T, D>((const T*)(smem + Y::kh(buf)), 16 * sb, (const T*)(smem + Y::qt(buf)), 16 * rt, ln);
  if (sb == rt) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * (lane >> 4) + e > (lane & 15)) t[e] = 0.f;
  }
  Blk<T>::store(smem + Y::pimg(rt, sb) + lane * 4 * Y::ES, t);
}
// Diagonal block b: T_bb = (I + A_bb)^{-1}, A_bb = diag(beta) strict_lower(
// Kt Kh^T) (16 x 16, nilpotent).  With N = -A_bb,
//   T_bb = (I + N)(I + N^2)(I + N^4)(I + N^8)
// (N^16 = 0), four levels of 16 x 16 x 16 fp32 MFMA products instead of a
// 16-step substitution.  A 16 x 16 matrix X is held in one of two layouts:
// coef(X) (lane (g, i) has X[i][4 g + e], a left operand) and acc(X) (lane
// (g, i) has X[4 g + e][i], a right operand and a product's result); coef(X)
// = acc(X^T), so for Z = X Y: acc(Z) = mma(coef(X), acc(Y)) and coef(Z) =
// mma(acc(Y), coef(X)).  The two Gram tiles give N in both layouts.  Lane
// (g, i) ends with coef(T_bb), the coefficient fragment, stored as an image
// (bf16: hi and lo).
template <typename T, int D, bool OUT>
__device__ __forceinline__ void diag_block(unsigned char* smem, int buf, int b, const Lanes<T, D>& ln) {
  typedef Lay<T, D, OUT> Y;
  const int lane = ln.lane, g = lane >> 4, i = lane & 15;
  const T* sK = (const T*)(smem + Y::KT);
  const T* sH = (const T*)(smem + Y::kh(buf));
  const float* sB = (const float*)(smem + Y::BETA) + 16 * b;
  const f32x4 tc = gram_tile<T, D>(sH, 16 * b, sK, 16 * b, ln);  // (Kt Kh^T)[i][4 g + e]
  const f32x4 ta = gram_tile<T, D>(sK, 16 * b, sH, 16 * b, ln);  // (Kt Kh^T)[4 g + e][i]
  const float bi = sB[i];
  const f32x4 b4 = *(const f32x4*)(sB + 4 * g);
  f32x4 cN, aN, cT;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    cN[e] = (4 * g + e < i) ? -bi * tc[e] : 0.f;
    aN[e] = (i < 4 * g + e) ? -b4[e] * ta[e] : 0.f;
    cT[e] = cN[e] + (4 * g + e == i ? 1.f : 0.f);  // coef(I + N)
  }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const f32x4 aN2 = mma(cN, aN, z), cN2 = mma(aN, cN, z);
  const f32x4 aN4 = mma(cN2, aN2, z), cN4 = mma(aN2, cN2, z);
  const f32x4 aN8 = mma(cN4, aN4, z);
  cT = mma(aN2, cT, cT);  // coef(T (I + N^2)) = coef(T) + coef(T N^2)
  cT = mma(aN4, cT, cT);
  cT = mma(aN8, cT, cT);
  Blk<T>::store_tri(smem + Y::timg(b) + lane * 16, cT);
}

// The Gram stage.  Waves 0-3 take a diagonal block each (its inverse is the
// critical path) and, in the output sweep, the diagonal P tile; the other
// tiles (the off-diagonal blocks of A and P) go to the other waves (all four
// waves at d = 64, where there are only four), in an order where consecutive
// tiles share their Kh rows.
template <typename T, int D, bool OUT>
__device__ __forceinline__ void gram_stage(unsigned char* smem, int buf, int wave, const Lanes<T, D>& lane) {
  constexpr int NW = D / 16;
  if (wave < 4) {
    diag_block<T, D, OUT>(smem, buf, wave, lane);
    if constexpr (OUT) p_block<T, D>(smem, buf, wave, wave, lane);
  }
  if (NW == 8 && wave < 4) return;
  const int q = NW == 8 ? wave - 4 : wave;  // wave-uniform
  if constexpr (OUT) {
    // A and P of blocks (1,0) (2,0) (3,0) (2,1) (3,1) (3,2), three tiles a wave
    switch (q) {
      case 0: a_block<T, D, OUT>(smem, buf, 1, 0, lane); p_block<T, D>(smem, buf, 1, 0, lane); a_block<T, D, OUT>(smem, buf, 2, 0, lane); break;
      case 1: p_block<T, D>(smem, buf, 2, 0, lane); a_block<T, D, OUT>(smem, buf, 3, 0, lane); p_block<T, D>(smem, buf, 3, 0, lane); break;
      case 2: a_block<T, D, OUT>(smem, buf, 2, 1, lane); p_block<T, D>(smem, buf, 2, 1, lane); a_block<T, D, OUT>(smem, buf, 3, 1, lane); break;
      default: p_block<T, D>(smem, buf, 3, 1, lane); a_block<T, D, OUT>(smem, buf, 3, 2, lane); p_block<T, D>(smem, buf, 3, 2, lane); break;
    }
  } else {
    switch (q) {
      case 0: a_block<T, D, OUT>(smem, buf, 1, 0, lane); a_block<T, D, OUT>(smem, buf, 2, 0, lane); break;
      case 1: a_block<T, D, OUT>(smem, buf, 3, 0, lane); a_block<T, D, OUT>(smem, buf, 2, 1, lane); break;
      case 2: a_block<T, D, OUT>(smem, buf, 3, 1, lane); break;
      default: a_block<T, D, OUT>(smem, buf, 3, 2, lane); break;
    }
  }
}

// ---- the triangular system (I + A) W = diag(beta) [Kt | V] ------------------
// By 16-row blocks, wave w on value columns 16 w .. 16 w + 15 of both halves:
//   W_i = T_ii (beta_i X_i - sum_{m < i} A_im W_m),
// X_i read as accumulator tiles by transpose reads.  Wk goes to LDS
// channel-major (Wk^T, 16 contiguous tokens of a channel per lane: no
// scatter); Wv stays in the wave's registers.
template <typename T, int D, bool OUT>
__device__ __forceinline__ void substitute(unsigned char* smem, int w, const Lanes<T, D>& ln, f32x4 (&Wv)[4]) {
  typedef Lay<T, D, OUT> Y;
  typedef Blk<T> Bk;
  const T* sK = (const T*)(smem + Y::KT);
  const T* sV = (const T*)(smem + Y::VV);
  const float* sB = (const float*)(smem + Y::BETA);
  const int lane = ln.lane, g = lane >> 4;
  f32x4 Wk[4];
  typename Bk::Opnd ok[3], ov[3];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x4 b4 = *(const f32x4*)(sB + 16 * b + 4 * g);
    f32x4 rk = b4 * widen4(colpiece<D>(sK, ln.d, 16 * b, 16 * w));
    f32x4 rv = b4 * widen4(colpiece<D>(sV, ln.d, 16 * b, 16 * w));
#pragma unroll
    for (int m = 0; m < b; ++m) {
      const typename Bk::Coef a = Bk::load(smem + Y::aimg(b, m) + lane * 16);
      rk = Bk::apply(a, ok[m], rk);
      rv = Bk::apply(a, ov[m], rv);
    }
    const typename Bk::Coef t1 = Bk::load(smem + Y::timg(b) + lane * 16);
    const typename Bk::Coef t2 = Bk::TRI2 ? Bk::load(smem + Y::timg(b) + Bk::TRI2 + lane * 16) : t1;
    Wk[b] = Bk::tri(t1, t2, Bk::opnd(rk));
    Wv[b] = Bk::tri(t1, t2, Bk::opnd(rv));
    if (b < 3) {
      ok[b] = Bk::opnd(Wk[b]);
      ov[b] = Bk::opnd(Wv[b]);
    }
  }
  T* sW = (T*)(smem + Y::WKT);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    T* p = sW + ln.c.row + 16 * w * (C + 16) + 16 * b;
    if constexpr (sizeof(T) == 2) *(s16x4*)p = to_bf16x4(Wk[b]);
    else *(f32x4*)p = Wk[b];
  }
}

// ---- the state step ---------------------------------------------------------
// Wave w owns column tile w of the state (rows = D key channels, accumulator
// tiles S[rr]).  The same bf16 fragments of S serve as the right operand of
// Wk S and as the left operand of S^T Qt^T; those of U as the right operand
// of Kh^T U and the left operand of U^T P^T.  The outputs come out transposed
// (O^T tiles: lane (g, i) holds O[token i][4 g .. 4 g + 3] of the wave's
// columns), so each lane stores 4 contiguous elements.
template <typename T, int D>
__device__ __forceinline__ typename Frag<T>::type pfrag(const unsigned char* smem, int rt, int kb, int lane) {
  typedef Lay<T, D, true> Y;
  if constexpr (sizeof(T) == 2) {
    const s16x4 a = *(const s16x4*)(smem + Y::pimg(rt, 2 * kb) + lane * 8);
    const s16x4 b = 2 * kb + 1 <= rt ? *(const s16x4*)(smem + Y::pimg(rt, 2 * kb + 1) + lane * 8)
                                     : (s16x4){0, 0, 0, 0};
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    return *(const f32x4*)(smem + Y::pimg(rt, kb) + lane * 16);
  }
}

// Operand fragments are fetched a row block ahead of their products (two
// register sets), so each group of MFMAs waits for loads issued a group
// earlier rather than for the one just before it.
template <typename T, int D>
__device__ __forceinline__ void state_out(const unsigned char* smem, int buf, f32x4 (&S)[D / 16],
                                          const f32x4 (&Wv)[4], int w, const Lanes<T, D>& ln,
                                          __amdgpu_buffer_rsrc_t ro, int H) {
  typedef Lay<T, D, true> Y;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = Elem<T>::KB, NKD = D / KB, NKC = C / KB, NR = D / 16;
  const T* sQ = (const T*)(smem + Y::qt(buf));
  const T* sH = (const T*)(smem + Y::kh(buf));
  const T* sW = (const T*)(smem + Y::WKT);
  const float* sG = (const float*)(smem + Y::gam(buf));
  const int lane = ln.lane, g = lane >> 4, i = lane & 15;
  FragT SB[NKD];
#pragma unroll
  for (int kb = 0; kb < NKD; ++kb) SB[kb] = Frag<T>::from_acc(S, kb);
  // U = Wv - Wk S
  f32x4 U[4];
  {
    FragT a[2][NKD];
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) a[0][kb] = colfrag<C>(sW, ln.c, kb * KB, 0);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt + 1 < 4) {
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) a[(rt + 1) & 1][kb] = colfrag<C>(sW, ln.c, kb * KB, 16 * (rt + 1));
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) acc = mma(a[rt & 1][kb], SB[kb], acc);
      U[rt] = Wv[rt] - acc;
    }
  }
  FragT UB[NKC];
#pragma unroll
  for (int kb = 0; kb < NKC; ++kb) UB[kb] = Frag<T>::from_acc(U, kb);
  // O^T = S^T Qt^T + U^T P^T, one token tile at a time
  {
    FragT q[2][NKD], pf[2][NKC];
    auto fetch = [&](int rt, FragT (&qq)[NKD], FragT (&pp)[NKC]) {
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) qq[kb] = rowfrag<D>(sQ, ln.d, 16 * rt, kb * KB);
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb)
        if (kb * KB <= 16 * rt + 15) pp[kb] = pfrag<T, D>(smem, rt, kb, lane);
    };
    fetch(0, q[0], pf[0]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt + 1 < 4) fetch(rt + 1, q[(rt + 1) & 1], pf[(rt + 1) & 1]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) acc = mma(SB[kb], q[rt & 1][kb], acc);
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb)
        if (kb * KB <= 16 * rt + 15) acc = mma(UB[kb], pf[rt & 1][kb], acc);
      // rows past the chunk's end fall outside the resource: not written.
      // Write-back stores: a lane writes 4 channels of one token, so the
      // eight waves' pieces of a token's row meet in L2 before it goes to
      // HBM (non-temporal stores sent the 32-byte pieces on their own, 1.65x
      // the bytes of o)
      const uint32_t voff = (uint32_t)((i * H * D + 16 * w + 4 * g) * (int)sizeof(T));
      const int soff = 16 * rt * H * D * (int)sizeof(T);
      if constexpr (sizeof(T) == 2) {
        const uint2 p = __builtin_bit_cast(uint2, to_bf16x4(acc));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, p), ro, voff, soff, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ro, voff, soff, 0);
      }
    }
  }
  // S <- diag(gamma) (S + Kh^T U), two row tiles at a time
  {
    FragT a[2][2][NKC];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) a[0][r][kb] = colfrag<D>(sH, ln.d, kb * KB, 16 * r);
#pragma unroll
    for (int rp = 0; rp < NR / 2; ++rp) {
      if (rp + 1 < NR / 2) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int kb = 0; kb < NKC; ++kb)
            a[(rp + 1) & 1][r][kb] = colfrag<D>(sH, ln.d, kb * KB, 16 * (2 * rp + 2 + r));
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int rr = 2 * rp + r;
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) S[rr] = mma(a[rp & 1][r][kb], UB[kb], S[rr]);
        S[rr] = S[rr] * *(const f32x4*)(sG + 16 * rr + 4 * g);
      }
    }
  }
}

// The map sweep's step: B (from 0) and M (from I, value part of U off).
template <typename T, int D>
__device__ __forceinline__ void state_map(const unsigned char* smem, int buf, f32x4 (&B)[D / 16],
                                          f32x4 (&M)[D / 16], const f32x4 (&Wv)[4], const Lanes<T, D>& ln) {
  typedef Lay<T, D, false> Y;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = Elem<T>::KB, NKD = D / KB, NKC = C / KB, NR = D / 16;
  const T* sH = (const T*)(smem + Y::kh(buf));
  const T* sW = (const T*)(smem + Y::WKT);
  const float* sG = (const float*)(smem + Y::gam(buf));
  const int g = ln.lane >> 4;
  FragT BB[NKD], MB[NKD];
#pragma unroll
  for (int kb = 0; kb < NKD; ++kb) {
    BB[kb] = Frag<T>::from_acc(B, kb);
    MB[kb] = Frag<T>::from_acc(M, kb);
  }
  f32x4 UBt[4], UMt[4];
  {
    FragT a[2][NKD];
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) a[0][kb] = colfrag<C>(sW, ln.c, kb * KB, 0);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt + 1 < 4) {
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) a[(rt + 1) & 1][kb] = colfrag<C>(sW, ln.c, kb * KB, 16 * (rt + 1));
      }
      f32x4 ab = {0.f, 0.f, 0.f, 0.f}, am = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        ab = mma(a[rt & 1][kb], BB[kb], ab);
        am = mma(a[rt & 1][kb], MB[kb], am);
      }
      UBt[rt] = Wv[rt] - ab;
      UMt[rt] = -am;
    }
  }
  FragT UB[NKC], UM[NKC];
#pragma unroll
  for (int kb = 0; kb < NKC; ++kb) {
    UB[kb] = Frag<T>::from_acc(UBt, kb);
    UM[kb] = Frag<T>::from_acc(UMt, kb);
  }
  {
    FragT a[2][NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) a[0][kb] = colfrag<D>(sH, ln.d, kb * KB, 0);
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      if (rr + 1 < NR) {
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) a[(rr + 1) & 1][kb] = colfrag<D>(sH, ln.d, kb * KB, 16 * (rr + 1));
      }
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        B[rr] = mma(a[rr & 1][kb], UB[kb], B[rr]);
        M[rr] = mma(a[rr & 1][kb], UM[kb], M[rr]);
      }
      const f32x4 gm = *(const f32x4*)(sG + 16 * rr + 4 * g);
      B[rr] = B[rr] * gm;
      M[rr] = M[rr] * gm;
    }
  }
}

// The segment map to its record: B from each wave's accumulator tiles, M
// through LDS (sM, [D][D + 4] fp32) into the scan's A-operand fragments.
template <typename T, int D>
__device__ __forceinline__ void save_map(float* sM, float* recs, const f32x4 (&XB)[D / 16], const f32x4 (&XM)[D / 16],
                                         int wave, int lane) {
  typedef Rec<T, D> R;
  constexpr int NR = D / 16, NW = D / 16, LDM = D + 4;
  const int idx = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    *(f32x4*)(recs + R::B + R::tile(rr, wave, lane)) = XB[rr];
#pragma unroll
    for (int e = 0; e < 4; ++e) sM[(16 * rr + 4 * gq + e) * LDM + 16 * wave + idx] = XM[rr][e];
  }
  __syncthreads();
  unsigned char* mf = (unsigned char*)(recs + R::M);
  for (int f = wave; f < NR * R::NKB; f += NW) {
    const int rr = f / R::NKB, kb = f % R::NKB;
    const float* src = sM + (16 * rr + idx) * LDM + R::KB * kb + 4 * gq;
    if constexpr (sizeof(T) == 2) {
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 16);
      const bf16x8 mh = frag_from_acc(lo, hi);
      f32x4 rl, rh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rl[e] = lo[e] - (float)mh[e];
        rh[e] = hi[e] - (float)mh[e + 4];
      }
      *(bf16x8*)(mf + R::frag(rr, kb, 0, lane)) = mh;
      *(bf16x8*)(mf + R::frag(rr, kb, 1, lane)) = frag_from_acc(rl, rh);
    } else {
      *(f32x4*)(mf + R::frag(rr, kb, 0, lane)) = *(const f32x4*)src;
    }
  }
}

// ---- the sweeps -------------------------------------------------------------
// One workgroup per (segment, head); wave w owns value-column tile w.  The
// output sweep (OUT) starts from the segment's S_in (with maps) or h0, writes
// o, the final state (last segment) and, with `states`, the state after
// every `every`-th full chunk of a sequence to its slot (the prefix-cache
// states of kda_chunk_forward_states).  The map sweep starts B from 0 and M
// from I and writes the segment's record; the last segment of a sequence has
// no map and exits.
template <typename T, int D, bool OUT, bool MX>
__global__ void __launch_bounds__(64 * (D / 16))
kda_chunk_sweep(const ChunkInputs in, const int32_t* __restrict__ cu, const int64_t* __restrict__ seqs, int n_rows,
                int T_per, int H, int L, int maps, float g_floor, int gate, float* __restrict__ ws, const float* h0,
                T* __restrict__ o, float* ht, float* __restrict__ states, int every) {
  typedef Lay<T, D, OUT> Y;
  typedef Rec<T, D> R;
  constexpr int NR = D / 16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Y::BYTES];
  const int64_t period = (OUT && states) ? (int64_t)C * every : 0;
  Seg sg;
  if (!locate(cu, seqs, n_rows, T_per, L, period, blockIdx.x, sg)) return;
  if (!OUT && sg.s == sg.nseg - 1) return;
  const int h = blockIdx.y, tid0 = threadIdx.x, lane0 = tid0 & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);  // uniform: scalar control flow
  const int g = lane0 >> 4, i = lane0 & 15;
  const int nch = (sg.len + C - 1) / C, j0 = sg.s * L, j1 = min(j0 + L, nch);
  float* rec = ws + ((size_t)blockIdx.x * H + h) * R::FLOATS;
  // OUT: X[0] = S.  Map sweep: X[0] = B, X[1] = M.
  f32x4 X[OUT ? 1 : 2][NR];
  if (OUT) {
    // uniform branches, so that every load below is unconditional and they
    // all go out before the first wait
    if (maps) {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) X[0][rr] = *(const f32x4*)(rec + R::SIN + R::tile(rr, wave, lane0));
    } else if (h0) {
      const float* h0p = h0 + ((size_t)sg.n * H + h) * D * D + 4 * g * D + 16 * wave + i;
#pragma unroll
      for (int rr = 0; rr < NR; ++rr)
#pragma unroll
        for (int e = 0; e < 4; ++e) X[0][rr][e] = h0p[(16 * rr + e) * D];
    } else {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) X[0][rr] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        X[0][rr][e] = 0.f;
        X[OUT ? 0 : 1][rr][e] = (16 * rr + 4 * g + e == 16 * wave + i) ? 1.f : 0.f;
      }
  }
  auto put_state = [&](float* dst) {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(16 * rr + 4 * g + e) * D + 16 * wave + i] = X[0][rr][e];
  };

  Raw<T, D, OUT, MX, OUT> raw;
  raw.load(in, sg.tok0 + (int64_t)C * j0, min(C, sg.len - C * j0), H, h, tid0, gate);
  // The state step of chunk j - 1 runs in the same barrier interval as the
  // element-wise stage of chunk j (which writes the other buffer set): waves
  // 0-3 take the element-wise stage first, waves 4-7 the state step, so that
  // the two waves sharing a SIMD feed its VALU and its matrix core at once.
  f32x4 Wv[4];
  auto state = [&](int jj, const Lanes<T, D>& ln) {
    const int buf = (jj - j0) & 1;
    if constexpr (OUT) {
      // o rows of the chunk as one buffer resource (rows past its end are not written)
      const int cl = min(C, sg.len - C * jj);
      const __amdgpu_buffer_rsrc_t ro =
          rsrc(o + ((size_t)(sg.tok0 + (int64_t)C * jj) * H + h) * D, ((uint32_t)(cl - 1) * H * D + D) * sizeof(T));
      state_out<T, D>(smem, buf, X[0], Wv, wave, ln, ro, H);
      if (states && (jj + 1) % every == 0 && (int64_t)(jj + 1) * C <= sg.len)
        put_state(states + ((size_t)(sg.slot0 + (jj + 1) / every - 1) * H + h) * D * D);
    } else {
      state_map<T, D>(smem, buf, X[0], X[OUT ? 0 : 1], Wv, ln);
    }
  };
  for (int j = j0; j < j1; ++j) {
    const int64_t tokc = sg.tok0 + (int64_t)C * j;
    const int buf = (j - j0) & 1;
    // thread and lane index as opaque per-chunk values: the LDS addresses
    // derived from them are formed inside the loop, not hoisted and held
    // across it, which would overflow the registers
    int tid = tid0, lane = lane0;
    asm volatile("" : "+v"(tid), "+v"(lane));
    const Lanes<T, D> ln(lane);
    float g0[8], g1[8];
    estage1<T, D, OUT, MX, OUT>(smem, raw, g_floor, gate, tid, g0, g1);
    lds_barrier();  // partial sums visible; the previous chunk's local stages are done
    const bool prev = Y::OVL && j > j0;
    if (prev && wave >= 4) state(j - 1, ln);
    estage2<T, D, OUT, MX, OUT>(smem, buf, raw, tid, g0, g1);
    if (j + 1 < j1) raw.load(in, tokc + C, min(C, sg.len - C * (j + 1)), H, h, tid, gate);
    if (prev && wave < 4) state(j - 1, ln);
    lds_barrier();
    gram_stage<T, D, OUT>(smem, buf, wave, ln);
    lds_barrier();
    substitute<T, D, OUT>(smem, wave, ln, Wv);
    lds_barrier();
    if (!Y::OVL) state(j, ln);
  }
  if (Y::OVL && j1 > j0) state(j1 - 1, Lanes<T, D>(lane0));
  if constexpr (OUT) {
    if (ht && sg.s == sg.nseg - 1) put_state(ht + ((size_t)sg.n * H + h) * D * D);
  } else {
    __syncthreads();  // every wave is done with the last chunk's LDS
    save_map<T, D>((float*)smem, rec, X[0], X[1], wave, lane0);
  }
}

// ---- segment scan S_{s+1} = M_s S_s + B_s -------------------------------------
// Workgroup = (sequence, head, 16 state columns), one wave per 16-row tile of
// S.  Each step a wave publishes its rows as halves of B-operand fragments
// through a double-buffered LDS area and forms the same rows of the next state
// from all k-blocks, so one barrier per step orders the exchange.  M_s and
// B_s do not depend on the state: each wave fetches its rows of them three
// steps ahead.  Without maps (one segment per sequence) the launch only gives
// empty sequences their final state (h0, or zero).
template <typename T, int D> struct ScanOps;
template <int D> struct ScanOps<bf16_t, D> {
  static constexpr int KB = 32, NKB = D / KB;
  // Published state, in B-fragment order: [hi/lo][k-block][lane] 16 bytes,
  // row tile t filling bytes 8 (t % 2) .. 8 (t % 2) + 7 of k-block t / 2.
  typedef uint4 PubArea[2][NKB][64];
  __device__ static __forceinline__ void publish(PubArea& a, int t, int lane, const f32x4& x) {
    const s16x4 h = to_bf16x4(x);
    *((uint2*)&a[0][t >> 1][lane] + (t & 1)) = __builtin_bit_cast(uint2, h);
    *((uint2*)&a[1][t >> 1][lane] + (t & 1)) = __builtin_bit_cast(uint2, to_bf16x4(x - widen4(h)));
  }
  struct SFrag {
    bf16x8 hi, lo;
  };
  __device__ static __forceinline__ SFrag gather(const PubArea& a, int kb, int lane) {
    return SFrag{__builtin_bit_cast(bf16x8, a[0][kb][lane]), __builtin_bit_cast(bf16x8, a[1][kb][lane])};
  }
  struct MRaw {
    bf16x8 hi, lo;
  };
  // k-block kb of this lane's M rows; off: byte offset of its (kb = 0, hi)
  // fragment in the segment record
  __device__ static __forceinline__ MRaw load_m(__amdgpu_buffer_rsrc_t r, uint32_t off, int kb) {
    typedef Rec<bf16_t, D> R;
    MRaw m;
    const uint32_t oh = off + (uint32_t)R::frag(0, kb, 0, 0), ol = off + (uint32_t)R::frag(0, kb, 1, 0);
    m.hi = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, oh, 0, 0));
    m.lo = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, ol, 0, 0));
    return m;
  }
  __device__ static __forceinline__ f32x4 product(const MRaw& m, const SFrag& s, f32x4 acc) {
    acc = mma(m.hi, s.hi, acc);
    acc = mma(m.hi, s.lo, acc);
    return mma(m.lo, s.hi, acc);
  }
};
template <int D> struct ScanOps<float, D> {
  static constexpr int KB = 16, NKB = D / KB;
  typedef f32x4 PubArea[NKB][64];  // row tile t is k-block t
  __device__ static __forceinline__ void publish(PubArea& a, int t, int lane, const f32x4& x) { a[t][lane] = x; }
  typedef f32x4 SFrag;
  __device__ static __forceinline__ SFrag gather(const PubArea& a, int kb, int lane) { return a[kb][lane]; }
  typedef f32x4 MRaw;
  __device__ static __forceinline__ MRaw load_m(__amdgpu_buffer_rsrc_t r, uint32_t off, int kb) {
    const uint32_t o = off + (uint32_t)Rec<float, D>::frag(0, kb, 0, 0);
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
  }
  __device__ static __forceinline__ f32x4 product(const MRaw& m, const SFrag& s, f32x4 acc) { return mma(m, s, acc); }
};

template <typename T, int D>
__global__ void __launch_bounds__(64 * (D / 16))
kda_seg_scan(const float* h0, float* ht, float* __restrict__ ws, const int32_t* __restrict__ cu,
             const int64_t* __restrict__ seqs, int n_rows, int T_per, int H, int L, int maps) {
  typedef ScanOps<T, D> Ops;
  constexpr int NKB = Ops::NKB, WPP = D / 16;
  __shared__ typename Ops::PubArea sS[2];  // published state, double-buffered
  const int n_pairs = n_rows * H;
  // XCD-aware order: the WPP workgroups of one (sequence, head) get ids with
  // the same residue mod 8, so they share one XCD's L2 for M and B.
  const int id = blockIdx.x, xcd = id & 7, jj = id >> 3;
  const int p = (jj / WPP) * 8 + xcd, ct = jj % WPP;
  if (p >= n_pairs) return;
  const int n = p / H, h = p % H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's row tile
  const int lane = threadIdx.x & 63, idx = lane & 15, gq = lane >> 4;
  const int col = 16 * ct + idx;

  int64_t base;
  int len;
  if (cu) {
    base = seqs[n];
    len = cu[n + 1] - cu[n];
  } else {
    base = (int64_t)n * n_segments(T_per, L);
    len = T_per;
  }
  const int nseg = n_segments(len, L);

  f32x4 Sk;
#pragma unroll
  for (int e = 0; e < 4; ++e) Sk[e] = h0 ? h0[((size_t)p * D + 16 * wave + 4 * gq + e) * D + col] : 0.f;
  if (nseg == 0) {
    if (ht) {
      float* dst = ht + (size_t)p * D * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(16 * wave + 4 * gq + e) * D + col] = Sk[e];
    }
    return;
  }
  if (!maps) return;
  typedef Rec<T, D> R;
  auto rec = [&](int s) -> float* { return ws + ((size_t)(base + s) * H + h) * R::FLOATS; };
  auto put = [&](float* dst) { *(f32x4*)(dst + R::tile(wave, ct, lane)) = Sk; };  // accumulator tile order
  put(rec(0) + R::SIN);
  struct Stage {
    typename Ops::MRaw m[NKB];
    f32x4 b;
  };
  // Buffer loads: a step's record is one scalar resource, the lanes' byte
  // offsets into it fixed registers, so the fetches take no per-lane address
  // registers.
  const uint32_t m_off = (uint32_t)(R::M * 4 + R::frag(wave, 0, 0, lane));
  const uint32_t b_off = (uint32_t)((R::B + R::tile(wave, ct, lane)) * 4);
  constexpr uint32_t kRecBytes = (uint32_t)(R::FLOATS * 4);
  auto fetch = [&](int s, Stage& st) {
    const __amdgpu_buffer_rsrc_t r = rsrc(rec(s), kRecBytes);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) st.m[kb] = Ops::load_m(r, m_off, kb);
    st.b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, b_off, 0, 0));
    // issued here, before the step's own temporaries are allocated
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int s, const Stage& st) {
    Ops::publish(sS[s & 1], wave, lane, Sk);
    lds_barrier();  // LDS only: the records fetched ahead stay in flight
    // two accumulators (even and odd k-blocks) keep the MFMA chains short
    f32x4 acc0 = st.b, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const typename Ops::SFrag sf = Ops::gather(sS[s & 1], kb, lane);
      if (kb & 1) acc1 = Ops::product(st.m[kb], sf, acc1);
      else acc0 = Ops::product(st.m[kb], sf, acc0);
    }
    Sk = acc0 + acc1;
    put(rec(s + 1) + R::SIN);
  };
  const int nsteps = nseg - 1;
  if (nsteps == 0) return;
  // Fetches past the last step re-read the last step's record (in bounds,
  // unused): unconditional loads keep the wait counts exact.  A ring of three
  // register stages, unrolled by six.
  auto clamp = [&](int s) { return s < nsteps ? s : nsteps - 1; };
  Stage b0, b1, b2;
  fetch(0, b0);
  fetch(clamp(1), b1);
  for (int s = 0; s < nsteps; s += 6) {
    fetch(clamp(s + 2), b2);
    step(s, b0);
    if (s + 1 >= nsteps) break;
    fetch(clamp(s + 3), b0);
    step(s + 1, b1);
    if (s + 2 >= nsteps) break;
    fetch(clamp(s + 4), b1);
    step(s + 2, b2);
    if (s + 3 >= nsteps) break;
    fetch(clamp(s + 5), b2);
    step(s + 3, b0);
    if (s + 4 >= nsteps) break;
    fetch(clamp(s + 6), b0);
    step(s + 4, b1);
    if (s + 5 >= nsteps) break;
    fetch(clamp(s + 7), b1);
    step(s + 5, b2);
  }
}

// ---- launch ---------------------------------------------------------------------
template <typename T, int D>
int launch_typed(int n_rows, int T_per, int H, const SegPlan& plan, float g_floor, int gate, const ChunkInputs& in,
                 const float* h0, const int32_t* cu, void* o, float* ht, float* states, int every, void* ws,
                 hipStream_t stream, void* const* events) {
  constexpr int NT = 64 * (D / 16);
  const int L = plan.seg_chunks, maps = plan.maps ? 1 : 0;
  float* wsf = (float*)ws;
  int64_t* seqs = cu ? (int64_t*)((unsigned char*)ws + plan.seq_off) : nullptr;
  const int64_t period = states ? (int64_t)C * every : 0;
  const bool mx = in.qs != nullptr;
  if (plan.rec_bytes != Rec<T, D>::FLOATS * sizeof(float)) return (int)hipErrorInvalidValue;
  if (mx && sizeof(T) != 2) return (int)hipErrorInvalidValue;  // MXFP8 inputs: bf16 path only
  hipError_t e;
  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord((hipEvent_t)events[i], stream) : hipSuccess;
  };
  const dim3 sweep_grid((unsigned)plan.n_seg_bound, H), sweep_block(NT);
  if ((e = mark(0)) != hipSuccess) return (int)e;
  if (cu && n_rows > 0 && (e = launch_kernel(kda_fwd_seqs, dim3(1), dim3(256), stream, cu, n_rows, L, period, seqs)) != hipSuccess)
    return (int)e;
  if (maps && plan.n_seg_bound > 0) {
    e = mx ? launch_kernel(kda_chunk_sweep<T, D, false, sizeof(T) == 2>, sweep_grid, sweep_block, stream, in, cu,
                           (const int64_t*)seqs, n_rows, T_per, H, L, maps, g_floor, gate, wsf, h0, (T*)o, ht, states,
                           every)
           : launch_kernel(kda_chunk_sweep<T, D, false, false>, sweep_grid, sweep_block, stream, in, cu,
                           (const int64_t*)seqs, n_rows, T_per, H, L, maps, g_floor, gate, wsf, h0, (T*)o, ht, states,
                           every);
    if (e != hipSuccess) return (int)e;
  }
  if ((e = mark(1)) != hipSuccess) return (int)e;
  if (maps || cu || T_per == 0) {
    const int64_t blocks = ((int64_t)n_rows * H + 7) / 8 * 8 * (D / 16);
    if ((e = launch_kernel(kda_seg_scan<T, D>, dim3((unsigned)blocks), dim3(NT), stream, h0, ht, wsf, cu,
                           (const int64_t*)seqs, n_rows, T_per, H, L, maps)) != hipSuccess)
      return (int)e;
  }
  if ((e = mark(2)) != hipSuccess) return (int)e;
  if (plan.n_seg_bound > 0) {
    e = mx ? launch_kernel(kda_chunk_sweep<T, D, true, sizeof(T) == 2>, sweep_grid, sweep_block, stream, in, cu,
                           (const int64_t*)seqs, n_rows, T_per, H, L, maps, g_floor, gate, wsf, h0, (T*)o, ht, states,
                           every)
           : launch_kernel(kda_chunk_sweep<T, D, true, false>, sweep_grid, sweep_block, stream, in, cu,
                           (const int64_t*)seqs, n_rows, T_per, H, L, maps, g_floor, gate, wsf, h0, (T*)o, ht, states,
                           every);
    if (e != hipSuccess) return (int)e;
  }
  return (int)mark(3);
}

}  // namespace

int scratch_buffer(void** ptr) {
  constexpr int kMaxDevices = 256;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: its copy
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return (int)hipSuccess;
}

int device_compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

int launch_chunk_forward(int is_bf16, int d, int n_rows, int T, int H, const SegPlan& plan, float g_floor,
                         int gate, const ChunkInputs& in, const float* h0, const int32_t* cu, void* o, float* ht,
                         float* states, int every, void* ws, void* stream, void* const* events) {
  hipStream_t s = (hipStream_t)stream;
  if (is_bf16 && d == 64)
    return launch_typed<bf16_t, 64>(n_rows, T, H, plan, g_floor, gate, in, h0, cu, o, ht, states, every, ws, s,
                                    events);
  if (is_bf16 && d == 128)
    return launch_typed<bf16_t, 128>(n_rows, T, H, plan, g_floor, gate, in, h0, cu, o, ht, states, every, ws, s,
                                     events);
  if (!is_bf16 && d == 64)
    return launch_typed<float, 64>(n_rows, T, H, plan, g_floor, gate, in, h0, cu, o, ht, states, every, ws, s,
                                   events);
  return (int)hipErrorInvalidValue;
}

}  // namespace kda
