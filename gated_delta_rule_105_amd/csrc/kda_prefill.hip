// Chunked KDA forward for gfx950: two chunk passes around a segment scan.
//
// Chunk algebra (per sequence and head; chunk rows r = 0..63, S the state
// entering the chunk, g floored, G = running sum of g over the chunk's rows,
// G_L its last row, gamma = e^{G_L} per key channel):
//   Qt = Q e^{G},  Kt = K e^{G},  Kh = K e^{-G}
//   A  = diag(beta) strict_lower(Kt Kh^T),   T = (I + A)^{-1}
//   Wk = T diag(beta) Kt,   Wv = T diag(beta) V,   P = lower_incl(Qt Kh^T)
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
// into segments of L chunks; the composition of a segment's maps is again
// affine, S_out = M S_in + B.  Three launches:
//   1. kda_chunk_prep (one workgroup per (segment, head), all in parallel):
//      the chunk-local part of each chunk (decay prefix sums, Gram blocks,
//      the inverse (I + A)^{-1}, Wk and Wv) from the inputs, written to a
//      per-chunk record: Qt, Wk, Kh^T, P and gamma as an image of the output
//      pass's LDS, and Wv.  The same workgroup runs each chunk, while its
//      operands are still in LDS, on the state started from 0 (giving B) and
//      from I with the value part of U switched off (giving M), and writes the
//      segment's map; the last segment of a sequence has none (no later
//      segment needs it).  When every sequence is one segment there are no
//      maps, and the chunks are grouped by a length of the pass's own.
//   2. kda_seg_scan (one workgroup per (sequence, head, 16 state columns)):
//      S_0 = h0, S_{s+1} = M_s S_s + B_s, writing every segment's incoming
//      state.  M S is done as three bf16 products of a hi/lo split of both
//      factors (about fp32 accuracy).
//   3. kda_seg_forward (one workgroup per (segment, head), all in parallel):
//      the state recurrence from the segment's incoming state over its chunk
//      records, writing o and, for the last segment, the final state.  It
//      keeps two record images in LDS (about 57 KiB each at d = 128): the
//      next chunk's image lands by direct global-to-LDS loads while the
//      current one is used.
// Within a workgroup, wave w owns 16 value columns of the state: columns of
// U, O and S never mix, so the state products need no exchange.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

#ifndef KDA_NW128
#define KDA_NW128 8
#endif
#ifndef KDA_NW128_FWD
#define KDA_NW128_FWD 4
#endif

namespace kda {
namespace {

constexpr int C = kChunk;

// Streaming accesses: the chunk inputs are read once and o is written once,
// and the chunk records are read back once per state pass; non-temporal
// hints keep them from displacing cached data.  (The record stores stay
// ordinary: a short workload's records are read back from cache.)
typedef uint32_t u32x4nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 stream_load16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4nt*)p));
}
__device__ __forceinline__ void stream_store16(void* p, const uint4& x) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4nt, x), (u32x4nt*)p);
}

// ---- LDS layout of the chunk engine -------------------------------------
template <typename T, int D> struct Lds {
  static constexpr int PADT = 16 / (int)sizeof(T);
  static constexpr int LDT = D + PADT;  // token-major arrays [64][LDT]
  static constexpr int LDC = C + PADT;  // channel-major arrays [D][LDC]; P [64][LDC]
  static constexpr int LDF = C + 4;     // fp32 [64][LDF]
  static constexpr int ROW_T = C * LDT * (int)sizeof(T);
  static constexpr int ROW_F = C * LDF * 4;
  static constexpr int ROW = ((ROW_T > ROW_F ? ROW_T : ROW_F) + 15) / 16 * 16;
  static constexpr int COL = (D * LDC * (int)sizeof(T) + 15) / 16 * 16;
  static constexpr int PSZ = (C * LDC * (int)sizeof(T) + 15) / 16 * 16;
  static constexpr int Q = 0;              // q, then Qt
  static constexpr int K = ROW;            // k, then Kt, then Wk
  static constexpr int G = 2 * ROW;        // g, then Kh, then T (fp32)
  static constexpr int V = 3 * ROW;        // v, then A (fp32)
  static constexpr int KT = 4 * ROW;       // Kt^T
  static constexpr int KH = KT + COL;      // Kh^T
  static constexpr int VT = KH + COL;      // V^T
  static constexpr int P = VT + COL;       // P
  static constexpr int BETA = P + PSZ;     // fp32 [64]
  static constexpr int PART = BETA + C * 4;  // fp32 [8][D] partial sums of g
  static constexpr int GL = PART + 8 * D * 4;  // fp32 [D] gamma
  static constexpr int TII = GL + D * 4;       // fp32 [4][16][16] diagonal-block inverses
  static constexpr int BYTES = TII + 4 * 16 * 16 * 4;
};

// ---- sequences and segments ---------------------------------------------
__device__ __forceinline__ int n_segments(int len, int L) { return ((len + C - 1) / C + L - 1) / L; }

struct Seg {
  int64_t tok0;    // first packed token of the sequence
  int64_t chunk0;  // chunks of all earlier sequences (first chunk-record slot)
  int len;         // tokens of the sequence
  int n;           // sequence
  int s;           // segment within the sequence
  int nseg;        // segments of the sequence
};

// Global segment gs -> its sequence.  false when gs is past the last one.
__device__ __forceinline__ bool locate(const int32_t* cu, int n_rows, int T, int L, int64_t gs, Seg& r) {
  if (!cu) {
    const int per = n_segments(T, L);
    if (per == 0) return false;
    const int64_t n = gs / per;
    if (n >= n_rows) return false;
    r.n = (int)n;
    r.s = (int)(gs % per);
    r.nseg = per;
    r.tok0 = n * (int64_t)T;
    r.chunk0 = n * (int64_t)((T + C - 1) / C);
    r.len = T;
    return true;
  }
  int64_t base = 0, chunks = 0;
  for (int n = 0; n < n_rows; ++n) {
    const int len = cu[n + 1] - cu[n];
    const int ns = n_segments(len, L);
    if (gs < base + ns) {
      r.n = n;
      r.s = (int)(gs - base);
      r.nseg = ns;
      r.tok0 = cu[n];
      r.chunk0 = chunks;
      r.len = len;
      return true;
    }
    base += ns;
    chunks += (len + C - 1) / C;
  }
  return false;
}

// ---- workspace record of one (segment, head): three d x d blocks of fp32 size
//   B    : [d/16 row tiles][d/16 column tiles][64 lanes][4] fp32, accumulator
//          tile order (lane 16 g + i holds rows 4 g .. 4 g + 3 of column i)
//   M    : A-operand fragments of M for the scan, [d/16 row tiles][k-blocks]
//          [64 lanes][16 bytes]; bf16 keeps a hi and a lo fragment per slot
//          (M = hi + lo to about 2^-17), fp32 keeps M itself
//   S_in : incoming state of the segment, accumulator tile order like B
template <typename T, int D> struct Rec {
  static constexpr int NRT = D / 16, KB = Elem<T>::KB, NKB = D / KB;
  static constexpr size_t B = 0, M = (size_t)D * D, SIN = 2 * (size_t)D * D, FLOATS = 3 * (size_t)D * D;
  // float offset of accumulator tile (rr, ct) in a tile-ordered block
  __device__ static __forceinline__ size_t tile(int rr, int ct, int lane) {
    return (((size_t)rr * NRT + ct) * 64 + lane) * 4;
  }
  // byte offset of the (rr, kb) fragment (part 0 = hi, 1 = lo for bf16)
  __device__ static __forceinline__ size_t frag(int rr, int kb, int part, int lane) {
    return ((((size_t)rr * NKB + kb) * (sizeof(T) == 2 ? 2 : 1) + part) * 64 + lane) * 16;
  }
};

// one element replicated over a 16-byte piece
__device__ __forceinline__ uint4 splat16(bf16_t x) {
  const uint32_t u = (uint32_t)x | ((uint32_t)x << 16);
  return (uint4){u, u, u, u};
}
__device__ __forceinline__ uint4 splat16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint4){u, u, u, u};
}

// ---- raw chunk inputs: global -> registers (prefetch) -> LDS -------------
// 8 e4m3 bytes (OCP, finite-only) times their block's scale 2^(s - 127),
// as 8 bf16 (exact: e4m3 has 3 significand bits, bf16 8; the gfx950
// conversion takes the scale as an fp32 multiplier)
__device__ __forceinline__ uint4 mx_decode8(const uint2& w, uint32_t s) {
  const float sc = __uint_as_float(s ? s << 23 : 0x00400000u);
  return (uint4){__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, sc, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, sc, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, sc, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, sc, true))};
}

// With MX, q, k and v arrive as e4m3 bytes with a scale byte per 32
// channels: each thread loads 16 bytes (16 channels of one token, inside one
// scale block) and their scale per tensor, decoded to two 16-byte vectors
// of bf16 when they are stored to LDS; everything after that is the bf16
// path.
template <typename T, int D, int NT, bool WITH_Q, bool MX = false> struct Raw {
  typedef Lds<T, D> M;
  static constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int VPR = D / EPV;              // vectors per token row
  static constexpr int PER = C * VPR / NT;         // vectors per thread per tensor
  static_assert(PER * NT == C * VPR, "thread count must divide the chunk");
  static_assert(!MX || (sizeof(T) == 2 && D % 32 == 0), "MXFP8 inputs feed the bf16 path");
  static constexpr int NB = MX ? 1 : PER;
  static constexpr int TPR = D / 16;  // MX: threads per token row (16 channels each)
  static_assert(!MX || C * TPR == NT, "MX: one 16-byte load per thread and tensor");
  uint4 q[WITH_Q ? NB : 1], k[NB], v[NB], g[PER];  // MX: q[0], k[0], v[0] hold e4m3 bytes
  uint32_t qs, ks, vs;                              // MX: their scale bytes
  float beta;

  // Rows past the chunk's end (a sequence's last chunk) are loaded as zeros
  // (beta and g of such rows must be 0; their q, k and v then reach no
  // output).  The buffer is scoped to one chunk iteration.  load = load_qkg
  // (q, k, g and beta) + load_v, which may be issued at different times.
  // gate: g per channel (16-byte pieces like q), one per (token, head)
  // replicated over the channels, or none (zeros: no decay).
  __device__ __forceinline__ void load_qkg(const ChunkInputs& in, int64_t tok0, int len, int H, int h, int tid,
                                           int gate) {
    const T* G = (const T*)in.g;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int vi = tid + j * NT, t = vi / VPR, cv = vi % VPR;
      const uint4 z = {0u, 0u, 0u, 0u};
      if (t < len) {
        const size_t off = ((size_t)(tok0 + t) * H + h) * D + cv * EPV;  // element index
        if (!MX) {
          if (WITH_Q) q[j] = stream_load16((const T*)in.q + off);
          k[j] = stream_load16((const T*)in.k + off);
        }
        g[j] = gate == kGateChannel ? stream_load16(G + off)
               : gate == kGateHead  ? splat16(G[(size_t)(tok0 + t) * H + h])
                                    : z;
      } else {
        if (!MX) {
          if (WITH_Q) q[j] = z;
          k[j] = z;
        }
        g[j] = z;
      }
    }
    if (MX) {
      const int t = tid / TPR;
      const size_t off = ((size_t)(tok0 + t) * H + h) * D + (tid % TPR) * 16;  // element (= byte) index
      const bool in_seq = t < len;
      if (WITH_Q) {
        q[0] = in_seq ? stream_load16((const uint8_t*)in.q + off) : (uint4){0u, 0u, 0u, 0u};
        qs = in_seq ? in.qs[off / 32] : 127u;
      }
      k[0] = in_seq ? stream_load16((const uint8_t*)in.k + off) : (uint4){0u, 0u, 0u, 0u};
      ks = in_seq ? in.ks[off / 32] : 127u;
    }
    beta = (tid < len) ? in.beta[(size_t)(tok0 + tid) * H + h] : 0.f;
  }
  __device__ __forceinline__ void load_v(const ChunkInputs& in, int64_t tok0, int len, int H, int h, int tid) {
    if (MX) {
      const int t = tid / TPR;
      const size_t off = ((size_t)(tok0 + t) * H + h) * D + (tid % TPR) * 16;
      v[0] = t < len ? stream_load16((const uint8_t*)in.v + off) : (uint4){0u, 0u, 0u, 0u};
      vs = t < len ? in.vs[off / 32] : 127u;
      return;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int vi = tid + j * NT, t = vi / VPR, cv = vi % VPR;
      v[j] = t < len ? stream_load16((const T*)in.v + ((size_t)(tok0 + t) * H + h) * D + cv * EPV)
                     : (uint4){0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void load(const ChunkInputs& in, int64_t tok0, int len, int H, int h, int tid,
                                       int gate) {
    load_qkg(in, tok0, len, H, h, tid, gate);
    load_v(in, tok0, len, H, h, tid);
  }
  // MX: 16 e4m3 bytes and their scale -> channels (tid % TPR) * 16 .. + 15 of
  // token tid / TPR, two bf16 vectors in the token-major array at `area`
  __device__ __forceinline__ static void store_mx(unsigned char* smem, int area, int tid, const uint4& b,
                                                  uint32_t s) {
    unsigned char* p = smem + area + (tid / TPR) * M::LDT * 2 + (tid % TPR) * 32;
    *(uint4*)p = mx_decode8((uint2){b.x, b.y}, s);
    *(uint4*)(p + 16) = mx_decode8((uint2){b.z, b.w}, s);
  }

  // into LDS: everything but v (store_qkg), v (store_v), or both (store)
  __device__ __forceinline__ void store_qkg(unsigned char* smem, int tid) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int vi = tid + j * NT, t = vi / VPR, cv = vi % VPR;
      const int off = t * M::LDT * (int)sizeof(T) + cv * 16;
      if (!MX) {
        if (WITH_Q) *(uint4*)(smem + M::Q + off) = q[j];
        *(uint4*)(smem + M::K + off) = k[j];
      }
      *(uint4*)(smem + M::G + off) = g[j];
    }
    if (MX) {
      if (WITH_Q) store_mx(smem, M::Q, tid, q[0], qs);
      store_mx(smem, M::K, tid, k[0], ks);
    }
    if (tid < C) ((float*)(smem + M::BETA))[tid] = beta;
  }
  __device__ __forceinline__ void store_v(unsigned char* smem, int tid) const {
    if (MX) {
      store_mx(smem, M::V, tid, v[0], vs);
      return;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int vi = tid + j * NT, t = vi / VPR, cv = vi % VPR;
      *(uint4*)(smem + M::V + t * M::LDT * (int)sizeof(T) + cv * 16) = v[j];
    }
  }
  __device__ __forceinline__ void store(unsigned char* smem, int tid) const {
    store_qkg(smem, tid);
    store_v(smem, tid);
  }

  // Chunk output [64][LDT] staged in LDS -> o rows tok0 .. tok0 + clen - 1.
  __device__ __forceinline__ static void store_out(const unsigned char* stage, T* o, int64_t tok0, int clen, int H,
                                                   int h, int tid) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int vi = tid + j * NT, t = vi / VPR, cv = vi % VPR;
      if (t < clen)
        stream_store16(o + ((size_t)(tok0 + t) * H + h) * D + cv * EPV,
                       *(const uint4*)(stage + t * M::LDT * (int)sizeof(T) + cv * 16));
    }
  }
};

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return Elem<T>::to_f32(x); }

// ---- element-wise stage: prefix sums of the floored log-decay and the
// decay-scaled operands.  Thread (channel pair c, c + 1; part p) owns TPP
// consecutive rows of its two channels; the parts exchange their sums through
// LDS.  Rows are processed in blocks of 8 whose LDS reads are issued together.
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
  typedef uint32_t word;  // two bf16 channels
  __device__ static __forceinline__ float lo(word w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(word w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static __forceinline__ word pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(a, b));
  }
};
template <> struct Pair<float> {
  typedef f32x2 word;
  __device__ static __forceinline__ float lo(word w) { return w[0]; }
  __device__ static __forceinline__ float hi(word w) { return w[1]; }
  __device__ static __forceinline__ word pack(float a, float b) { return (f32x2){a, b}; }
};

// Channel-major store of 8 consecutive rows of a channel pair, given the 8
// token-major pair words: channel c gets the low halves, c + 1 the high ones.
__device__ __forceinline__ void store_cols8(bf16_t* dst, int ldc, const uint32_t (&w)[8]) {
  uint32_t a[4], b[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    a[u] = (w[2 * u] & 0xffffu) | (w[2 * u + 1] << 16);
    b[u] = (w[2 * u] >> 16) | (w[2 * u + 1] & 0xffff0000u);
  }
  *(uint4*)dst = (uint4){a[0], a[1], a[2], a[3]};
  *(uint4*)(dst + ldc) = (uint4){b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store_cols8(float* dst, int ldc, const f32x2 (&w)[8]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    *(f32x4*)(dst + 4 * u) = (f32x4){w[4 * u][0], w[4 * u + 1][0], w[4 * u + 2][0], w[4 * u + 3][0]};
    *(f32x4*)(dst + ldc + 4 * u) = (f32x4){w[4 * u][1], w[4 * u + 1][1], w[4 * u + 2][1], w[4 * u + 3][1]};
  }
}

template <typename T, int D, int NW, bool WITH_Q>
__device__ __forceinline__ void elementwise(unsigned char* smem, float g_floor, int tid) {
  typedef Lds<T, D> M;
  typedef Pair<T> PW;
  typedef typename PW::word word;
  constexpr int LDT = M::LDT, LDC = M::LDC;
  constexpr int NT = 64 * NW, NPR = D / 2, NP = NT / NPR, TPP = C / NP;
  static_assert(NP * NPR == NT && NP * TPP == C && NP <= 8 && TPP % 8 == 0, "thread layout");
  word* sQ = (word*)(smem + M::Q);
  word* sK = (word*)(smem + M::K);
  word* sG = (word*)(smem + M::G);
  const word* sV = (const word*)(smem + M::V);
  T* sKT = (T*)(smem + M::KT);
  T* sKH = (T*)(smem + M::KH);
  T* sVT = (T*)(smem + M::VT);
  float* sPart = (float*)(smem + M::PART);
  float* sGL = (float*)(smem + M::GL);
  const int cp = tid % NPR, c = 2 * cp, part = tid / NPR, t0 = TPP * part;
  auto at = [&](int t) { return t * (LDT / 2) + cp; };  // pair index of (row t, channel c)

  // decays in log2 units, so that every factor is one v_exp_f32 (exp2)
  constexpr float kLog2e = 1.4426950408889634f;
  float g0[TPP], g1[TPP];
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int s = 0; s < TPP; ++s) {
    const word w = sG[at(t0 + s)];
    const float x0 = PW::lo(w), x1 = PW::hi(w);
    g0[s] = (x0 < g_floor ? g_floor : x0) * kLog2e;  // NaN stays NaN
    g1[s] = (x1 < g_floor ? g_floor : x1) * kLog2e;
    p0 += g0[s];
    p1 += g1[s];
  }
  *(f32x2*)(sPart + part * D + c) = (f32x2){p0, p1};
  __syncthreads();
  float gam0 = 0.f, gam1 = 0.f, gl0 = 0.f, gl1 = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const f32x2 x = *(const f32x2*)(sPart + p * D + c);
    gam0 += p < part ? x[0] : 0.f;
    gam1 += p < part ? x[1] : 0.f;
    gl0 += x[0];
    gl1 += x[1];
  }
  if (part == 0) *(f32x2*)(sGL + c) = (f32x2){__builtin_amdgcn_exp2f(gl0), __builtin_amdgcn_exp2f(gl1)};

#pragma unroll
  for (int b0 = 0; b0 < TPP; b0 += 8) {
    const int tb = t0 + b0;
    word kw[8], qw[8], vw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kw[s] = sK[at(tb + s)];
      vw[s] = sV[at(tb + s)];
      if (WITH_Q) qw[s] = sQ[at(tb + s)];
    }
    word kt[8], kh[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      gam0 += g0[b0 + s];
      gam1 += g1[b0 + s];
      const float e0 = __builtin_amdgcn_exp2f(gam0), e1 = __builtin_amdgcn_exp2f(gam1);
      const float ei0 = __builtin_amdgcn_exp2f(-gam0), ei1 = __builtin_amdgcn_exp2f(-gam1);
      const float k0 = PW::lo(kw[s]), k1 = PW::hi(kw[s]);
      kt[s] = PW::pack(k0 * e0, k1 * e1);
      kh[s] = PW::pack(k0 * ei0, k1 * ei1);
      sK[at(tb + s)] = kt[s];
      sG[at(tb + s)] = kh[s];
      if (WITH_Q) sQ[at(tb + s)] = PW::pack(PW::lo(qw[s]) * e0, PW::hi(qw[s]) * e1);
    }
    store_cols8(sKT + c * LDC + tb, LDC, kt);
    store_cols8(sKH + c * LDC + tb, LDC, kh);
    store_cols8(sVT + c * LDC + tb, LDC, vw);
  }
  __syncthreads();
}

// (I + A_bb)^{-1} for diagonal block b (16 x 16, unit lower triangular) by
// fp32 forward substitution, lane idx solving column idx; written to
// sTii[b][16][16].  Called by the wave that has just written row tile b of A
// (its own LDS writes are visible to its later reads).
template <int LDF>
__device__ __forceinline__ void diag_inverse(const float* sA, float* sTii, int b, int lane) {
  const int idx = lane & 15, b0 = 16 * b;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float acc = (r == idx) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < r; ++m) acc -= sA[(b0 + r) * LDF + b0 + m] * x[m];
    x[r] = acc;
  }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sTii[(b * 16 + r) * 16 + idx] = x[r];
  }
}

// ---- Gram blocks: A = diag(beta) strict_lower(Kt Kh^T) (fp32) and
// P = lower_incl(Qt Kh^T) (operand type), as 16 x 16 tiles on and below the
// diagonal, each one MMA chain over the key channels: rows from Kt (A) or Qt
// (P), columns from Kh.  Four waves: wave w takes row tile w of A and row
// tile 3 - w of P (five tiles each; every Kh fragment it loads serves the A
// and the P tile of its column).  Eight waves: waves 0-3 take the diagonal
// tiles (b, b) of A and P, waves 4-7 three of the twelve others each, in an
// order where consecutive tiles mostly share their column.  Of the upper P
// tiles only (0, 1) and (2, 3) share a 32-wide k-block with needed ones; they
// are zeroed (bf16 path).  A's upper tiles are never read.
// Eight-wave tile lists, wave w's tile t in byte w of kGram8[t]: bit 6 set for
// a tile (clear: the list has ended), bit 4 P (else A), bits 2-3 the row
// tile, bits 0-1 the column tile.  Immediate operands, taken apart with
// scalar shifts (a table in memory would be read by vector loads, which wait
// behind the prefetch of the next chunk's inputs).
constexpr uint64_t gram_code(int p, int r, int c) { return (uint64_t)(64 | 16 * p | 4 * r | c); }
constexpr uint64_t gram_list(const int (&x)[8][3]) {
  uint64_t v = 0;
  for (int w = 0; w < 8; ++w)
    if (x[w][0] >= 0) v |= gram_code(x[w][0], x[w][1], x[w][2]) << (8 * w);
  return v;
}
constexpr int kGramT0[8][3] = {{0, 0, 0}, {0, 1, 1}, {0, 2, 2}, {0, 3, 3}, {0, 1, 0}, {1, 2, 0}, {0, 2, 1}, {1, 3, 1}};
constexpr int kGramT1[8][3] = {{1, 0, 0}, {1, 1, 1}, {1, 2, 2}, {1, 3, 3}, {1, 1, 0}, {0, 3, 0}, {1, 2, 1}, {0, 3, 2}};
constexpr int kGramT2[8][3] = {{-1, 0, 0}, {-1, 0, 0}, {-1, 0, 0}, {-1, 0, 0},
                               {0, 2, 0},  {1, 3, 0},  {0, 3, 1},  {1, 3, 2}};
constexpr uint64_t kGram8[3] = {gram_list(kGramT0), gram_list(kGramT1), gram_list(kGramT2)};

template <typename T, int D>
__device__ __forceinline__ void gram_store(unsigned char* smem, bool is_p, int r, int c, const f32x4& acc,
                                           int lane) {
  typedef Lds<T, D> M;
  const int idx = lane & 15, gq = lane >> 4, s = 16 * c + idx;
  if (!is_p) {
    float* sA = (float*)(smem + M::V);
    const float* sBeta = (const float*)(smem + M::BETA);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * r + 4 * gq + i;
      sA[row * M::LDF + s] = s < row ? sBeta[row] * acc[i] : 0.f;
    }
  } else {
    T* sP = (T*)(smem + M::P);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * r + 4 * gq + i;
      sP[row * M::LDC + s] = Elem<T>::from_f32(s <= row ? acc[i] : 0.f);
    }
  }
}

template <typename T, int D, int NW, bool WITH_P>
__device__ __forceinline__ void gram(unsigned char* smem, int wave, int lane) {
  typedef Lds<T, D> M;
  typedef typename Frag<T>::type FragT;
  static_assert(NW == 4 || NW == 8, "Gram tiles over four or eight waves");
  static_assert(NW == 4 || WITH_P, "the eight-wave split includes P");
  constexpr int KB = Elem<T>::KB, NKD = D / KB, LDT = M::LDT, LDC = M::LDC, LDF = M::LDF;
  const T* sQ = (const T*)(smem + M::Q);
  const T* sK = (const T*)(smem + M::K);
  const T* sG = (const T*)(smem + M::G);
  T* sP = (T*)(smem + M::P);
  const int idx = lane & 15, gq = lane >> 4;
  if constexpr (NW == 8) {
    FragT fb[NKD];
    int cprev = -1;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int code = (int)(kGram8[t] >> (8 * wave)) & 0xff;  // wave-uniform
      if (!(code & 64)) break;
      const bool is_p = code & 16;
      const int r = (code >> 2) & 3, c = code & 3;
      if (c != cprev) {
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) fb[kb] = frag_rows(sG, LDT, 16 * c + idx, kb * KB, gq);
        cprev = c;
      }
      const T* src = is_p ? sQ : sK;
      FragT fr[NKD];
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) fr[kb] = frag_rows(src, LDT, 16 * r + idx, kb * KB, gq);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) acc = mma(fr[kb], fb[kb], acc);
      gram_store<T, D>(smem, is_p, r, c, acc, lane);
    }
    if (KB == 32 && (wave == 0 || wave == 2)) {
      // P tile (0, 1) from wave 0, tile (2, 3) from wave 2
#pragma unroll
      for (int i = 0; i < 4; ++i) sP[(16 * wave + 4 * gq + i) * LDC + 16 * wave + 16 + idx] = Elem<T>::from_f32(0.f);
    }
    // the diagonal block of A just written, by the same wave
    if (wave < 4) diag_inverse<LDF>((const float*)(smem + M::V), (float*)(smem + M::TII), wave, lane);
  } else {
    const int rA = wave, rP = 3 - wave;  // wave-uniform
    FragT fa[NKD], fq[NKD];
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      fa[kb] = frag_rows(sK, LDT, 16 * rA + idx, kb * KB, gq);
      if (WITH_P) fq[kb] = frag_rows(sQ, LDT, 16 * rP + idx, kb * KB, gq);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bool doA = ct <= rA, doP = WITH_P && ct <= rP;
      if (doA || doP) {
        FragT fb[NKD];
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) fb[kb] = frag_rows(sG, LDT, 16 * ct + idx, kb * KB, gq);
        if (doA) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKD; ++kb) acc = mma(fa[kb], fb[kb], acc);
          gram_store<T, D>(smem, false, rA, ct, acc, lane);
        }
        if (doP) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKD; ++kb) acc = mma(fq[kb], fb[kb], acc);
          gram_store<T, D>(smem, true, rP, ct, acc, lane);
        }
      }
    }
    if (WITH_P && KB == 32 && (rP == 0 || rP == 2)) {
      // P tile (0, 1) from the wave with rP = 0, tile (2, 3) from rP = 2
#pragma unroll
      for (int i = 0; i < 4; ++i) sP[(16 * rP + 4 * gq + i) * LDC + 16 * rP + 16 + idx] = Elem<T>::from_f32(0.f);
    }
    diag_inverse<LDF>((const float*)(smem + M::V), (float*)(smem + M::TII), rA, lane);
  }
  __syncthreads();
}

// ---- the inverse (I + A)^{-1} and the WY products -----------------------
// Tp = (I + A)^{-1} diag(beta) (64 x 64, lower triangular) is formed once per
// chunk, by 16-column blocks: wave j < 4 takes column block j,
//   Tp_jj = T_jj diag(beta_j),   Tp_ij = -T_ii sum_{m=j}^{i-1} A_im Tp_mj  (i > j),
// with the diagonal inverses T_ii = (I + A_ii)^{-1} from fp32 forward
// substitution.  The 16 x 16 x 16 products take A_im and T_ii rounded to bf16
// and Tp_mj as a hi/lo bf16 pair (fp32 path: fp32 MFMA), accumulating in
// fp32.  Tp goes to LDS as a hi and a lo bf16 array (fp32 path: one fp32
// array), zeros above the diagonal.  Then
//   Wk = Tp Kt,   Wv = Tp V
// are plain MFMA products whose right-hand operands are the chunk operands
// themselves (exact in bf16): only Tp needs the two-term split.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 to_bf16x4(const f32x4& x) {
  const uint32_t a = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[0], x[1]));
  const uint32_t b = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[2], x[3]));
  return __builtin_bit_cast(s16x4, (uint2){a, b});
}
__device__ __forceinline__ f32x4 from_bf16x4(const s16x4& h) {
  const uint2 w = __builtin_bit_cast(uint2, h);
  return (f32x4){__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xffff0000u)};
}

// c + a b over k = 16 for one 16 x 16 tile: a is a coefficient fragment (row
// idx, k = 4 g .. 4 g + 3), b an accumulator tile whose rows run over k,
// prepared once as an operand (Opnd) and used by every product it enters.
template <typename T> struct Sub;
template <> struct Sub<bf16_t> {
  typedef s16x4 Coef;
  struct Opnd { s16x4 hi, lo; };
  __device__ static __forceinline__ Coef coef(const float* p, bool neg) {
    const f32x4 v = *(const f32x4*)p;
    return to_bf16x4(neg ? -v : v);
  }
  __device__ static __forceinline__ Opnd opnd(const f32x4& b) {
    Opnd o;
    o.hi = to_bf16x4(b);
    o.lo = to_bf16x4(b - from_bf16x4(o.hi));
    return o;
  }
  __device__ static __forceinline__ f32x4 apply(const Coef& a, const Opnd& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b.hi, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b.lo, c, 0, 0, 0);
  }
};
template <> struct Sub<float> {
  typedef f32x4 Coef;
  typedef f32x4 Opnd;
  __device__ static __forceinline__ Coef coef(const float* p, bool neg) {
    const f32x4 v = *(const f32x4*)p;
    return neg ? -v : v;
  }
  __device__ static __forceinline__ Opnd opnd(const f32x4& b) { return b; }
  __device__ static __forceinline__ f32x4 apply(const Coef& a, const Opnd& b, f32x4 c) { return mma(a, b, c); }
};

// Tp in the K area (free after the Gram blocks): rows of LD elements; bf16
// keeps Tp = hi + lo in two arrays.
template <typename T, int D> struct TpArea {
  static constexpr int LD = C + 4;
  static constexpr int HI = Lds<T, D>::K;
  static constexpr int LO = HI + C * LD * (int)sizeof(T);
  static_assert((sizeof(T) == 2 ? 2 : 1) * C * LD * sizeof(T) <= (size_t)Lds<T, D>::ROW, "Tp fits the K area");
};

// tile (i, j) of Tp (accumulator layout) into the Tp area
template <typename T, int D>
__device__ __forceinline__ void store_tp(unsigned char* smem, const f32x4& w, int i, int j, int lane) {
  typedef TpArea<T, D> TP;
  const int idx = lane & 15, gq = lane >> 4;
  const int off = (16 * i + 4 * gq) * TP::LD + 16 * j + idx;
  if constexpr (sizeof(T) == 2) {
    const s16x4 hi = to_bf16x4(w);
    const uint2 h = __builtin_bit_cast(uint2, hi);
    const uint2 l = __builtin_bit_cast(uint2, to_bf16x4(w - from_bf16x4(hi)));
    bf16_t* ph = (bf16_t*)(smem + TP::HI) + off;
    bf16_t* pl = (bf16_t*)(smem + TP::LO) + off;
    ph[0] = (bf16_t)(h.x & 0xffffu);
    ph[TP::LD] = (bf16_t)(h.x >> 16);
    ph[2 * TP::LD] = (bf16_t)(h.y & 0xffffu);
    ph[3 * TP::LD] = (bf16_t)(h.y >> 16);
    pl[0] = (bf16_t)(l.x & 0xffffu);
    pl[TP::LD] = (bf16_t)(l.x >> 16);
    pl[2 * TP::LD] = (bf16_t)(l.y & 0xffffu);
    pl[3 * TP::LD] = (bf16_t)(l.y >> 16);
  } else {
    float* p = (float*)(smem + TP::HI) + off;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e * TP::LD] = w[e];
  }
}

// Column block j = wave (< 4) of Tp into the Tp area.  Reads A (V area) and
// the diagonal inverses (TII area).
template <typename T, int D>
__device__ __forceinline__ void inverse_cols(unsigned char* smem, int wave, int lane) {
  typedef Lds<T, D> M;
  typedef Sub<T> S;
  const float* sA = (const float*)(smem + M::V);
  const float* sTii = (const float*)(smem + M::TII);  // [4][16][16]
  const float* sBeta = (const float*)(smem + M::BETA);
  const int idx = lane & 15, gq = lane >> 4, j = wave;
  typename S::Opnd wo[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (i == j) {
      const float b = sBeta[16 * i + idx];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = sTii[(16 * i + 4 * gq + e) * 16 + idx] * b;
    } else if (i > j) {
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < i; ++m)
        if (m >= j) r = S::apply(S::coef(sA + (16 * i + idx) * M::LDF + 16 * m + 4 * gq, true), wo[m], r);
      w = S::apply(S::coef(sTii + (16 * i + idx) * 16 + 4 * gq, false), S::opnd(r),
                   (f32x4){0.f, 0.f, 0.f, 0.f});
    }
    if (i < 3 && i >= j) wo[i] = S::opnd(w);
    store_tp<T, D>(smem, w, i, j, lane);
  }
}

// W = Tp X for NX column tiles: tile ct[t] of the channel-major X^T array
// xt[t]; w[t][rb] is row tile rb.  Tp's zero blocks above the diagonal are
// skipped where a whole k-block is zero.
template <typename T, int D, int NX>
__device__ __forceinline__ void w_products(const unsigned char* smem, const T* const (&xt)[NX], const int (&ct)[NX],
                                           int lane, f32x4 (&w)[NX][4]) {
  typedef Lds<T, D> M;
  typedef TpArea<T, D> TP;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = Elem<T>::KB, NKC = C / KB;
  const int idx = lane & 15, gq = lane >> 4;
  const T* tph = (const T*)(smem + TP::HI);
  const T* tpl = (const T*)(smem + TP::LO);
  FragT xb[NX][NKC];
#pragma unroll
  for (int t = 0; t < NX; ++t)
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) xb[t][kb] = frag_rows(xt[t], M::LDC, 16 * ct[t] + idx, kb * KB, gq);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
    for (int t = 0; t < NX; ++t) w[t][rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
      if (kb * KB > 16 * rb + 15) continue;
      const FragT ah = frag_rows(tph, TP::LD, 16 * rb + idx, kb * KB, gq);
#pragma unroll
      for (int t = 0; t < NX; ++t) w[t][rb] = mma(ah, xb[t][kb], w[t][rb]);
      if constexpr (sizeof(T) == 2) {
        const FragT al = frag_rows(tpl, TP::LD, 16 * rb + idx, kb * KB, gq);
#pragma unroll
        for (int t = 0; t < NX; ++t) w[t][rb] = mma(al, xb[t][kb], w[t][rb]);
      }
    }
  }
}

// Wk tile (all 64 rows, 16 channels from 16 ct) into LDS area AREA, token-major.
template <typename T, int D, int AREA>
__device__ __forceinline__ void store_wk(unsigned char* smem, const f32x4 (&w)[4], int ct, int lane) {
  typedef Lds<T, D> M;
  T* sW = (T*)(smem + AREA);
  const int idx = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sW[(16 * rt + 4 * gq + i) * M::LDT + 16 * ct + idx] = Elem<T>::from_f32(w[rt][i]);
}

// ---- chunk record: what the chunk pass leaves for the two state passes,
// per (chunk, head), in device memory.  It starts with an image of the state
// passes' LDS (Img), copied linearly: the A-operand fragments of the state
// products, each 64 lanes x 16 bytes in lane order (one 16-byte LDS read per
// lane and fragment):
//   WF  Wk rows       [4 row tiles][D / KB k-blocks]
//   KF  Kh^T rows     [D / 16 row tiles][64 / KB k-blocks]
//   GAM gamma         [D] fp32, padded to 1 KiB
//   QF  Qt rows       [4 row tiles][D / KB k-blocks]
//   PF  P rows        [4 row tiles][64 / KB k-blocks]
// then
//   WV  [D/16 column tiles][4 row tiles][64 lanes][4]  Wv in the operand type (bf16
//       path: rounded to bf16, as U = Wv - Wk S is before every product it
//       enters), accumulator order.
// Chunk j of sequence n has slot (chunks of sequences 0 .. n - 1) + j.
template <typename T, int D> struct Img {
  static constexpr int KB = Elem<T>::KB, NKD = D / KB, NKC = C / KB, NR = D / 16;
  static constexpr int WF = 0, KF = WF + 4 * NKD * 1024, GAM = KF + NR * NKC * 1024,
                       QF = GAM + (D * 4 + 1023) / 1024 * 1024, PF = QF + 4 * NKD * 1024, BYTES = PF + 4 * NKC * 1024;
  __device__ static __forceinline__ int q(int rt, int kb, int lane) { return QF + ((rt * NKD + kb) * 64 + lane) * 16; }
  __device__ static __forceinline__ int w(int rt, int kb, int lane) { return WF + ((rt * NKD + kb) * 64 + lane) * 16; }
  __device__ static __forceinline__ int k(int rr, int kb, int lane) { return KF + ((rr * NKC + kb) * 64 + lane) * 16; }
  __device__ static __forceinline__ int p(int rt, int kb, int lane) { return PF + ((rt * NKC + kb) * 64 + lane) * 16; }
};
template <typename T, int D> struct CRec {
  static constexpr size_t ES = sizeof(T);
  static constexpr size_t WV = Img<T, D>::BYTES, BYTES = WV + (size_t)C * D * ES;
  __device__ static __forceinline__ size_t wv(int ct, int rt, int lane) {
    return WV + (((size_t)ct * 4 + rt) * 64 + lane) * 4 * ES;
  }
  typedef typename std::conditional<sizeof(T) == 2, uint2, f32x4>::type WvRaw;
  // one lane's 4 accumulator values of a Wv tile, in the operand type
  __device__ static __forceinline__ WvRaw pack(const f32x4& w) {
    if constexpr (sizeof(T) == 2) {
      return (uint2){__builtin_bit_cast(uint32_t, f32x2_to_bf16x2(w[0], w[1])),
                     __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(w[2], w[3]))};
    } else {
      return w;
    }
  }
  __device__ static __forceinline__ void put_wv(unsigned char* p, const f32x4& w) { *(WvRaw*)p = pack(w); }
  // loaded as raw words (a prefetch then holds them without waiting for the
  // load) and widened only where they are used
  __device__ static __forceinline__ WvRaw load_wv(const unsigned char* p) {
    if constexpr (sizeof(T) == 2) return __builtin_bit_cast(WvRaw, __builtin_nontemporal_load((const u32x2nt*)p));
    else return __builtin_bit_cast(WvRaw, __builtin_nontemporal_load((const u32x4nt*)p));
  }
  __device__ static __forceinline__ f32x4 widen(const WvRaw& u) {
    if constexpr (sizeof(T) == 2) {
      return (f32x4){__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u)};
    } else {
      return u;
    }
  }
  // w rounded as the record stores it
  __device__ static __forceinline__ f32x4 as_stored(const f32x4& w) { return widen(pack(w)); }
};

// The chunk's record from the chunk pass's LDS, in two parts:
//   save_early: Qt (Q area), Kh^T (KH), P (P) fragments and gamma (GL), ready
//               once the Gram blocks are done;
//   save_wk:    Wk fragments (area WKA), ready after the W products.
// Waves w0 .. w0 + nw - 1 take the fragments w - w0, w - w0 + nw, ...
template <typename T, int D>
__device__ __forceinline__ void save_early(const unsigned char* smem, unsigned char* rec, int w, int nw, int lane) {
  typedef Lds<T, D> M;
  typedef Img<T, D> I;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = I::KB, NQ = 4 * I::NKD, NK = I::NR * I::NKC, NP = 4 * I::NKC, NF = NQ + NK + NP;
  const int idx = lane & 15, gq = lane >> 4;
  const T* sQ = (const T*)(smem + M::Q);
  const T* sKH = (const T*)(smem + M::KH);
  const T* sP = (const T*)(smem + M::P);
  for (int f = w; f < NF; f += nw) {
    FragT x;
    int off;
    if (f < NQ) {
      const int rt = f / I::NKD, kb = f % I::NKD;
      x = frag_rows(sQ, M::LDT, 16 * rt + idx, kb * KB, gq);
      off = I::q(rt, kb, lane);
    } else if (f < NQ + NK) {
      const int rr = (f - NQ) / I::NKC, kb = (f - NQ) % I::NKC;
      x = frag_rows(sKH, M::LDC, 16 * rr + idx, kb * KB, gq);
      off = I::k(rr, kb, lane);
    } else {
      const int rt = (f - NQ - NK) / I::NKC, kb = (f - NQ - NK) % I::NKC;
      x = frag_rows(sP, M::LDC, 16 * rt + idx, kb * KB, gq);
      off = I::p(rt, kb, lane);
    }
    *(FragT*)(rec + off) = x;
  }
  if (w == 0 && lane < D / 4) *(f32x4*)(rec + I::GAM + 16 * lane) = *(const f32x4*)(smem + M::GL + 16 * lane);
}
template <typename T, int D, int WKA>
__device__ __forceinline__ void save_wk(const unsigned char* smem, unsigned char* rec, int w, int nw, int lane) {
  typedef Lds<T, D> M;
  typedef Img<T, D> I;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = I::KB, NQ = 4 * I::NKD;
  const int idx = lane & 15, gq = lane >> 4;
  const T* sW = (const T*)(smem + WKA);
  for (int f = w; f < NQ; f += nw) {
    const int rt = f / I::NKD, kb = f % I::NKD;
    *(FragT*)(rec + I::w(rt, kb, lane)) = frag_rows(sW, M::LDT, 16 * rt + idx, kb * KB, gq);
  }
}

// Record image bytes [0, NBYTES) -> LDS `dst` by direct global-to-LDS loads
// (lane i of a wave fills bytes 16 i .. 16 i + 15 of a 1 KiB block; no
// registers held).  Wave w takes blocks w, w + NW, ...; part k of NPARTS
// issues the k-th slice of them, so that the issue can be spread over other
// work.  The loads are only issued: vmcnt_wait_all() and a barrier make them
// visible.
constexpr int kCpolNt = 2;  // cache-policy operand of the direct loads: non-temporal
template <int NW, int NBYTES, int NPARTS>
__device__ __forceinline__ void issue_image(unsigned char* dst, const unsigned char* rec, int wave, int lane, int k) {
  constexpr int NB = NBYTES / 1024;
  static_assert(NBYTES % 1024 == 0, "whole blocks");
  const int nbw = (NB - wave + NW - 1) / NW;  // blocks of this wave
  const int i0 = k * nbw / NPARTS, i1 = (k + 1) * nbw / NPARTS;
  for (int i = i0; i < i1; ++i) {
    const int b = wave + NW * i;
    __builtin_amdgcn_global_load_lds((const void*)(rec + 1024 * b + 16 * lane),
                                     (__attribute__((address_space(3))) void*)(dst + 1024 * b), 16, 0,
                                     kCpolNt);
  }
}
__device__ __forceinline__ void vmcnt_wait_all() { __builtin_amdgcn_s_waitcnt(0); }
// Workgroup barrier that orders LDS reads and writes only: it waits for this
// wave's LDS operations but not for its global loads, so direct-to-LDS loads
// into the other image buffer stay in flight (__syncthreads() would wait for
// them as pending LDS writes).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Where a state step reads its A operands (each one 16-byte LDS read per
// lane): a record image (ImgSrc, the state passes), or the chunk pass's own
// arrays (LdsSrc: Qt, Kh^T, P, gamma and Wk in area WKA), from which the
// image fragments are cut, so both give the same values.
template <typename T, int D> struct ImgSrc {
  typedef Img<T, D> I;
  typedef typename Frag<T>::type FragT;
  const unsigned char* img;
  int lane;
  __device__ __forceinline__ FragT at(int off) const { return *(const FragT*)(img + off); }
  __device__ __forceinline__ FragT w(int rt, int kb) const { return at(I::w(rt, kb, lane)); }
  __device__ __forceinline__ FragT q(int rt, int kb) const { return at(I::q(rt, kb, lane)); }
  __device__ __forceinline__ FragT p(int rt, int kb) const { return at(I::p(rt, kb, lane)); }
  __device__ __forceinline__ FragT k(int rr, int kb) const { return at(I::k(rr, kb, lane)); }
  __device__ __forceinline__ f32x4 gam(int rr) const {
    return *(const f32x4*)(img + I::GAM + 4 * (16 * rr + 4 * (lane >> 4)));
  }
};
template <typename T, int D, int WKA> struct LdsSrc {
  typedef Lds<T, D> M;
  typedef typename Frag<T>::type FragT;
  static constexpr int KB = Elem<T>::KB;
  const unsigned char* smem;
  int lane;
  __device__ __forceinline__ FragT rows(int area, int ld, int r, int kb) const {
    return frag_rows((const T*)(smem + area), ld, r + (lane & 15), kb * KB, lane >> 4);
  }
  __device__ __forceinline__ FragT w(int rt, int kb) const { return rows(WKA, M::LDT, 16 * rt, kb); }
  __device__ __forceinline__ FragT q(int rt, int kb) const { return rows(M::Q, M::LDT, 16 * rt, kb); }
  __device__ __forceinline__ FragT p(int rt, int kb) const { return rows(M::P, M::LDC, 16 * rt, kb); }
  __device__ __forceinline__ FragT k(int rr, int kb) const { return rows(M::KH, M::LDC, 16 * rr, kb); }
  __device__ __forceinline__ f32x4 gam(int rr) const {
    return *(const f32x4*)(smem + M::GL + 4 * (16 * rr + 4 * (lane >> 4)));
  }
};

// CT column tiles of the state (rows = D key channels) through one chunk:
// U = Wv - Wk S; S <- diag(gamma) (S + Kh^T U).  With WITH_O also
// O = Qt S + P U.  `wv` holds Wv's tiles for these columns.  The A operands
// come from `src` (ImgSrc or LdsSrc), each loaded once per phase and fed to
// the CT tiles.  hook(k), k = 0 .. 4 + D / 16 - 1, is called between the row
// blocks (the callers spread the next image's loads there).
template <typename T, int D, int CT, bool WITH_O, typename Src, typename Hook>
__device__ __forceinline__ void state_step(const Src& src, f32x4 (&S)[CT][D / 16], const f32x4 (&wv)[CT][4],
                                           f32x4 (&O)[CT][4], int lane, Hook&& hook) {
  typedef Img<T, D> I;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = I::KB, NKD = I::NKD, NKC = I::NKC, NR = I::NR;

  FragT SB[CT][NKD];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) SB[c][kb] = Frag<T>::from_acc(S[c], kb);
  // U and Qt S
  f32x4 U[CT][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    FragT aw[NKD], aq[NKD];
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      aw[kb] = src.w(rt, kb);
      if (WITH_O) aq[kb] = src.q(rt, kb);
    }
    f32x4 ws[CT], qs[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) ws[c] = qs[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        ws[c] = mma(aw[kb], SB[c][kb], ws[c]);
        if (WITH_O) qs[c] = mma(aq[kb], SB[c][kb], qs[c]);
      }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) U[c][rt][i] = wv[c][rt][i] - ws[c][i];
      O[c][rt] = qs[c];
    }
    hook(rt);
  }
  FragT UB[CT][NKC];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) UB[c][kb] = Frag<T>::from_acc(U[c], kb);
  if (WITH_O) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      FragT ap[NKC];
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb)
        if (kb * KB <= 16 * rt + 15) ap[kb] = src.p(rt, kb);
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb)
        if (kb * KB <= 16 * rt + 15) {
#pragma unroll
          for (int c = 0; c < CT; ++c) O[c][rt] = mma(ap[kb], UB[c][kb], O[c][rt]);
        }
    }
  }
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    FragT ak[NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) ak[kb] = src.k(rr, kb);
    const f32x4 gm = src.gam(rr);
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
      for (int c = 0; c < CT; ++c) S[c][rr] = mma(ak[kb], UB[c][kb], S[c][rr]);
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[c][rr][i] *= gm[i];
    hook(4 + rr);
  }
}

// The segment map in the segment record (Rec): B from each wave's accumulator
// tiles, M through LDS (sM, [D][D + 4] fp32) into the scan's A-operand
// fragments.  wave owns the column tiles cols[x] of B (XB[x]) and of M (XM[x]).
template <typename T, int D, int NW, int NC>
__device__ __forceinline__ void save_map(float* sM, float* recs, const f32x4 (&XB)[NC][D / 16],
                                         const f32x4 (&XM)[NC][D / 16], const int (&cols)[NC], int wave,
                                         int lane) {
  typedef Rec<T, D> R;
  constexpr int NR = D / 16, LDM = D + 4;
  const int idx = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int x = 0; x < NC; ++x)
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      *(f32x4*)(recs + R::B + R::tile(rr, cols[x], lane)) = XB[x][rr];
#pragma unroll
      for (int i = 0; i < 4; ++i) sM[(16 * rr + 4 * gq + i) * LDM + 16 * cols[x] + idx] = XM[x][rr][i];
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

// ---- pass 1: the chunk-local part of every chunk -> its record -----------
// One workgroup per (group of L consecutive chunks of a sequence, head)
// walks its chunks; the inputs of the next chunk are fetched while the
// current one is finished.  Wave w forms Wk and Wv for the value-column tiles
// w + NW x.
// With MAPS the groups are the segments of the state passes, and the
// workgroup also composes its segment's affine map S_out = M S_in + B (not
// for the last segment of a sequence: no later segment needs it): after each
// chunk's W products it takes the chunk's Wk, Kh^T, gamma and Wv, still in
// LDS and registers, through a state step on B (started from 0) and on M
// (started from I, value part of U off), wave w on the column tiles it owns.
// Without MAPS (every sequence is one segment) the group length is the chunk
// pass's own.
template <typename T, int D, int NW, bool MAPS, bool MX>
__global__ void __launch_bounds__(64 * NW)
kda_chunk_prep(const ChunkInputs in, const int32_t* __restrict__ cu, int n_rows, int T_per, int H, int L,
               float g_floor, int gate, unsigned char* __restrict__ crec, float* __restrict__ ws) {
  typedef Lds<T, D> M;
  typedef CRec<T, D> CR;
  constexpr int NT = 64 * NW, NR = D / 16, NV = NR / NW;
  static_assert(NV >= 1 && NV * NW == NR, "waves must split the value columns");
  static_assert(D * (D + 4) * 4 <= M::BYTES, "M staging fits the chunk pass's LDS");
  __shared__ __attribute__((aligned(16))) unsigned char smem[M::BYTES];
  Seg sg;
  if (!locate(cu, n_rows, T_per, L, blockIdx.x, sg)) return;
  const int h = blockIdx.y, tid0 = threadIdx.x, lane0 = tid0 & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);  // uniform: scalar control flow
  const int idx = lane0 & 15, gq = lane0 >> 4;
  const int nch = (sg.len + C - 1) / C, j0 = sg.s * L, j1 = min(j0 + L, nch);
  const bool maps = MAPS && sg.s < sg.nseg - 1;
  int cts[NV];
#pragma unroll
  for (int x = 0; x < NV; ++x) cts[x] = wave + NW * x;
  // the segment map's column tiles cts[x]: B in X[x], M in X[NV + x]
  f32x4 X[MAPS ? 2 * NV : 1][NR];
  if (MAPS) {
#pragma unroll
    for (int x = 0; x < NV; ++x)
#pragma unroll
      for (int rr = 0; rr < NR; ++rr)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          X[x][rr][i] = 0.f;
          X[NV + x][rr][i] = (16 * rr + 4 * gq + i == 16 * cts[x] + idx) ? 1.f : 0.f;
        }
  }

  {
    Raw<T, D, NT, true, MX> first;
    first.load(in, sg.tok0 + (int64_t)C * j0, min(C, sg.len - C * j0), H, h, tid0, gate);
    first.store(smem, tid0);
  }
  __syncthreads();
  for (int j = j0; j < j1; ++j) {
    // With MAPS (the map's state tiles take 64 registers), thread and lane
    // index as opaque per-chunk values: the addresses derived from them are
    // formed inside the loop, not hoisted and held across it, which would
    // overflow the registers.
    int tid = tid0, lane = lane0;
    if (MAPS) asm volatile("" : "+v"(tid), "+v"(lane));
    elementwise<T, D, NW, true>(smem, g_floor, tid);
    // the next chunk's inputs are fetched while this one is worked on: q, k,
    // g and beta now (into LDS once Wk is complete), v now as well, or with
    // MAPS (short of registers) once Wk is complete, the map's state step
    // covering its latency (into LDS at the end of the chunk)
    Raw<T, D, NT, true, MX> raw;
    const bool more = j + 1 < j1;
    const int64_t tok_n = sg.tok0 + (int64_t)C * (j + 1);
    const int len_n = min(C, sg.len - C * (j + 1));
    if (more) {
      raw.load_qkg(in, tok_n, len_n, H, h, tid, gate);
      if (!MAPS) raw.load_v(in, tok_n, len_n, H, h, tid);
    }
    gram<T, D, NW, true>(smem, wave, lane);  // also the diagonal-block inverses
    unsigned char* cr = crec + ((size_t)(sg.chunk0 + j) * H + h) * CR::BYTES;
    // waves 0-3 form Tp; with eight waves the other four meanwhile write the
    // record parts that are already final
    if (wave < 4) inverse_cols<T, D>(smem, wave, lane);
    if (NW > 4 && wave >= 4) save_early<T, D>(smem, cr, wave - 4, NW - 4, lane);
    if (NW <= 4) save_early<T, D>(smem, cr, wave, NW, lane);
    __syncthreads();  // Tp complete; A and the diagonal inverses are dead
    // Wk and Wv in one pass over Tp: operands x < NV are Kt^T column tiles,
    // the others V^T tiles
    const T* xo[2 * NV];
    int co[2 * NV];
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      xo[x] = (const T*)(smem + M::KT);
      xo[NV + x] = (const T*)(smem + M::VT);
      co[x] = co[NV + x] = cts[x];
    }
    f32x4 wvt[NV][4];
    {
      f32x4 w[2 * NV][4];
      w_products<T, D, 2 * NV>(smem, xo, co, lane, w);
#pragma unroll
      for (int x = 0; x < NV; ++x) {
        store_wk<T, D, M::V>(smem, w[x], cts[x], lane);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) wvt[x][rt] = w[NV + x][rt];
      }
    }
    __syncthreads();  // Wk complete; Tp, Qt, Kh and beta are dead
    // the next chunk's q, k, g and beta go to their areas now (v's area holds
    // Wk until the end of the chunk).  With MAPS, v is fetched only after
    // that store: the store's wait for q, k and g would otherwise cover the v
    // loads too (loads complete in order), leaving no time to hide them.
    if (more) {
      raw.store_qkg(smem, tid);
      if (MAPS) raw.load_v(in, tok_n, len_n, H, h, tid);
    }
    save_wk<T, D, M::V>(smem, cr, wave, NW, lane);
#pragma unroll
    for (int x = 0; x < NV; ++x)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) CR::put_wv(cr + CR::wv(cts[x], rt, lane), wvt[x][rt]);
    if (maps) {
      // Wv as the record holds it, so that the map and the output pass see
      // the same chunk
      f32x4 wvx[MAPS ? 2 * NV : 1][4], unused[MAPS ? 2 * NV : 1][4];
#pragma unroll
      for (int x = 0; x < NV; ++x)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          wvx[x][rt] = CR::as_stored(wvt[x][rt]);
          wvx[NV + x][rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      state_step<T, D, MAPS ? 2 * NV : 1, false>(LdsSrc<T, D, M::V>{smem, lane}, X, wvx, unused, lane,
                                                  [](int) {});
    }
    __syncthreads();  // done with this chunk's LDS
    if (more) {
      raw.store_v(smem, tid);
      __syncthreads();
    }
  }
  if (maps) {
    f32x4 XB[NV][NR], XM[NV][NR];
#pragma unroll
    for (int x = 0; x < NV; ++x)
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        XB[x][rr] = X[x][rr];
        XM[x][rr] = X[MAPS ? NV + x : 0][rr];
      }
    save_map<T, D, NW, NV>((float*)smem, ws + ((size_t)blockIdx.x * H + h) * Rec<T, D>::FLOATS, XB, XM, cts,
                           wave, lane0);
  }
}

// ---- pass 3: outputs from every segment's incoming state -----------------
// Reads the chunk records into two LDS image buffers; wave w owns the
// value-column tiles w + NW x, x < CT.  O is staged at the start of the
// current image (Wk and Kh^T fragments, dead after the products) so that the
// global stores are whole 16-byte pieces of rows.  The next chunk's image is
// issued piecewise between the row blocks of the state step.  With `states`,
// the state after every `every`-th full chunk of a sequence goes to its slot
// (the prefix-cache states of kda_chunk_forward_states).
template <typename T, int D, int NW, int CT>
__global__ void __launch_bounds__(64 * NW)
kda_seg_forward(const int32_t* __restrict__ cu, int n_rows, int T_per, int H, int L,
                const float* __restrict__ ws, const unsigned char* __restrict__ crec, T* __restrict__ o,
                float* ht, float* __restrict__ states, int every) {
  typedef Lds<T, D> M;
  typedef CRec<T, D> CR;
  typedef Img<T, D> I;
  constexpr int NT = 64 * NW, NR = D / 16;
  static_assert(NW * CT == NR, "waves must split the value columns");
  static_assert(M::ROW_T <= I::GAM, "O staging fits the Wk and Kh^T fragments");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * I::BYTES];
  Seg sg;
  if (!locate(cu, n_rows, T_per, L, blockIdx.x, sg)) return;
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar control flow
  const int idx = lane & 15, gq = lane >> 4;
  const int nch = (sg.len + C - 1) / C, j0 = sg.s * L, j1 = min(j0 + L, nch);
  auto rec = [&](int j) -> const unsigned char* { return crec + ((size_t)(sg.chunk0 + j) * H + h) * CR::BYTES; };
  typedef typename CR::WvRaw WvRaw;
  auto load_wv = [&](int j, WvRaw (&w)[CT][4]) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) w[c][rt] = CR::load_wv(rec(j) + CR::wv(wave + NW * c, rt, lane));
  };

  constexpr int NP = 4 + NR;  // hook points of a state step
  for (int k = 0; k < NP; ++k) issue_image<NW, I::BYTES, NP>(smem, rec(j0), wave, lane, k);
  WvRaw wv[CT][4];
  load_wv(j0, wv);
  typedef Rec<T, D> R;
  const float* sin = ws + ((size_t)(blockIdx.x) * H + h) * R::FLOATS + R::SIN;
  f32x4 S[CT][NR];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) S[c][rr] = *(const f32x4*)(sin + R::tile(rr, wave + NW * c, lane));
  // this wave's columns of S, row-major [D][D] at dst (ht and the states)
  auto put_state = [&](float* dst) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rr = 0; rr < NR; ++rr)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * rr + 4 * gq + i) * D + 16 * (wave + NW * c) + idx] = S[c][rr][i];
  };
  // first state slot of this sequence: full state periods of the earlier ones
  const int64_t period = (int64_t)C * every;
  int64_t slot0 = 0;
  if (states) {
    if (cu) {
      for (int m = 0; m < sg.n; ++m) slot0 += (cu[m + 1] - cu[m]) / period;
    } else {
      slot0 = (int64_t)sg.n * (T_per / period);
    }
  }

  for (int j = j0; j < j1; ++j) {
    const int clen = min(C, sg.len - C * j);
    const int64_t tokc = sg.tok0 + (int64_t)C * j;
    unsigned char* cur = smem + ((j - j0) & 1) * I::BYTES;
    unsigned char* nxt = smem + ((j + 1 - j0) & 1) * I::BYTES;
    vmcnt_wait_all();
    __syncthreads();  // image j in LDS; every wave is done with the other buffer
    WvRaw wvn[CT][4];
    const bool more = j + 1 < j1;
    if (more) load_wv(j + 1, wvn);
    f32x4 wvf[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) wvf[c][rt] = CR::widen(wv[c][rt]);
    f32x4 O[CT][4];
    state_step<T, D, CT, true>(ImgSrc<T, D>{cur, lane}, S, wvf, O, lane, [&](int k) {
      if (more) issue_image<NW, I::BYTES, NP>(nxt, rec(j + 1), wave, lane, k);
    });
    lds_barrier();  // every wave is done with the Wk and Kh^T fragments
    T* sO = (T*)cur;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sO[(16 * rt + 4 * gq + i) * M::LDT + 16 * (wave + NW * c) + idx] = Elem<T>::from_f32(O[c][rt][i]);
    lds_barrier();
    Raw<T, D, NT, true>::store_out(cur, o, tokc, clen, H, h, tid);
    if (states && (j + 1) % every == 0 && (int64_t)(j + 1) * C <= sg.len)
      put_state(states + ((size_t)(slot0 + (j + 1) / every - 1) * H + h) * D * D);
    if (j + 1 < j1) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) wv[c][rt] = wvn[c][rt];
    }
  }
  if (ht && sg.s == sg.nseg - 1) put_state(ht + ((size_t)sg.n * H + h) * D * D);
}

// ---- pass 2: segment scan S_{s+1} = M_s S_s + B_s ------------------------
// Workgroup = (sequence, head, 16 state columns), one wave per 16-row tile of
// S.  Each step a wave publishes its rows as halves of B-operand fragments
// through a double-buffered LDS area and forms the same rows of the next state
// from all k-blocks, so one barrier per step orders the exchange.  M_s and
// B_s do not depend on the state: each wave fetches its rows of them three
// steps ahead.
template <typename T, int D> struct ScanOps;
template <int D> struct ScanOps<bf16_t, D> {
  static constexpr int KB = 32, NKB = D / KB;
  // Published state, in B-fragment order: [hi/lo][k-block][lane] 16 bytes,
  // row tile t filling bytes 8 (t % 2) .. 8 (t % 2) + 7 of k-block t / 2.
  typedef uint4 PubArea[2][NKB][64];
  __device__ static __forceinline__ void publish(PubArea& a, int t, int lane, const f32x4& x) {
    const s16x4 h = to_bf16x4(x);
    *((uint2*)&a[0][t >> 1][lane] + (t & 1)) = __builtin_bit_cast(uint2, h);
    *((uint2*)&a[1][t >> 1][lane] + (t & 1)) = __builtin_bit_cast(uint2, to_bf16x4(x - from_bf16x4(h)));
  }
  struct SFrag { bf16x8 hi, lo; };
  __device__ static __forceinline__ SFrag gather(const PubArea& a, int kb, int lane) {
    return SFrag{__builtin_bit_cast(bf16x8, a[0][kb][lane]), __builtin_bit_cast(bf16x8, a[1][kb][lane])};
  }
  struct MRaw { bf16x8 hi, lo; };
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
kda_seg_scan(const float* h0, float* ht, float* __restrict__ ws, const int32_t* __restrict__ cu, int n_rows,
             int T_per, int H, int L) {
  typedef ScanOps<T, D> Ops;
  constexpr int NKB = Ops::NKB, NWS = D / 16, WPP = D / 16;
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

  int64_t base = 0;
  int len;
  if (cu) {
    for (int m = 0; m < n; ++m) base += n_segments(cu[m + 1] - cu[m], L);
    len = cu[n + 1] - cu[n];
  } else {
    base = (int64_t)n * n_segments(T_per, L);
    len = T_per;
  }
  const int nseg = n_segments(len, L);

  f32x4 Sk;
#pragma unroll
  for (int i = 0; i < 4; ++i) Sk[i] = h0 ? h0[((size_t)p * D + 16 * wave + 4 * gq + i) * D + col] : 0.f;
  typedef Rec<T, D> R;
  auto rec = [&](int s) -> float* { return ws + ((size_t)(base + s) * H + h) * R::FLOATS; };
  auto put = [&](float* dst) { *(f32x4*)(dst + R::tile(wave, ct, lane)) = Sk; };  // accumulator tile order
  if (nseg == 0) {
    if (ht) {
      float* dst = ht + (size_t)p * D * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * wave + 4 * gq + i) * D + col] = Sk[i];
    }
    return;
  }
  put(rec(0) + R::SIN);
  struct Stage {
    typename Ops::MRaw m[NKB];
    f32x4 b;
  };
  // Buffer loads: a step's record is one scalar resource, the lanes' byte
  // offsets into it fixed registers, so the fetches take no per-lane address
  // registers (64-bit address temporaries were placed over registers still
  // being loaded, which made every fetch wait for the ones in flight).
  const uint32_t m_off = (uint32_t)(R::M * 4 + R::frag(wave, 0, 0, lane));
  const uint32_t b_off = (uint32_t)((R::B + R::tile(wave, ct, lane)) * 4);
  constexpr int kRecBytes = (int)(R::FLOATS * 4), kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 family
  auto fetch = [&](int s, Stage& st) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(rec(s), (short)0, kRecBytes, kRsrcWord3);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) st.m[kb] = Ops::load_m(r, m_off, kb);
    st.b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, b_off, 0, 0));
    // issued here, before the step's own temporaries are allocated (moved
    // below them, a load's target registers were handed out as temporaries,
    // whose writes then wait for the load)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int s, const Stage& st) {
    Ops::publish(sS[s & 1], wave, lane, Sk);
    __syncthreads();
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
  // unused): unconditional loads keep the wait counts exact, so a step waits
  // only for its own stage and never for the fetches issued after it.  A ring
  // of three register stages (the loop unrolled by three, so that the stages
  // never move between registers).
  auto clamp = [&](int s) { return s < nsteps ? s : nsteps - 1; };
  // Unrolled by six (two turns of the ring), so that the conservative wait
  // after the loop head (where the pending loads of the two incoming paths are
  // merged) falls on one step in six.
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

// MXFP8 inputs are decoded into the bf16 path (the fp32 path takes none).
template <typename T, int D> struct MxOk { static constexpr bool value = sizeof(T) == 2 && D % 32 == 0; };

template <typename T, int D, int NW, int NW2>
int launch_typed(int n_rows, int T_per, int H, const SegPlan& plan, float g_floor, int gate, const ChunkInputs& in,
                 const float* h0, const int32_t* cu, void* o, float* ht, float* states, int every, void* ws,
                 hipStream_t stream, void* const* events) {
  constexpr int NR = D / 16;
  const int L = plan.seg_chunks;
  float* wsf = (float*)ws;
  unsigned char* crec = (unsigned char*)ws + plan.crec_off;
  if (plan.crec_bytes != CRec<T, D>::BYTES) return (int)hipErrorInvalidValue;
  if (in.qs && !MxOk<T, D>::value) return (int)hipErrorInvalidValue;  // MXFP8 inputs: bf16 path only
  const bool has_segments = plan.n_seg_bound > 0;
  hipError_t e;
  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord((hipEvent_t)events[i], stream) : hipSuccess;
  };
  if ((e = mark(0)) != hipSuccess) return (int)e;
  if (has_segments) {
    const bool mx = in.qs != nullptr;
    const unsigned grid = (unsigned)(plan.maps_in_prep ? plan.n_seg_bound : plan.n_prep_bound);
    const int gl = plan.maps_in_prep ? L : plan.prep_chunks;
    const dim3 g3(grid, H), b3(64 * NW);
    if (plan.maps_in_prep && mx)
      hipLaunchKernelGGL((kda_chunk_prep<T, D, NW, true, MxOk<T, D>::value>), g3, b3, 0, stream, in, cu, n_rows,
                         T_per, H, gl, g_floor, gate, crec, wsf);
    else if (plan.maps_in_prep)
      hipLaunchKernelGGL((kda_chunk_prep<T, D, NW, true, false>), g3, b3, 0, stream, in, cu, n_rows, T_per, H, gl,
                         g_floor, gate, crec, wsf);
    else if (mx)
      hipLaunchKernelGGL((kda_chunk_prep<T, D, NW, false, MxOk<T, D>::value>), g3, b3, 0, stream, in, cu, n_rows,
                         T_per, H, gl, g_floor, gate, crec, wsf);
    else
      hipLaunchKernelGGL((kda_chunk_prep<T, D, NW, false, false>), g3, b3, 0, stream, in, cu, n_rows, T_per, H, gl,
                         g_floor, gate, crec, wsf);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  if ((e = mark(1)) != hipSuccess) return (int)e;
  const int64_t pairs = (int64_t)n_rows * H;
  const int64_t blocks = (pairs + 7) / 8 * 8 * NR;
  hipLaunchKernelGGL((kda_seg_scan<T, D>), dim3((unsigned)blocks), dim3(64 * (D / 16)), 0, stream,
                     h0, ht, wsf, cu, n_rows, T_per, H, L);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if ((e = mark(2)) != hipSuccess) return (int)e;
  if (has_segments) {
    hipLaunchKernelGGL((kda_seg_forward<T, D, NW2, NR / NW2>), dim3((unsigned)plan.n_seg_bound, H), dim3(64 * NW2),
                       0, stream, cu, n_rows, T_per, H, L, (const float*)wsf, (const unsigned char*)crec, (T*)o, ht,
                       states, every);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  return (int)mark(3);
}

}  // namespace

int launch_chunk_forward(int is_bf16, int d, int n_rows, int T, int H, const SegPlan& plan, float g_floor,
                         int gate, const ChunkInputs& in, const float* h0, const int32_t* cu, void* o, float* ht,
                         float* states, int every, void* ws, void* stream, void* const* events) {
  hipStream_t s = (hipStream_t)stream;
  if (is_bf16 && d == 64)
    return launch_typed<bf16_t, 64, 4, 4>(n_rows, T, H, plan, g_floor, gate, in, h0, cu, o, ht, states, every, ws,
                                          s, events);
  if (is_bf16 && d == 128)
    return launch_typed<bf16_t, 128, KDA_NW128, KDA_NW128_FWD>(n_rows, T, H, plan, g_floor, gate, in, h0, cu, o,
                                                               ht, states, every, ws, s, events);
  if (!is_bf16 && d == 64)
    return launch_typed<float, 64, 4, 4>(n_rows, T, H, plan, g_floor, gate, in, h0, cu, o, ht, states, every, ws,
                                         s, events);
  return (int)hipErrorInvalidValue;
}

}  // namespace kda
