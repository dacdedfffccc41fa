// Backward pass of the chunked KDA forward (gfx950 / CDNA4).
//
// Per sequence and head, a chunk of C = 64 rows r with incoming state S maps
// (Gamma_r = sum_{s<=r} g_s per key channel, gamma = e^{Gamma_last}):
//   Qt = Q e^{Gamma}, Kt = K e^{Gamma}, Kh = K e^{-Gamma},
//   Abar = strict_lower(Kt Kh^T), T = (I + diag(beta) Abar)^{-1},
//   Wk = T diag(beta) Kt, Wv = T diag(beta) V, P = lower_incl(Qt Kh^T),
//   U = Wv - Wk S,  O = Qt S + P U,  S_next = diag(gamma)(S + Kh^T U).
// This is the recurrence S_t = (I - b k k^T) diag(a) S_{t-1} + b k v^T,
// o_t = S_t^T q_t unrolled over the chunk (the delta rule of "Kimi K3 深度拆解"
// (chenxutan.com), 4.2 "线性注意力与 Delta Rule", with the channel-wise gate of
// "Kimi K3 技術報告" (akiraxclaw.com), "長度：KDA 為什麼還要搭配 Gated MLA？";
// the floor on the log-decay keeps e^{-Gamma} bounded, "3 分钟看懂 Kimi K3"
// (landx.limxdynamics.com), "第一条主线", Figure 3).  The pages give no
// gradient; the one below is the chain rule on those lines.
//
// With dH the gradient of the chunk's end state and dO that of its outputs:
//   dU   = P^T dO + Kh diag(gamma) dH
//   dS   = Qt^T dO + diag(gamma) dH - Wk^T dU            (to the previous chunk)
//   dP   = lower_incl(dO U^T)
//   dQt  = dO S^T + dP Kh
//   Dk   = T^T (-dU S^T) = -Dv S^T,   Dv = T^T dU
//   dA   = strict_lower(-Dk Wk^T - Dv Wv^T)
//   dKt  = diag(beta)(Dk + dA Kh)
//   dKh  = U dH^T diag(gamma) + dP^T Qt + dA^T diag(beta) Kt
//   dV   = diag(beta) Dv
//   dbeta_r = <Dk_r, Kt_r> + <Dv_r, V_r> + sum_{s<r} dA_rs Abar_rs
//   dGamma = dQt*Qt + dKt*Kt - dKh*Kh, and the last row gets
//            sum_j dH_cj S_next_cj (the chunk-end decay)
//   dq = dQt e^{Gamma},  dk = dKt e^{Gamma} + dKh e^{-Gamma},
//   dg_r = sum_{s>=r} dGamma_s, passed where g >= floor (0 below it).
//
// Launches (after a forward replay that keeps the state at every full chunk
// boundary):
//   kda_bwd_chunk : one workgroup per (chunk, head): the chunk record (the
//                   quantities above that do not involve the state), fp32
//                   (kda_bwd_chunk_fused at D = 128, which leaves v, dO and
//                   Gamma to be read from the inputs by the later passes).
//   kda_bwd_state : one workgroup per (sequence, head, 16 state columns):
//                   dS walked backward over the chunks (column j of dS only
//                   needs column j of dH and dO), writing every chunk's dH;
//                   the next chunk's operands load during the current step.
//   kda_bwd_local : one workgroup per (chunk, head): everything else
//                   (kda_bwd_local_fused at D = 128, with every intermediate
//                   on chip; through a scratch area at D = 64).
// Products run on fp32 MFMA (v_mfma_f32_16x16x4f32) on the fp32 path; on the
// bf16 path the record pass's, the walk's and the local gradients' take
// hi/lo bf16 MFMA (x = hi + lo to about 2^-16: see HL8), the inverse's
// small block products excepted.  In the
// per-chunk kernels the operands pass through LDS in k-slices (each element
// read once per product); the state-gradient pass keeps its operands in
// registers.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_launch.h"
#include "kda_rows.h"

namespace kda {
namespace {

constexpr int C = kChunk;
// Launches of the state-gradient walk in the overlapped call (one window):
// four, or two when a window spans at most kBwdShortSpan chunks of a
// sequence (at T = 4096, H = 16: 722 against 733 us; at T = 65,536 four
// parts take 10.9 against 11.1 ms).
constexpr int kBwdParts = 4, kBwdShortSpan = 64;

// Barrier for LDS hand-offs only: the waves' LDS operations are complete,
// global loads may still be in flight (__syncthreads() is a release fence and
// would first wait for every outstanding load, prefetches included).  The
// kernels keep __syncthreads() where a barrier orders global-memory data.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float ldx(const float* p) { return *p; }
__device__ __forceinline__ float ldx(const bf16_t* p) { return bf16_to_f32(*p); }
// four bf16 (first in the low half of u.x) to fp32
__device__ __forceinline__ f32x4 bf4_to_f32(const uint2& u) {
  return (f32x4){__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}
// four consecutive elements (p 8-byte aligned for bf16, 16-byte for fp32)
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 ld4(const bf16_t* p) { return bf4_to_f32(*(const uint2*)p); }
__device__ __forceinline__ void stx(float* p, float x) { *p = x; }
__device__ __forceinline__ void stx(bf16_t* p, float x) { *p = f32_to_bf16(x); }
// four consecutive elements (p 8-byte aligned for bf16, 16-byte for fp32)
__device__ __forceinline__ void st4(float* p, const f32x4& x) { *(f32x4*)p = x; }
__device__ __forceinline__ void st4(bf16_t* p, const f32x4& x) {
  *(uint2*)p = make_uint2(__builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[0], x[1])),
                          __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[2], x[3])));
}

// Operand views for one product: A is M x K, B is K x N.
struct MatA {
  const float* p;
  int ai, ak;
};
struct MatB {
  const float* p;
  int bk, bj;
  const float* bs;
};
__device__ __forceinline__ MatA rows(const float* p, int ld) { return MatA{p, ld, 1}; }      // X, X[i][k]
__device__ __forceinline__ MatA trans(const float* p, int ld) { return MatA{p, 1, ld}; }     // X^T, X[k][i]
__device__ __forceinline__ MatB krows(const float* p, int ld, const float* s = nullptr) {    // X, X[k][j]
  return MatB{p, ld, 1, s};
}
__device__ __forceinline__ MatB kcols(const float* p, int ld) { return MatB{p, 1, ld, nullptr}; }  // X^T, X[j][k]

// Mask of a stored tile element (row r, column c).
enum Mask { kFull = 0, kLowerIncl = 1, kStrictLower = 2 };

// Threads of the per-chunk kernels (eight waves).
constexpr int kThreads = 512;

// out[r][c] = alpha * (A1 B1 + A2 B2)[r][c] (+ out[r][c] when acc_in, + add[r][c]
// when add is given, add laid out like out), then column scale cs[c] if
// given, masked; 64 rows, N = 64 or 128 columns, K1,
// K2 multiples of 64 (A2 null: one product).  Called by every thread of a
// kThreads workgroup.
//
// The k range is walked in slices of KS = 64: the workgroup copies the
// slice's A (64 x KS) and B (KS x N) into LDS, each element read once from
// memory (B's per-k scale applied on the way), both stored k-contiguous so
// that every MFMA operand fragment is one 16-byte LDS read.  The next
// slice's loads are issued before the current slice's products.  Wave w
// owns row tile w / 2 and N / 32 consecutive column tiles of half w % 2, so
// one A fragment serves all of its tiles.  The lane layout is the one of
// kda_device.h: lane 16 g + i supplies row i of A and column i of B at
// k = 16 kk + 4 g + e in issue e, and holds D[4 g + r][i].
//
// HL (the bf16 path): each fp32 operand x is split into bf16 hi = rn(x) and
// lo = rn(x - hi) on its way into LDS, and a 32-wide k-block of the product
// is three bf16 MFMAs, A_hi B_hi + A_hi B_lo + A_lo B_hi (the dropped
// A_lo B_lo and the rounding of lo leave a relative error of about 2^-16
// per term, against the 2^-8 of a plain bf16 product).  The bf16 matrix
// rate is 16 times the fp32 one, so the three products take about a fifth
// of the time of fp32 MFMA.  In LDS, the element k of a 32-wide block sits
// at 8 (k / 4 % 4) + 4 (k / 16) + k % 4, so that the 8 elements a lane
// supplies (k = 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3) are 16
// contiguous bytes; rows are KSH = KS + 8 elements (36 dwords, so 8
// consecutive rows' 16-byte reads cover the 32 banks once).
constexpr int KS = 64, KSP = KS + 4, GM_ROWS = 64, KSH = KS + 8;
constexpr int kGemmLdsF32 = (GM_ROWS + 128) * KSP;      // floats, fp32 operands
constexpr int kGemmLdsHL = (GM_ROWS + 128) * KSH;       // floats: hi and lo bf16 planes
constexpr int kGemmLds = kGemmLdsF32 > kGemmLdsHL ? kGemmLdsF32 : kGemmLdsHL;  // the caller's buffer
// position of k (0 .. KS - 1) in an HL row
__device__ __forceinline__ int hl_pos(int k) { return (k & ~31) + 8 * ((k >> 2) & 3) + 4 * ((k >> 4) & 1) + (k & 3); }
template <int N, bool HL>
__device__ void gemm(float* lds, float* out, int ldo, float alpha, bool acc_in, Mask mask, const float* cs,
                     const MatA& A1, const MatB& B1, int K1, const MatA* A2, const MatB* B2, int K2,
                     const float* add = nullptr) {
  constexpr int M = GM_ROWS, NA = M * KS / kThreads, NB = N * KS / kThreads, NT = N / 32;
  static_assert(NA * kThreads == M * KS && NB * kThreads == N * KS, "slices tile the workgroup");
  static_assert(NA % 2 == 0 && NB % 2 == 0, "pairs of k");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int r0 = 16 * (wave >> 1), c0 = (wave & 1) * (N / 2);
  float ra[NA], rb[NB];
  f32x4 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if constexpr (!HL) {
    float(*sA)[KSP] = (float(*)[KSP])lds;
    float(*sB)[KSP] = (float(*)[KSP])(lds + M * KSP);
    auto fetch = [&](const MatA& A, const MatB& B, int k0) {
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const int x = tid + kThreads * e;
        const int r = A.ak == 1 ? x / KS : x % M, k = A.ak == 1 ? x % KS : x / M;
        ra[e] = A.p[r * A.ai + (k0 + k) * A.ak];
      }
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const int x = tid + kThreads * e;
        const int c = B.bk == 1 ? x / KS : x % N, k = B.bk == 1 ? x % KS : x / N;
        float val = B.p[(k0 + k) * B.bk + c * B.bj];
        if (B.bs) val *= B.bs[k0 + k];
        rb[e] = val;
      }
    };
    auto stash = [&](const MatA& A, const MatB& B) {
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const int x = tid + kThreads * e;
        const int r = A.ak == 1 ? x / KS : x % M, k = A.ak == 1 ? x % KS : x / M;
        sA[r][k] = ra[e];
      }
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const int x = tid + kThreads * e;
        const int c = B.bk == 1 ? x / KS : x % N, k = B.bk == 1 ? x % KS : x / N;
        sB[c][k] = rb[e];
      }
    };
    auto run = [&](const MatA& A, const MatB& B, int K) {
      fetch(A, B, 0);
      for (int k0 = 0; k0 < K; k0 += KS) {
        lds_barrier();  // every wave is done with the previous slice
        stash(A, B);
        lds_barrier();
        if (k0 + KS < K) fetch(A, B, k0 + KS);
#pragma unroll
        for (int kk = 0; kk < KS / 16; ++kk) {
          const f32x4 a = *(const f32x4*)&sA[r0 + i][16 * kk + 4 * g];
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            const f32x4 b = *(const f32x4*)&sB[c0 + 16 * u + i][16 * kk + 4 * g];
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc[u], 0, 0, 0);
          }
        }
      }
    };
    run(A1, B1, K1);
    if (A2) run(*A2, *B2, K2);
  } else {
    // planes: A hi, A lo ([M][KSH] each), B hi, B lo ([N][KSH] each), bf16
    bf16_t* sAh = (bf16_t*)lds;
    bf16_t* sAl = sAh + M * KSH;
    bf16_t* sBh = sAl + M * KSH;
    bf16_t* sBl = sBh + N * KSH;
    // thread pair p holds two consecutive k of one row (A) or column (B):
    // elements 2 p and 2 p + 1 of ra / rb
    auto fetch = [&](const MatA& A, const MatB& B, int k0) {
#pragma unroll
      for (int e = 0; e < NA / 2; ++e) {
        const int x = tid + kThreads * e;
        if (A.ak == 1) {  // k contiguous: one 8-byte load
          const int r = x / (KS / 2), k = 2 * (x % (KS / 2));
          const float2 v2 = *(const float2*)&A.p[r * A.ai + k0 + k];
          ra[2 * e] = v2.x;
          ra[2 * e + 1] = v2.y;
        } else {  // rows contiguous across the threads
          const int r = x % M, k = 2 * (x / M);
          ra[2 * e] = A.p[r * A.ai + (k0 + k) * A.ak];
          ra[2 * e + 1] = A.p[r * A.ai + (k0 + k + 1) * A.ak];
        }
      }
#pragma unroll
      for (int e = 0; e < NB / 2; ++e) {
        const int x = tid + kThreads * e;
        int k;
        if (B.bk == 1) {
          const int c = x / (KS / 2);
          k = 2 * (x % (KS / 2));
          const float2 v2 = *(const float2*)&B.p[k0 + k + c * B.bj];
          rb[2 * e] = v2.x;
          rb[2 * e + 1] = v2.y;
        } else {
          const int c = x % N;
          k = 2 * (x / N);
          rb[2 * e] = B.p[(k0 + k) * B.bk + c * B.bj];
          rb[2 * e + 1] = B.p[(k0 + k + 1) * B.bk + c * B.bj];
        }
        if (B.bs) {
          rb[2 * e] *= B.bs[k0 + k];
          rb[2 * e + 1] *= B.bs[k0 + k + 1];
        }
      }
    };
    // hi and lo of a pair as two packed bf16 words
    auto split = [](float x0, float x1, uint32_t& hi, uint32_t& lo) {
      hi = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x0, x1));
      lo = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x0 - __uint_as_float(hi << 16),
                                                        x1 - __uint_as_float(hi & 0xffff0000u)));
    };
    auto stash = [&](const MatA& A, const MatB& B) {
#pragma unroll
      for (int e = 0; e < NA / 2; ++e) {
        const int x = tid + kThreads * e;
        const int r = A.ak == 1 ? x / (KS / 2) : x % M, k = A.ak == 1 ? 2 * (x % (KS / 2)) : 2 * (x / M);
        uint32_t hi, lo;
        split(ra[2 * e], ra[2 * e + 1], hi, lo);
        const int o = r * KSH + hl_pos(k);  // even: the pair is one 32-bit word
        *(uint32_t*)&sAh[o] = hi;
        *(uint32_t*)&sAl[o] = lo;
      }
#pragma unroll
      for (int e = 0; e < NB / 2; ++e) {
        const int x = tid + kThreads * e;
        const int c = B.bk == 1 ? x / (KS / 2) : x % N, k = B.bk == 1 ? 2 * (x % (KS / 2)) : 2 * (x / N);
        uint32_t hi, lo;
        split(rb[2 * e], rb[2 * e + 1], hi, lo);
        const int o = c * KSH + hl_pos(k);
        *(uint32_t*)&sBh[o] = hi;
        *(uint32_t*)&sBl[o] = lo;
      }
    };
    auto run = [&](const MatA& A, const MatB& B, int K) {
      fetch(A, B, 0);
      for (int k0 = 0; k0 < K; k0 += KS) {
        lds_barrier();  // every wave is done with the previous slice
        stash(A, B);
        lds_barrier();
        if (k0 + KS < K) fetch(A, B, k0 + KS);
#pragma unroll
        for (int kb = 0; kb < KS / 32; ++kb) {
          const int oa = (r0 + i) * KSH + 32 * kb + 8 * g;
          const bf16x8 ah = *(const bf16x8*)&sAh[oa], al = *(const bf16x8*)&sAl[oa];
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            const int ob = (c0 + 16 * u + i) * KSH + 32 * kb + 8 * g;
            const bf16x8 bh = *(const bf16x8*)&sBh[ob], bl = *(const bf16x8*)&sBl[ob];
            acc[u] = mma(ah, bh, acc[u]);
            acc[u] = mma(ah, bl, acc[u]);
            acc[u] = mma(al, bh, acc[u]);
          }
        }
      }
    };
    run(A1, B1, K1);
    if (A2) run(*A2, *B2, K2);
  }
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int c = c0 + 16 * u + i;
    const float sc = cs ? cs[c] : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + 4 * g + e;
      float* dst = out + r * ldo + c;
      float x = alpha * acc[u][e];
      if (acc_in) x += *dst;
      if (add) x += add[r * ldo + c];
      x *= sc;
      const bool keep = mask == kFull || (mask == kLowerIncl ? r >= c : r > c);
      *dst = keep ? x : 0.f;
    }
  }
}

// Floats of one (chunk, head) record at key/value width D: Qt, Kt, Kh, V,
// dO, Wk, Wv, Gamma ([C][D] each, rows past the chunk's end zero; Gamma
// there repeats the last row), P, T, Abar ([C][C]), gamma [D], beta [C] (0
// past the end).
template <int D> struct RecBase {
  static constexpr int QT = 0, KT = C * D, KH = 2 * C * D, WK = 3 * C * D, WV = 4 * C * D, PM = 5 * C * D,
                       TM = PM + C * C, AB = TM + C * C, GAM = AB + C * C, BET = GAM + D, END = BET + C;
};
// At D = 64 the record also holds copies of v and dO and Gamma for the
// products of kda_bwd_local.  At D = 128 it does not: the record pass is
// bound by its writes, and the walk and kda_bwd_local_fused read v and dO
// from the inputs and sum Gamma from the gate themselves.
template <int D> struct Rec : RecBase<D> {
  static constexpr int VV = RecBase<D>::END, DO = VV + C * D, GM = DO + C * D, FLOATS = GM + C * D;
};
template <> struct Rec<128> : RecBase<128> {
  static constexpr int FLOATS = END;
};
// How the per-chunk kernels split the rows of a chunk for the prefix sums
// over rows: NG groups of RG rows, one thread per (group, channel).
template <int D> struct RowSplit {
  static constexpr int NG = kThreads / D, RG = C / NG;
  static_assert(NG * D == kThreads && NG * RG == C, "row groups tile the chunk");
};
// Floats of one (chunk, head) scratch area of kda_bwd_local: U (then Dk),
// dU (then E = Dk + dA Kh), Dv, dQt, dKh ([C][D] each), dP, dA ([C][C]),
// dgamma-last [D].
template <int D> struct Scr {
  static constexpr int U = 0, DU = C * D, DV = 2 * C * D, DQT = 3 * C * D, DKH = 4 * C * D, DP = 5 * C * D,
                       DA = DP + C * C, DGL = DA + C * C, FLOATS = DGL + D;
};

// Chunk `slot` of the call (slots count the chunks of all sequences in
// order) as sequence n, chunk m of nc, tokens [tok0, tok0 + len), and the
// first prefix-state slot of its sequence (full chunks of the earlier
// sequences).  Returns false past the last chunk.
struct ChunkPos {
  int n, m, nc, len;
  int64_t tok0, st0;
};
// Per-sequence prefix sums of a packed batch (kda_bwd_seqs): seqs[n] = chunks
// of sequences 0 .. n-1 (the first chunk slot of sequence n), and
// seqs[n_rows + 1 + n] = full chunks of sequences 0 .. n-1 (the first
// prefix-state slot of sequence n, the layout of kda_chunk_forward_states).
// A chunk slot finds its sequence by binary search over the first array.
__device__ bool chunk_pos(int64_t slot, const int32_t* cu, const int64_t* seqs, int n_rows, int T_per,
                          ChunkPos* p) {
  if (!cu) {
    const int64_t per = (T_per + C - 1) / C;
    if (per == 0 || slot >= per * n_rows) return false;
    p->n = (int)(slot / per);
    p->m = (int)(slot % per);
    p->nc = (int)per;
    p->tok0 = (int64_t)p->n * T_per + (int64_t)p->m * C;
    p->len = min(C, T_per - p->m * C);
    p->st0 = (int64_t)p->n * (T_per / C);
    return true;
  }
  if (n_rows == 0 || slot >= seqs[n_rows]) return false;
  // the largest n with seqs[n] <= slot: that sequence is not empty
  int lo = 0, hi = n_rows - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (seqs[mid] <= slot) lo = mid;
    else hi = mid - 1;
  }
  const int n = lo;
  const int64_t L = (int64_t)cu[n + 1] - cu[n];
  p->n = n;
  p->m = (int)(slot - seqs[n]);
  p->nc = (int)((L + C - 1) / C);
  p->tok0 = (int64_t)cu[n] + (int64_t)p->m * C;
  p->len = (int)min((int64_t)C, L - (int64_t)p->m * C);
  p->st0 = seqs[n_rows + 1 + n];
  return true;
}

// The prefix sums above, for n_rows sequences: one workgroup, each thread
// summing a contiguous range of sequences, then the ranges' offsets.
__global__ void __launch_bounds__(256) kda_bwd_seqs(const int32_t* __restrict__ cu, int n_rows,
                                                    int64_t* __restrict__ seqs) {
  __shared__ int64_t part[2][256];
  const int tid = threadIdx.x, per = (n_rows + 255) / 256;
  const int n0 = min(n_rows, tid * per), n1 = min(n_rows, n0 + per);
  int64_t a = 0, f = 0;
  for (int n = n0; n < n1; ++n) {
    const int64_t L = (int64_t)cu[n + 1] - cu[n];
    a += (L + C - 1) / C;
    f += L / C;
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
    const int64_t L = (int64_t)cu[n + 1] - cu[n];
    oa += (L + C - 1) / C;
    of += L / C;
  }
  if (tid == 255) {
    seqs[n_rows] = oa;  // every chunk (the last thread's range ends at n_rows)
    seqs[2 * n_rows + 1] = of;
  }
}

// The window a launch works in: chunk indices [lo, hi) of every sequence,
// chunk m of sequence n at area slot n width + (m - lo).  width = 0: one
// window (lo = 0, hi unbounded), the area slot is the chunk's slot of the
// call.  The per-chunk records, scratch and end-state gradients are indexed
// by area slot.
struct Win {
  int64_t lo, hi, width;
};
__device__ __forceinline__ int64_t area_slot(const Win& w, int64_t n, int64_t base, int64_t m) {
  return w.width ? n * w.width + (m - w.lo) : base + m;
}

// The chunk at area slot a of window w; false for a slot no chunk has.
__device__ bool chunk_pos_win(int64_t a, const Win& w, const int32_t* cu, const int64_t* seqs, int n_rows, int T_per,
                              ChunkPos* p) {
  if (w.width == 0) return chunk_pos(a, cu, seqs, n_rows, T_per, p);
  const int64_t n = a / w.width, m = w.lo + a % w.width;
  if (n >= n_rows || m >= w.hi) return false;
  int64_t L, tok, st0;
  if (cu) {
    L = (int64_t)cu[n + 1] - cu[n];
    tok = cu[n];
    st0 = seqs[n_rows + 1 + n];
  } else {
    L = T_per;
    tok = n * T_per;
    st0 = n * (T_per / C);
  }
  const int64_t nc = (L + C - 1) / C;
  if (m >= nc) return false;
  p->n = (int)n;
  p->m = (int)m;
  p->nc = (int)nc;
  p->tok0 = tok + m * C;
  p->len = (int)min((int64_t)C, L - m * C);
  p->st0 = st0;
  return true;
}

// Same position, found once per workgroup by thread 0 and shared via LDS.
__device__ bool chunk_pos_shared(int64_t a, const Win& w, const int32_t* cu, const int64_t* seqs, int n_rows,
                                 int T_per, ChunkPos* sh) {
  __shared__ int ok;
  if (threadIdx.x == 0) ok = chunk_pos_win(a, w, cu, seqs, n_rows, T_per, sh) ? 1 : 0;
  __syncthreads();
  return ok != 0;
}

__device__ __forceinline__ float gate_at(const void* g, int gate, bool bf16, int64_t th, int D, int c) {
  if (gate == kGateNone) return 0.f;
  const int64_t idx = gate == kGateChannel ? th * D + c : th;
  return bf16 ? bf16_to_f32(((const bf16_t*)g)[idx]) : ((const float*)g)[idx];
}

// ---------------------------------------------------------------------------
// Chunk record: Gamma and the scaled rows, the two Gram blocks, the inverse
// by forward substitution, Wk and Wv.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads) kda_bwd_chunk(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const void* __restrict__ g,
                                                     const float* __restrict__ beta, const T* __restrict__ dout,
                                                     const int32_t* __restrict__ cu, const int64_t* __restrict__ seqs,
                                                     int n_rows, int T_per, int H,
                                                     float g_floor, int gate, float* __restrict__ rec,
                                                     float* __restrict__ zero_state, Win win) {
  typedef Rec<D> R;
  constexpr bool HL = sizeof(T) == 2;  // bf16 path: products on hi/lo bf16 MFMA
  __shared__ ChunkPos pos;
  // the products' slices, and later (once the Gram products are done) the
  // inverse's operands diag(beta) Abar and T
  constexpr int kLds = kGemmLds > 2 * C * (C + 1) ? kGemmLds : 2 * C * (C + 1);
  __shared__ __align__(16) float lds[kLds];
  float(*As)[C + 1] = (float(*)[C + 1])lds;
  float(*Ts)[C + 1] = (float(*)[C + 1])(lds + C * (C + 1));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int64_t slot = blockIdx.x;
  if (slot == 0 && h == 0 && win.lo == 0)
    for (int x = tid; x < D * D; x += blockDim.x) zero_state[x] = 0.f;
  if (!chunk_pos_shared(slot, win, cu, seqs, n_rows, T_per, &pos)) return;
  float* Rp = rec + (slot * H + h) * (int64_t)R::FLOATS;
  const bool bf = sizeof(T) == 2;
  const int len = pos.len;

  // element-wise.  Gamma: per channel, each group of RG rows takes its own
  // prefix sums, then adds the sums of the groups before it.
  {
    typedef RowSplit<D> RS;
    __shared__ float gsum[RS::NG][D];
    const int c = tid % D, grp = tid / D, r0 = grp * RS::RG;
    float gl[RS::RG];
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < RS::RG; ++i) {
      const int r = r0 + i;
      if (r < len) run += fmaxf(gate_at(g, gate, bf, (pos.tok0 + r) * H + h, D, c), g_floor);
      gl[i] = run;
    }
    gsum[grp][c] = run;
    __syncthreads();
    float off = 0.f;
    for (int j = 0; j < grp; ++j) off += gsum[j][c];
#pragma unroll
    for (int i = 0; i < RS::RG; ++i) {
      const int r = r0 + i;
      float qv = 0.f, kv = 0.f;
      if (r < len) {
        const int64_t th = (pos.tok0 + r) * H + h;
        qv = ldx(q + th * D + c);
        kv = ldx(k + th * D + c);
      }
      const float G = off + gl[i];
      const float e = __expf(G), ei = __expf(-G);
      const int x = r * D + c;
      Rp[R::GM + x] = G;
      Rp[R::QT + x] = qv * e;
      Rp[R::KT + x] = kv * e;
      Rp[R::KH + x] = kv * ei;
      if (r == C - 1) Rp[R::GAM + c] = e;
    }
  }
  for (int x = tid; x < C * D; x += blockDim.x) {
    const int r = x / D, c = x % D;
    const int64_t th = (pos.tok0 + r) * H + h;
    Rp[R::VV + x] = r < len ? ldx(v + th * D + c) : 0.f;
    Rp[R::DO + x] = r < len ? ldx(dout + th * D + c) : 0.f;
  }
  if (tid < C) Rp[R::BET + tid] = tid < len ? beta[(pos.tok0 + tid) * H + h] : 0.f;
  __syncthreads();

  // Abar = strict_lower(Kt Kh^T), P = lower_incl(Qt Kh^T)
  gemm<C, HL>(lds, Rp + R::AB, C, 1.f, false, kStrictLower, nullptr, rows(Rp + R::KT, D), kcols(Rp + R::KH, D), D,
       nullptr, nullptr, 0);
  gemm<C, HL>(lds, Rp + R::PM, C, 1.f, false, kLowerIncl, nullptr, rows(Rp + R::QT, D), kcols(Rp + R::KH, D), D,
       nullptr, nullptr, 0);
  __syncthreads();
  for (int x = tid; x < C * C; x += blockDim.x) {
    const int r = x / C, c = x % C;
    As[r][c] = Rp[R::BET + r] * Rp[R::AB + x];
    Ts[r][c] = r == c ? 1.f : 0.f;
  }
  __syncthreads();
  // T = (I + A)^{-1}, A strictly lower, over 4 x 4 blocks of 16.  Diagonal
  // blocks by forward substitution, one lane per column:
  //   T[r][s] = -sum_{s <= m < r} A[r][m] T[m][s]   (s < r in the same block)
  if (tid < C) {
    const int s = tid, end = (s | 15) + 1;
    for (int r = s + 1; r < end; ++r) {
      float acc = 0.f;
      for (int m = s; m < r; ++m) acc += As[r][m] * Ts[m][s];
      Ts[r][s] = -acc;
    }
  }
  __syncthreads();
  // then block row i from the rows above it, one wave per block (i, j < i):
  //   T_ij = -T_ii sum_{j <= m < i} A_im T_mj
  // two 16 x 16 MFMA products; the first one's accumulator is the second
  // one's B operand as it stands (its rows run over k).
  for (int bi = 1; bi < C / 16; ++bi) {
    if (wave < bi) {
      const int bj = wave, ii = lane & 15, g = lane >> 4;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int bm = bj; bm < bi; ++bm)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = 16 * bm + 4 * g + e;  // issue e: lane group g supplies k = 4 g + e of the block
          x = __builtin_amdgcn_mfma_f32_16x16x4f32(As[16 * bi + ii][kk], Ts[kk][16 * bj + ii], x, 0, 0, 0);
        }
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(Ts[16 * bi + ii][16 * bi + 4 * g + e], x[e], y, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ts[16 * bi + 4 * g + e][16 * bj + ii] = -y[e];
    }
    __syncthreads();
  }
  for (int x = tid; x < C * C; x += blockDim.x) Rp[R::TM + x] = Ts[x / C][x % C];
  __syncthreads();
  // Wk = T diag(beta) Kt, Wv = T diag(beta) V
  gemm<D, HL>(lds, Rp + R::WK, D, 1.f, false, kFull, nullptr, rows(Rp + R::TM, C), krows(Rp + R::KT, D, Rp + R::BET), C,
       nullptr, nullptr, 0);
  gemm<D, HL>(lds, Rp + R::WV, D, 1.f, false, kFull, nullptr, rows(Rp + R::TM, C), krows(Rp + R::VV, D, Rp + R::BET), C,
       nullptr, nullptr, 0);
}

// fp32 operand fragment of a 16 x 16 x 4 product taken down a column:
// X[k0 + 4 g + e][c] in issue e (frag_rows takes it along a row).
__device__ __forceinline__ f32x4 frag_cols(const float* X, int ld, int c, int k0, int g) {
  const float* p = X + (k0 + 4 * g) * ld + c;
  return (f32x4){p[0], p[ld], p[2 * ld], p[3 * ld]};
}
// hi/lo bf16 operands of the 16 x 16 x 32 products on the bf16 path: x ~ hi
// + lo to about 2^-16, a 32-wide k-block as A_hi B_hi + A_hi B_lo + A_lo
// B_hi (three bf16 MFMAs against eight fp32 16 x 16 x 4 for the same k).
struct HL8 {
  bf16x8 h, l;
};
__device__ __forceinline__ void split4(const f32x4& x, uint2& hi, uint2& lo) {
  const uint32_t a = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[0], x[1]));
  const uint32_t b = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[2], x[3]));
  hi = make_uint2(a, b);
  lo = make_uint2(__builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[0] - __uint_as_float(a << 16),
                                                               x[1] - __uint_as_float(a & 0xffff0000u))),
                  __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x[2] - __uint_as_float(b << 16),
                                                               x[3] - __uint_as_float(b & 0xffff0000u))));
}
// the fragment of a lane from its k = 4 g .. 4 g + 3 (x0) and 16 + 4 g ..
// 16 + 4 g + 3 (x1) of a 32-wide k-block
__device__ __forceinline__ HL8 hl_of(const f32x4& x0, const f32x4& x1) {
  uint2 h0, l0, h1, l1;
  split4(x0, h0, l0);
  split4(x1, h1, l1);
  return HL8{__builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y)),
             __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y))};
}
__device__ __forceinline__ f32x4 mma3(const HL8& a, const HL8& b, f32x4 c) {
  c = mma(a.h, b.h, c);
  c = mma(a.h, b.l, c);
  return mma(a.l, b.h, c);
}
// the lower-triangular 16 x 16 tiles (a, b), b <= a, of a 64 x 64 matrix
__device__ __forceinline__ void low_tile(int t, int& a, int& b) {
  a = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
  b = t - a * (a + 1) / 2;
}

// Chunk record at D = 128 in one pass with the operands on chip: q, k, v
// and the gate are read once, Qt, Kt and Kh built in LDS, and the Gram
// blocks, the inverse, Wk and Wv computed from there (the Gram blocks, Wk
// and Wv on hi/lo bf16 MFMA, the inverse's block rows on fp32 MFMA).  The
// pass is bound by its writes, so the record gets only what the later passes
// cannot take from the inputs (no copies of v and dO, no Gamma).  LDS: three
// [64][D + 4] fp32 arrays (Qt, Kt, Kh; the first one holds diag(beta) V once
// the Gram products are done) and [64][65] diag(beta) Abar, T and P.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads) kda_bwd_chunk_fused(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const void* __restrict__ g,
                                                           const float* __restrict__ beta,
                                                           const T* __restrict__ /* dout: not copied */,
                                                           const int32_t* __restrict__ cu,
                                                           const int64_t* __restrict__ seqs, int n_rows, int T_per,
                                                           int H, float g_floor, int gate, float* __restrict__ rec,
                                                           float* __restrict__ zero_state, Win win) {
  static_assert(sizeof(T) == 2, "the bf16 path (inputs read as pairs)");
  typedef Rec<D> R;
  // element-wise mapping of the forward's input rows (Raw): thread (part, cp)
  // takes channels 2 cp, 2 cp + 1 of rows RP part .. RP part + RP - 1
  constexpr int NPR = D / 2, NPART = kThreads / NPR, RP = C / NPART;
  static_assert(NPART * NPR == kThreads && RP == 8, "the row groups of Raw");
  constexpr int LX = D + 4, AX = C * LX;
  __shared__ ChunkPos pos;
  __shared__ __align__(16) float lds[3 * AX];
  __shared__ float As[C][C + 1], Ts[C][C + 1], Ps[C][C + 1];
  __shared__ float2 gsum[NPART][NPR];
  __shared__ float sb[C];
  float* const LQ = lds;
  float* const LK = lds + AX;
  float* const LH = lds + 2 * AX;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, gq = lane >> 4, i = lane & 15;
  const int h = blockIdx.y;
  const int64_t slot = blockIdx.x;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  if (slot == 0 && h == 0 && win.lo == 0)
    for (int x = tid; x < D * D; x += blockDim.x) zero_state[x] = 0.f;
  if (!chunk_pos_shared(slot, win, cu, seqs, n_rows, T_per, &pos)) return;
  float* Rp = rec + (slot * H + h) * (int64_t)R::FLOATS;
  const int len = pos.len;
  const int cp = tid % NPR, part = tid / NPR, c0 = 2 * cp, r0 = RP * part;
  // Gamma: each row group takes its own prefix sums of the floored
  // log-decays, then adds the totals of the groups before it
  // (kda_bwd_local_fused sums them in the same order)
  typedef PairT<T> PW;
  // the inputs: branch-free buffer loads, all issued before the first use
  // (rows past the chunk's end read as zeros)
  Raw<T, D, true, false, false> raw;
  raw.load(ChunkInputs{q, k, v, g, beta, nullptr, nullptr, nullptr}, pos.tok0, len, H, h, tid, gate);
  float2 gl[RP];
  {
    if (tid < C) sb[tid] = raw.beta;
    const bool gh = gate == kGateHead;  // one log-decay per row, for both channels
    float2 run = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      if (r0 + j < len) {
        const float x = PW::lo(raw.g[j]);
        run.x += fmaxf(x, g_floor);
        run.y += fmaxf(gh ? x : PW::hi(raw.g[j]), g_floor);
      }
      gl[j] = run;
    }
    gsum[part][cp] = run;
    for (int x = tid; x < C * C; x += kThreads) {
      const int r = x / C, s2 = x % C;
      Ts[r][s2] = r == s2 ? 1.f : 0.f;
    }
    __syncthreads();
    float2 off = {0.f, 0.f};
    for (int j = 0; j < part; ++j) {
      off.x += gsum[j][cp].x;
      off.y += gsum[j][cp].y;
    }
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      const int r = r0 + j;
      const float G0 = off.x + gl[j].x, G1 = off.y + gl[j].y;
      const float e0 = __expf(G0), e1 = __expf(G1);
      const float i0 = __expf(-G0), i1 = __expf(-G1);
      const float q0 = PW::lo(raw.qw(j)), q1 = PW::hi(raw.qw(j));
      const float k0 = PW::lo(raw.kw(j)), k1 = PW::hi(raw.kw(j));
      *(float2*)&LQ[r * LX + c0] = make_float2(q0 * e0, q1 * e1);
      *(float2*)&LK[r * LX + c0] = make_float2(k0 * e0, k1 * e1);
      *(float2*)&LH[r * LX + c0] = make_float2(k0 * i0, k1 * i1);
      if (r == C - 1) *(float2*)&Rp[R::GAM + c0] = make_float2(e0, e1);
    }
  }
  if (tid < C) Rp[R::BET + tid] = sb[tid];
  __syncthreads();
  // Abar = strict_lower(Kt Kh^T), P = lower_incl(Qt Kh^T): the 10 tiles of
  // the lower triangle of each, one wave per tile
  for (int t = w; t < 20; t += kThreads / 64) {
    const bool isP = t < 10;
    int ta, tb;
    low_tile(isP ? t : t - 10, ta, tb);
    const float* XA = isP ? LQ : LK;
    f32x4 acc = z4;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      acc = mma3(hl_of(frag_rows(XA, LX, 16 * ta + i, 32 * kb, gq), frag_rows(XA, LX, 16 * ta + i, 32 * kb + 16, gq)),
                 hl_of(frag_rows(LH, LX, 16 * tb + i, 32 * kb, gq), frag_rows(LH, LX, 16 * tb + i, 32 * kb + 16, gq)),
                 acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ta + 4 * gq + e, s2 = 16 * tb + i;
      if (isP) {
        Ps[r][s2] = (ta > tb || 4 * gq + e >= i) ? acc[e] : 0.f;
      } else {
        const float a = (ta > tb || 4 * gq + e > i) ? acc[e] : 0.f;
        Rp[R::AB + r * C + s2] = a;
        As[r][s2] = sb[r] * a;
      }
    }
  }
  __syncthreads();
  // T = (I + A)^{-1} (A = diag(beta) Abar strictly lower) over 4 x 4 blocks
  // of 16, as in kda_bwd_chunk: diagonal blocks by forward substitution, one
  // lane of wave 0 per column, then the blocks below them one block row at a
  // time.  Lane s keeps column s of its diagonal block in registers (zero
  // above the diagonal: the sums start at the same term as the plain
  // substitution), so that a step waits on no LDS round trip; meanwhile the
  // other waves write Qt, Kt, Kh as rows, P, and the upper tiles of Abar (zero).
  if (w == 0) {
    const int o = 16 * (tid >> 4), j = tid & 15;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = r == j ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) acc += As[o + r][o + m] * t[m];
      if (r > j) t[r] = -acc;
    }
#pragma unroll
    for (int r = 1; r < 16; ++r)
      if (r > j) Ts[o + r][o + j] = t[r];
  } else {
    constexpr int NT = kThreads - 64;
    for (int x = tid - 64; x < C * D / 4; x += NT) {
      const int r = x / (D / 4), c4 = 4 * (x % (D / 4));
      *(f32x4*)&Rp[R::QT + r * D + c4] = *(const f32x4*)&LQ[r * LX + c4];
      *(f32x4*)&Rp[R::KT + r * D + c4] = *(const f32x4*)&LK[r * LX + c4];
      *(f32x4*)&Rp[R::KH + r * D + c4] = *(const f32x4*)&LH[r * LX + c4];
    }
    for (int x = tid - 64; x < C * C; x += NT) {
      const int r = x / C, s2 = x % C;
      const bool up = (s2 >> 4) > (r >> 4);
      Rp[R::PM + x] = up ? 0.f : Ps[r][s2];
      if (up) Rp[R::AB + x] = 0.f;
    }
  }
  __syncthreads();
  // diag(beta) V over Qt (every thread is past the row stores)
#pragma unroll
  for (int j = 0; j < RP; ++j)
    *(float2*)&LQ[(r0 + j) * LX + c0] =
        make_float2(sb[r0 + j] * PW::lo(raw.vw(j)), sb[r0 + j] * PW::hi(raw.vw(j)));
  for (int bi = 1; bi < C / 16; ++bi) {
    if (w < bi) {
      const int bj = w;
      f32x4 x = z4;
      for (int bm = bj; bm < bi; ++bm)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = 16 * bm + 4 * gq + e;
          x = __builtin_amdgcn_mfma_f32_16x16x4f32(As[16 * bi + i][kk], Ts[kk][16 * bj + i], x, 0, 0, 0);
        }
      f32x4 y = z4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(Ts[16 * bi + i][16 * bi + 4 * gq + e], x[e], y, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ts[16 * bi + 4 * gq + e][16 * bj + i] = -y[e];
    }
    __syncthreads();
  }
  for (int x = tid; x < C * C; x += kThreads) Rp[R::TM + x] = Ts[x / C][x % C];
  // Wk = T diag(beta) Kt, Wv = T diag(beta) V: wave w takes columns 16 w ..
  // 16 w + 15 of both, every row tile (T is lower triangular: row tile rt
  // needs the 32-wide k-blocks kb <= rt / 2 only, whose tiles above the
  // diagonal are zeros in Ts)
  const int cw = 16 * w;
  f32x4 wk[4] = {z4, z4, z4, z4}, wv[4] = {z4, z4, z4, z4};
  auto sb4 = [&](int k0) { return (f32x4){sb[k0], sb[k0 + 1], sb[k0 + 2], sb[k0 + 3]}; };
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb) {
    const int k0 = 32 * kb + 4 * gq, k1 = k0 + 16;
    const HL8 bk = hl_of(frag_cols(LK, LX, cw + i, 32 * kb, gq) * sb4(k0),
                         frag_cols(LK, LX, cw + i, 32 * kb + 16, gq) * sb4(k1));
    const HL8 bv = hl_of(frag_cols(LQ, LX, cw + i, 32 * kb, gq), frag_cols(LQ, LX, cw + i, 32 * kb + 16, gq));
#pragma unroll
    for (int rt = 2 * kb; rt < 4; ++rt) {
      const int r = 16 * rt + i;
      const HL8 a = hl_of((f32x4){Ts[r][k0], Ts[r][k0 + 1], Ts[r][k0 + 2], Ts[r][k0 + 3]},
                          (f32x4){Ts[r][k1], Ts[r][k1 + 1], Ts[r][k1 + 2], Ts[r][k1 + 3]});
      wk[rt] = mma3(a, bk, wk[rt]);
      wv[rt] = mma3(a, bv, wv[rt]);
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = (16 * rt + 4 * gq + e) * D + cw + i;
      Rp[R::WK + x] = wk[rt][e];
      Rp[R::WV + x] = wv[rt][e];
    }
}

// ---------------------------------------------------------------------------
// Reverse pass over the chunks of one sequence for 16 columns of dS.
//
// Fragments of one 16-row (or 16-column) panel over a full k range, loaded
// in one go: A(i, k) = p[i * ai + k * ak] (lane row i, k = 16 kk + 4 g + e).
template <int NK>
__device__ __forceinline__ void load_panel(f32x4 (&f)[NK], const float* p, int ai, int ak, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const float* q = p + i * ai + 4 * g * ak;
  if (ak == 1) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) f[kk] = *(const f32x4*)(q + 16 * kk);
  } else {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const float* r = q + 16 * kk * ak;
      f[kk] = (f32x4){r[0], r[ak], r[2 * ak], r[3 * ak]};
    }
  }
}
// HL: on hi/lo bf16 MFMA, the panels split as they are used (k-blocks of
// 32: fragments 2 kb and 2 kb + 1), else on fp32 MFMA
template <bool HL, int NK>
__device__ __forceinline__ f32x4 mma_panels(f32x4 acc, const f32x4 (&a)[NK], const f32x4 (&b)[NK]) {
  if constexpr (HL) {
    static_assert(NK % 2 == 0, "whole 32-wide k-blocks");
#pragma unroll
    for (int kb = 0; kb < NK / 2; ++kb) acc = mma3(hl_of(a[2 * kb], a[2 * kb + 1]), hl_of(b[2 * kb], b[2 * kb + 1]), acc);
  } else {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk][0], b[kk][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk][1], b[kk][1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk][2], b[kk][2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk][3], b[kk][3], acc, 0, 0, 0);
    }
  }
  return acc;
}

// One workgroup per (sequence, head, 16 state columns), eight waves.  With
// dH the gradient of a chunk's end state (these 16 columns) and
// G = diag(gamma) dH, a step is
//   dU = P^T dO + Kh G,   dH_in = G + Qt^T dO - Wk^T dU.
// Row tile t (of 4) of dU is split over k between waves t and t + 4, each
// taking half of P^T dO and half of Kh G; the two partial tiles sit in LDS
// and are added where dU is read.  Wave w < D / 16 owns row tile w of dH.
// Every record operand of the next chunk (the step's k-panels and the gamma
// of the wave's own rows) is loaded while the current chunk is computed, so
// the chain of chunks waits on memory once, not once per step.  For that
// every wave issues the same loads on every step (46 at d = 128 on waves 0-3,
// which also load the dO columns for all, 45 on the others: below the 63 that
// the hardware counts, so that waiting for the current operands never means
// waiting for the next ones).  Workgroups are ordered so that the column
// blocks of one (sequence, head) pair have the same block index mod 8, i.e.
// share one XCD's L2 (the record operands are common to them).
template <int D> struct StateOps {
  static constexpr int NKC = C / 16, NKH = D / 32, NKP = C / 32;
  f32x4 aP[NKP], aKh[NKH], aQ[NKC], aW[NKC];
  uint4 bOw;  // waves 0-3: dO[tid / 4][j0 + 4 (tid % 4) ..] as loaded, shared through LDS
  // the dH values this set's step stored, held until the next step's dU
  // products are issued: a store's data registers cannot be reused before
  // it completes, so reusing them at once would make the next step wait
  // for the stores
  float keep[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 gr;   // gamma of rows 16 w + 4 g + e (this wave's dH tile)
  // gamma first: a step needs the next chunk's gamma before its other operands
  // (loads complete in issue order).  Waves past D / 16 (d = 64) load a
  // copy of another wave's dH operands and do not use them.  The dO columns
  // every wave needs whole are loaded once, from the input, a row piece of
  // four elements per thread of waves 0-3 (put; rows past the end of the
  // sequence read as zeros, with no branch: a masked load would make the
  // wave wait for every load in flight): sixteen fewer load instructions
  // per wave and step on an address unit that sets the step time.
  template <typename T>
  __device__ void load(const float* Rp, const ChunkRows<T>& dO, int j0, int wave, int lane) {
    typedef Rec<D> R;
    const int t = wave & 3, half = wave >> 2, w = wave % (D / 16), tid = 64 * wave + lane;
    gr = *(const f32x4*)(Rp + R::GAM + 16 * w + 4 * (lane >> 4));
    if (wave < 4) bOw = dO.raw4(tid >> 2, j0 + 4 * (tid & 3));
    load_panel(aKh, Rp + R::KH + 16 * t * D + half * (D / 2), D, 1, lane);      // Kh rows 16 t.., k in this half
    load_panel(aP, Rp + R::PM + half * (C / 2) * C + 16 * t, 1, C, lane);       // P^T rows 16 t.., k in this half
  }
  // the dH products' panels, issued later in the step than the others so
  // that the address unit works through them while the waves compute
  __device__ void load2(const float* Rp, int wave, int lane) {
    typedef Rec<D> R;
    const int w = wave % (D / 16);
    load_panel(aQ, Rp + R::QT + 16 * w, 1, D, lane);                            // Qt^T rows 16 w..
    load_panel(aW, Rp + R::WK + 16 * w, 1, D, lane);                            // Wk^T rows 16 w..
  }
  // waves 0-3: the loaded dO piece into the fragment image o[kk][lane][e] =
  // B(k = 16 kk + 4 g + e, j = i) = dO[16 kk + 4 g + e][j0 + i] (lane 16 g + i)
  template <typename T> __device__ void put(float (*o)[64][4], int wave, int lane) const {
    if (wave >= 4) return;
    const int tid = 64 * wave + lane, r = tid >> 2, c0 = 4 * (tid & 3);
    const f32x4 v = ChunkRows<T>::to_f32x4(bOw);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[r >> 4][16 * ((r & 15) >> 2) + c0 + j][r & 3] = v[j];
  }
};

template <typename T, int D>
__global__ void __launch_bounds__(512) kda_bwd_state(const float* __restrict__ rec, const T* __restrict__ dout,
                                                     const float* __restrict__ dht,
                                                     const int32_t* __restrict__ cu, const int64_t* __restrict__ seqs,
                                                     int n_rows, int T_per, int H, int64_t m_lo, int64_t m_hi,
                                                     Win win, float* __restrict__ dHs, float* __restrict__ dh0,
                                                     const float* __restrict__ carry_in, float* carry_out) {
  typedef Rec<D> R;
  constexpr int NCB = D / 16, NKC = C / 16, NKH = D / 32;
  // the bf16 path's products on hi/lo bf16 MFMA (about 2^-16 relative per
  // product, against fp32 MFMA on the fp32 path)
  constexpr bool HL = sizeof(T) == 2;
  __shared__ __align__(16) float G[D][16];
  __shared__ __align__(16) float dU[2][C][16];
  __shared__ __align__(16) float bOs[2][C / 16][64][4];  // dO fragment images, by step parity
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level branches stay scalar
  const int b = blockIdx.x;
  const int cb = (b / 8) % NCB, pair = 8 * (b / (8 * NCB)) + b % 8;
  const int n = pair / H, h = pair % H;
  if (n >= n_rows) return;
  const int j0 = cb * 16, ii = lane & 15, g = lane >> 4;
  int64_t base = 0, nc, tok_n, len_n;  // first area slot, chunks; first token, tokens
  if (cu) {
    base = seqs[n];
    tok_n = cu[n];
    len_n = (int64_t)cu[n + 1] - cu[n];
    nc = (len_n + C - 1) / C;
  } else {
    nc = (T_per + C - 1) / C;
    base = (int64_t)n * nc;
    tok_n = (int64_t)n * T_per;
    len_n = T_per;
  }
  const int64_t sd = ((int64_t)n * H + h) * D * D;
  auto rec_of = [&](int64_t m) { return rec + (area_slot(win, n, base, m) * H + h) * (int64_t)R::FLOATS; };
  auto dhs_of = [&](int64_t m) { return dHs + (area_slot(win, n, base, m) * H + h) * (int64_t)D * D; };
  // chunk m's rows of dO (m < nc)
  auto do_of = [&](int64_t m) {
    const int64_t rest = len_n - (int64_t)C * m;
    return ChunkRows<T>(dout, tok_n + (int64_t)C * m, rest < C ? (int)rest : C, H, h, D);
  };
  if (nc == 0) {  // no tokens: the gradient passes through unchanged
    if (dh0 && m_lo == 0)
      for (int x = tid; x < D * 16; x += blockDim.x) {
        const int c = x / 16, j = x % 16;
        dh0[sd + c * D + j0 + j] = dht ? dht[sd + c * D + j0 + j] : 0.f;
      }
    return;
  }
  // this launch walks chunks [m_lo, top) of the sequence (m_hi <= win.hi)
  const int64_t top = nc < m_hi ? nc : m_hi;
  if (top <= m_lo) return;
  // the end-state gradient of chunk top - 1: dht for the sequence's last
  // chunk, the carry of the later window at this window's top, else what the
  // launch over the later chunks of this window stored; the first two are
  // stored for the local gradients
  {
    const float* Rp = rec_of(top - 1);
    float* dHo = dhs_of(top - 1);
    const bool from_dht = top == nc, from_carry = !from_dht && top == win.hi;
    for (int x = tid; x < D * 16; x += blockDim.x) {
      const int c = x / 16, j = x % 16;
      float v;
      if (from_dht) v = dht ? dht[sd + c * D + j0 + j] : 0.f;
      else if (from_carry) v = carry_in[sd + c * D + j0 + j];
      else v = dHo[c * D + j0 + j];
      if (from_dht || from_carry) dHo[c * D + j0 + j] = v;
      G[c][j] = Rp[R::GAM + c] * v;
    }
  }
  // two operand sets used in turn: step m computes from one while the other
  // receives chunk m - 1
  StateOps<D> opsA, opsB;
  const int t = wave & 3, half = wave >> 2, koff = half * (D / 2);
  auto step = [&](StateOps<D>& cur, StateOps<D>& nxt, int64_t m) {
    // cur arrived during the previous step: wait for it here, leaving at most
    // that step's four dH stores in flight, so that no later wait for cur can
    // take the loads issued next with it
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4) expcnt(7) lgkmcnt(15)
    // this chunk's dO fragments to LDS (the buffer of this step's parity: the
    // other one may still be read by a wave finishing the previous step)
    float(*const bo)[64][4] = bOs[m & 1];
    cur.template put<T>(bo, wave, lane);
    const int64_t mn = m > m_lo ? m - 1 : m;  // (the last step loads a chunk it does not use)
    lds_barrier();  // G and the dO fragments ready
    nxt.load(rec_of(mn), do_of(mn), j0, wave, lane);
    // dU: this wave's halves of P^T dO and Kh G
    {
      f32x4 bG[NKH], bOh[StateOps<D>::NKP];
#pragma unroll
      for (int kk = 0; kk < NKH; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) bG[kk][e] = G[koff + 16 * kk + 4 * g + e][ii];
#pragma unroll
      for (int kk = 0; kk < StateOps<D>::NKP; ++kk) bOh[kk] = *(const f32x4*)bo[half * StateOps<D>::NKP + kk][lane];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mma_panels<HL>(acc, cur.aP, bOh);
      acc = mma_panels<HL>(acc, cur.aKh, bG);
#pragma unroll
      for (int e = 0; e < 4; ++e) dU[wave >> 2][16 * t + 4 * g + e][ii] = acc[e];
    }
    asm volatile("" ::"v"(nxt.keep[0]), "v"(nxt.keep[1]), "v"(nxt.keep[2]), "v"(nxt.keep[3]));
    nxt.load2(rec_of(mn), wave, lane);
    lds_barrier();  // both halves of dU
    if (D / 16 >= 8 || wave < D / 16) {
      f32x4 bU[NKC];
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * kk + 4 * g + e;
          bU[kk][e] = dU[0][r][ii] + dU[1][r][ii];
        }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f}, neg = {0.f, 0.f, 0.f, 0.f};
      f32x4 bO[NKC];
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) bO[kk] = *(const f32x4*)bo[kk][lane];
      acc = mma_panels<HL>(acc, cur.aQ, bO);
      neg = mma_panels<HL>(neg, cur.aW, bU);
      // chunk m - 1's end-state gradient: to the carry when that chunk is in
      // the earlier window
      // (a buffer store: its per-lane offset is the same on every step, so
      // no address register is overwritten while the stores are in flight)
      float* dHo = m > 0 ? (m == win.lo ? carry_out + sd : dhs_of(m - 1)) : nullptr;
      const __amdgpu_buffer_rsrc_t rh = rsrc(dHo, m > 0 ? (uint32_t)(D * D * sizeof(float)) : 0u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wave + 4 * g + e;
        const float v = G[r][ii] + acc[e] - neg[e];  // this lane's own element of G
        cur.keep[e] = v;
        if (m > 0) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cur.keep[e]), rh,
                                                (uint32_t)((r * D + j0 + ii) * sizeof(float)), 0, 0);
          G[r][ii] = nxt.gr[e] * v;
        } else if (dh0) {
          dh0[sd + r * D + j0 + ii] = v;
        }
      }
    }
  };
  opsA.load(rec_of(top - 1), do_of(top - 1), j0, wave, lane);
  opsA.load2(rec_of(top - 1), wave, lane);
  for (int64_t m = top - 1; m >= m_lo; m -= 2) {
    step(opsA, opsB, m);
    if (m == m_lo) break;
    step(opsB, opsA, m - 1);
  }
}

// ---------------------------------------------------------------------------
// Local gradients of one chunk, for the chunks m_lo <= m < m_hi of their
// sequences (the other workgroups of the grid exit at once).  Workgroup x
// takes area slot a0 + x.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads) kda_bwd_local(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ /* v: its copy in the record */,
    const T* __restrict__ /* dout: its copy in the record */, const void* __restrict__ g, const int32_t* __restrict__ cu,
    const int64_t* __restrict__ seqs, int n_rows, int T_per, int H, float g_floor, int gate, const float* __restrict__ rec,
    const float* __restrict__ h0, const float* __restrict__ ht, const float* __restrict__ states,
    const float* __restrict__ zero_state, const float* __restrict__ dHs, float* __restrict__ scr,
    T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv, T* __restrict__ dg, float* __restrict__ dbeta,
    int64_t m_lo, int64_t m_hi, Win win, int64_t a0) {
  typedef Rec<D> R;
  typedef Scr<D> W;
  // fp32 MFMA on both paths here: with hi/lo bf16 products this kernel ran
  // slower (measured when it also served D = 128: 550 against 491 us at
  // T = 4096, H = 16), since its time goes to the scratch round trips
  // between products, not to the matrix cores, and the splits cost
  // registers (a 48-byte spill) and VALU work
  constexpr bool HL = false;
  __shared__ ChunkPos pos;
  // the products' slices, and later the per-element dGamma of the chunk
  constexpr int kLds = kGemmLds > C * D ? kGemmLds : C * D;
  __shared__ __align__(16) float lds[kLds];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t slot = a0 + blockIdx.x;
  if (!chunk_pos_shared(slot, win, cu, seqs, n_rows, T_per, &pos)) return;
  if (pos.m < m_lo || pos.m >= m_hi) return;  // another launch's chunks
  const float* Rp = rec + (slot * H + h) * (int64_t)R::FLOATS;
  float* Wp = scr + (slot * H + h) * (int64_t)W::FLOATS;
  const float* dH = dHs + (slot * H + h) * (int64_t)D * D;
  const int64_t dd = (int64_t)D * D;
  const float* S = pos.m == 0 ? (h0 ? h0 + ((int64_t)pos.n * H + h) * dd : zero_state)
                              : states + ((pos.st0 + pos.m - 1) * H + h) * dd;
  const float* Sn = pos.m == pos.nc - 1 ? ht + ((int64_t)pos.n * H + h) * dd
                                        : states + ((pos.st0 + pos.m) * H + h) * dd;
  const float* gam = Rp + R::GAM;
  const float* bet = Rp + R::BET;

  // 1: U = Wv - Wk S;  dU = P^T dO + Kh diag(gamma) dH
  gemm<D, HL>(lds, Wp + W::U, D, -1.f, false, kFull, nullptr, rows(Rp + R::WK, D), krows(S, D), D, nullptr, nullptr, 0,
          Rp + R::WV);
  {
    const MatA a1 = trans(Rp + R::PM, C), a2 = rows(Rp + R::KH, D);
    const MatB b1 = krows(Rp + R::DO, D), b2 = krows(dH, D, gam);
    gemm<D, HL>(lds, Wp + W::DU, D, 1.f, false, kFull, nullptr, a1, b1, C, &a2, &b2, D);
  }
  // dgamma-last: sum_j dH_cj S_next_cj per channel; NP neighbouring lanes
  // share a channel and combine their partial sums by shuffles
  {
    constexpr int NP = kThreads / D;
    const int c = tid / NP, part = tid % NP;
    float acc = 0.f;
    for (int j = part; j < D; j += NP) acc += dH[c * D + j] * Sn[c * D + j];
#pragma unroll
    for (int m = 1; m < NP; m <<= 1) acc += __shfl_xor(acc, m);
    if (part == 0) Wp[W::DGL + c] = acc;
  }
  __syncthreads();
  // 2: dP = lower_incl(dO U^T); Dv = T^T dU; dKh = U dH^T diag(gamma)
  gemm<C, HL>(lds, Wp + W::DP, C, 1.f, false, kLowerIncl, nullptr, rows(Rp + R::DO, D), kcols(Wp + W::U, D), D, nullptr,
       nullptr, 0);
  gemm<D, HL>(lds, Wp + W::DV, D, 1.f, false, kFull, nullptr, trans(Rp + R::TM, C), krows(Wp + W::DU, D), C, nullptr,
       nullptr, 0);
  gemm<D, HL>(lds, Wp + W::DKH, D, 1.f, false, kFull, gam, rows(Wp + W::U, D), kcols(dH, D), D, nullptr, nullptr, 0);
  __syncthreads();
  // 3: Dk = T^T (-dU S^T) = -Dv S^T (into U); dQt = dO S^T + dP Kh;
  //    dKh += dP^T Qt
  gemm<D, HL>(lds, Wp + W::U, D, -1.f, false, kFull, nullptr, rows(Wp + W::DV, D), kcols(S, D), D, nullptr, nullptr, 0);
  {
    const MatA a1 = rows(Rp + R::DO, D), a2 = rows(Wp + W::DP, C);
    const MatB b1 = kcols(S, D), b2 = krows(Rp + R::KH, D);
    gemm<D, HL>(lds, Wp + W::DQT, D, 1.f, false, kFull, nullptr, a1, b1, D, &a2, &b2, C);
  }
  gemm<D, HL>(lds, Wp + W::DKH, D, 1.f, true, kFull, nullptr, trans(Wp + W::DP, C), krows(Rp + R::QT, D), C, nullptr,
       nullptr, 0);
  __syncthreads();
  // 4: dA = strict_lower(-Dk Wk^T - Dv Wv^T)
  {
    const MatA a1 = rows(Wp + W::U, D), a2 = rows(Wp + W::DV, D);
    const MatB b1 = kcols(Rp + R::WK, D), b2 = kcols(Rp + R::WV, D);
    gemm<C, HL>(lds, Wp + W::DA, C, -1.f, false, kStrictLower, nullptr, a1, b1, D, &a2, &b2, D);
  }
  __syncthreads();
  // 5: E = Dk + dA Kh (into dU); dKh += dA^T diag(beta) Kt
  gemm<D, HL>(lds, Wp + W::DU, D, 1.f, false, kFull, nullptr, rows(Wp + W::DA, C), krows(Rp + R::KH, D), C, nullptr,
       nullptr, 0, Wp + W::U);
  gemm<D, HL>(lds, Wp + W::DKH, D, 1.f, true, kFull, nullptr, trans(Wp + W::DA, C), krows(Rp + R::KT, D, bet), C,
       nullptr, nullptr, 0);
  __syncthreads();

  // 6: element-wise.
  const bool bf = sizeof(T) == 2;
  const int len = pos.len;
  // dbeta: 8 neighbouring lanes per row, combined by shuffles
  {
    const int r = tid / 8, part = tid % 8;
    float acc = 0.f;
    for (int c = part; c < D; c += 8)
      acc += Wp[W::U + r * D + c] * Rp[R::KT + r * D + c] + Wp[W::DV + r * D + c] * Rp[R::VV + r * D + c];
    for (int s2 = part; s2 < r; s2 += 8) acc += Wp[W::DA + r * C + s2] * Rp[R::AB + r * C + s2];
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) acc += __shfl_xor(acc, m);
    if (part == 0 && r < len) dbeta[(pos.tok0 + r) * H + h] = acc;
  }
  for (int x = tid; x < len * D; x += blockDim.x) {
    const int r = x / D, c = x % D;
    stx(dv + ((pos.tok0 + r) * H + h) * D + c, bet[r] * Wp[W::DV + x]);
  }
  // dq, dk and dGamma per element (Gamma from the record)
  float(*dG)[D] = (float(*)[D])lds;  // the products are done with it
  for (int x = tid; x < C * D; x += blockDim.x) {
    const int r = x / D, c = x % D;
    const float G = Rp[R::GM + x];
    const float e = __expf(G), ei = __expf(-G);
    const float dqt = Wp[W::DQT + x], dkt = bet[r] * Wp[W::DU + x], dkh = Wp[W::DKH + x];
    dG[r][c] = dqt * Rp[R::QT + x] + dkt * Rp[R::KT + x] - dkh * Rp[R::KH + x];
    if (r < len) {
      const int64_t o = ((pos.tok0 + r) * H + h) * D + c;
      stx(dq + o, dqt * e);
      stx(dk + o, dkt * e + dkh * ei);
    }
  }
  __syncthreads();
  // dg_r = sum_{s >= r} dGamma_s plus the chunk-end decay (it depends on
  // every row), masked by the floor.  Per channel, each group of RG rows sums
  // its rows, then walks them backward from the sums of the later groups.
  {
    typedef RowSplit<D> RS;
    __shared__ float gsum[RS::NG][D];
    const int c = tid % D, grp = tid / D, r0 = grp * RS::RG;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < RS::RG; ++i) part += dG[r0 + i][c];
    gsum[grp][c] = part;
    __syncthreads();
    float acc = Wp[W::DGL + c];
    for (int j = grp + 1; j < RS::NG; ++j) acc += gsum[j][c];
#pragma unroll
    for (int i = RS::RG - 1; i >= 0; --i) {
      const int r = r0 + i;
      acc += dG[r][c];
      float out = 0.f;
      if (r < len) {
        const float graw = gate_at(g, gate, bf, (pos.tok0 + r) * H + h, D, c);
        out = graw >= g_floor ? acc : 0.f;
      }
      dG[r][c] = out;  // this thread's own element
      if (gate == kGateChannel && r < len) stx(dg + ((pos.tok0 + r) * H + h) * D + c, out);
    }
  }
  if (gate == kGateHead) {
    __syncthreads();
    // per (token, head): the channel sum of the masked per-channel values (the
    // mask is the head's own, the same on every channel); 8 lanes per row
    const int r = tid / 8, part = tid % 8;
    float acc = 0.f;
    for (int c = part; c < D; c += 8) acc += dG[r][c];
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) acc += __shfl_xor(acc, m);
    if (part == 0 && r < len) stx(dg + (pos.tok0 + r) * H + h, acc);
  }
}

// ---------------------------------------------------------------------------
// Local gradients of one chunk at D = 128, fused: the same products and
// element-wise stage as kda_bwd_local, with every intermediate kept on chip
// instead of passing through the scratch area.  Wave w owns column tile w
// (16 columns): of the value side (U, dU, Dv) first, then of the key side
// (Dk, dQt, dKh, E), so its own products stay in registers.  Operands every
// wave reads whole go to LDS, each copied once: Wk, Kh, P, T and dO from the
// record, then U, Dv, dP, Dk and dA as the waves produce them.  The other
// operands are the wave's own columns, read straight from the record, the
// states and dH.  So each record element is read about once per chunk (the
// scratch version reads about 1.9 MB per (chunk, head) in all).
//   phase 1 (value column tile w): U = Wv - Wk S, dU = P^T dO + Kh G
//            (G = diag(gamma) dH), Dv = T^T dU, dv = diag(beta) Dv
//   phase 2: dP = lower_incl(dO U^T) (tiles shared among the waves), then
//            (key column tile w) Dk = -Dv S^T, dQt = dO S^T + dP Kh,
//            dKh = U dH^T diag(gamma) + dP^T Qt
//   phase 3: dA = strict_lower(-Dk Wk^T - Dv Wv^T) (tiles shared)
//   phase 4: E = Dk + dA Kh, dKh += dA^T diag(beta) Kt, then the
//            element-wise stage on the wave's key columns
// Only the lower-triangular blocks of P, T, dP and dA enter the products.
// Every product takes hi/lo bf16 MFMA, with Wk, Kh, dO, U, Dv and Dk kept in
// LDS as hi and lo planes, and the [64][64] matrices P, T, dP and dA (fp32 in
// LDS) and the register operands split as they are read: one MFMA shape
// throughout, so that no accumulation chain mixes shapes.
// An LDS operand as hi and lo planes of [64][LH] bf16, element (r, k) at
// r * LH + hl_pos(k) (a lane's fragment is 16 contiguous bytes of each
// plane); rows of 68 dwords, so 8 consecutive rows' 16-byte reads fall on
// distinct banks.
constexpr int LH = 128 + 8, PLANE = C * LH;
__device__ __forceinline__ HL8 hl_lds(const bf16_t* P, int r, int kb, int g) {
  const int o = r * LH + 32 * kb + 8 * g;
  return HL8{*(const bf16x8*)(P + o), *(const bf16x8*)(P + PLANE + o)};
}
__device__ __forceinline__ void hl_put(bf16_t* P, int r, int k, float x) {
  const uint32_t a = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x, 0.f));
  const int o = r * LH + hl_pos(k);
  P[o] = (bf16_t)a;
  P[PLANE + o] = (bf16_t)__builtin_bit_cast(uint32_t, f32x2_to_bf16x2(x - __uint_as_float(a << 16), 0.f));
}
__device__ __forceinline__ float hl_get(const bf16_t* P, int r, int k) {
  const int o = r * LH + hl_pos(k);
  return bf16_to_f32(P[o]) + bf16_to_f32(P[PLANE + o]);
}
// four consecutive k (k % 4 == 0, contiguous in each plane) of row r
__device__ __forceinline__ f32x4 hl_get4(const bf16_t* P, int r, int k) {
  const int o = r * LH + hl_pos(k);
  return bf4_to_f32(*(const uint2*)(P + o)) + bf4_to_f32(*(const uint2*)(P + PLANE + o));
}
// four consecutive k (k % 4 == 0) of row r
__device__ __forceinline__ void hl_put4(bf16_t* P, int r, int k, const f32x4& x) {
  uint2 hi, lo;
  split4(x, hi, lo);
  const int o = r * LH + hl_pos(k);
  *(uint2*)(P + o) = hi;
  *(uint2*)(P + PLANE + o) = lo;
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads) kda_bwd_local_fused(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const void* __restrict__ g, const int32_t* __restrict__ cu,
    const int64_t* __restrict__ seqs, int n_rows, int T_per, int H, float g_floor, int gate, const float* __restrict__ rec,
    const float* __restrict__ h0, const float* __restrict__ /* ht: S_next not read */,
    const float* __restrict__ states,
    const float* __restrict__ zero_state, const float* __restrict__ dHs, float* __restrict__ scr,
    T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv, T* __restrict__ dg, float* __restrict__ dbeta,
    int64_t m_lo, int64_t m_hi, Win win, int64_t a0) {
  static_assert(D == 16 * (kThreads / 64), "one 16-column tile per wave");
  typedef Rec<D> R;
  static_assert(D == 128, "hi/lo planes of 128 columns");
  static_assert(sizeof(T) == 2, "the bf16 path: dO's hi/lo planes hold it exactly");
  // H0, H1, H3, H4: hi/lo planes of [64][128] operands (2 PLANE bf16 each);
  // R2a (over H4's start), R2b: fp32 [64][64] with rows of 4 extra floats
  // (16-byte aligned, and the 16-byte reads of 8 consecutive rows fall on
  // distinct banks).  At the end R0, R3 and Q2 (over H4) hold fp32 [64][LX]
  // output rows.
  constexpr int LX = D + 4, LC = C + 4, AC = C * LC, AP = PLANE;  // AP: floats of a plane pair
  static_assert(AP >= C * LX && AP >= AC, "fp32 rows and [64][64] arrays fit a plane pair's region");
  __shared__ ChunkPos pos;
  __shared__ __align__(16) float lds[4 * AP + AC];
  bf16_t* const H0 = (bf16_t*)lds;             // Wk, then U, then Dk (hi/lo)
  bf16_t* const H1 = (bf16_t*)(lds + AP);      // Kh, then Dv (hi/lo)
  bf16_t* const H3 = (bf16_t*)(lds + 2 * AP);  // dO, then Wk (hi/lo)
  bf16_t* const H4 = (bf16_t*)(lds + 3 * AP);  // Wv in phase 3 (hi/lo)
  float* const R0 = lds;                       // fp32 output rows at the end
  float* const R3 = lds + 2 * AP;
  float* const R2a = lds + 3 * AP;             // P, then dP
  float* const R2b = lds + 4 * AP;             // T, then dA
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, gq = lane >> 4, i = lane & 15;
  const int h = blockIdx.y;
  const int64_t slot = a0 + blockIdx.x;
  if (!chunk_pos_shared(slot, win, cu, seqs, n_rows, T_per, &pos)) return;
  if (pos.m < m_lo || pos.m >= m_hi) return;  // another launch's chunks
  const float* Rp = rec + (slot * H + h) * (int64_t)R::FLOATS;
  const float* dH = dHs + (slot * H + h) * (int64_t)D * D;
  const int64_t dd = (int64_t)D * D;
  const float* S = pos.m == 0 ? (h0 ? h0 + ((int64_t)pos.n * H + h) * dd : zero_state)
                              : states + ((pos.st0 + pos.m - 1) * H + h) * dd;
  const float* gam = Rp + R::GAM;
  const float* bet = Rp + R::BET;
  const int len = pos.len;
  const int cw = 16 * w;  // this wave's column tile
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

  // phase 1's own columns of S and G = diag(gamma) dH (k down the key
  // channels), loaded first so that they are in flight during the staging
  f32x4 fs[D / 16], fg[D / 16];
  const float gc = gam[cw + i];  // gamma of this lane's key column (phase 2)
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    fs[kb] = frag_cols(S, D, cw + i, 16 * kb, gq);
    fg[kb] = frag_cols(dH, D, cw + i, 16 * kb, gq) * *(const f32x4*)(gam + 16 * kb + 4 * gq);
  }
  // this chunk's rows of v and dO as buffer resources (ChunkRows): rows past
  // the chunk's end read as zeros, with no branch; a masked load would wait
  // for every load before it
  const ChunkRows<T> vrows(v, pos.tok0, len, H, h, D), orows(dout, pos.tok0, len, H, h, D);
  {
    // every staging load before the first LDS store
    constexpr int NS = C * D / 4 / kThreads, NP = C * C / 4 / kThreads;
    f32x4 sw[NS], sk[NS], so[NS], sp[NP], st[NP];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int x = tid + j * kThreads, r = x / (D / 4), c4 = 4 * (x % (D / 4));
      sw[j] = *(const f32x4*)&Rp[R::WK + r * D + c4];
      sk[j] = *(const f32x4*)&Rp[R::KH + r * D + c4];
      so[j] = orows.ld4(r, c4);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int x = tid + j * kThreads, r = x / (C / 4), c4 = 4 * (x % (C / 4));
      sp[j] = *(const f32x4*)&Rp[R::PM + r * C + c4];
      st[j] = *(const f32x4*)&Rp[R::TM + r * C + c4];
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int x = tid + j * kThreads, r = x / (D / 4), c4 = 4 * (x % (D / 4));
      hl_put4(H0, r, c4, sw[j]);
      hl_put4(H1, r, c4, sk[j]);
      hl_put4(H3, r, c4, so[j]);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int x = tid + j * kThreads, r = x / (C / 4), c4 = 4 * (x % (C / 4));
      *(f32x4*)&R2a[r * LC + c4] = sp[j];
      *(f32x4*)&R2b[r * LC + c4] = st[j];
    }
  }
  __syncthreads();

  // ---- phase 1: value columns cw .. cw + 15
  // A 32-wide k-block kb of a product with a lower-triangular [64][64]
  // factor is nonzero for row tile rt when kb <= rt / 2 (the factor's rows
  // along k) or kb >= rt / 2 (its columns along k); the zero tiles a block
  // takes in are zeros in LDS.
  f32x4 U[4], dU[4] = {z4, z4, z4, z4}, Dv[4] = {z4, z4, z4, z4};
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)  // Wv's columns, U = Wv - Wk S once the products are done
#pragma unroll
    for (int e = 0; e < 4; ++e) U[rt][e] = Rp[R::WV + (16 * rt + 4 * gq + e) * D + cw + i];
  {
    f32x4 a[4] = {z4, z4, z4, z4};
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      const HL8 bs = hl_of(fs[2 * kb], fs[2 * kb + 1]), bg = hl_of(fg[2 * kb], fg[2 * kb + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        a[rt] = mma3(hl_lds(H0, 16 * rt + i, kb, gq), bs, a[rt]);    // Wk S
        dU[rt] = mma3(hl_lds(H1, 16 * rt + i, kb, gq), bg, dU[rt]);  // Kh G
      }
    }
    // dU += P^T dO: dO's column fragments from its planes (bf16 values are
    // hi + 0 there: exact)
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      f32x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] = hl_get(H3, 32 * kb + 4 * gq + e, cw + i);
        o1[e] = hl_get(H3, 32 * kb + 16 + 4 * gq + e, cw + i);
      }
      const HL8 bo = hl_of(o0, o1);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        if (kb >= rt / 2)
          dU[rt] = mma3(hl_of(frag_cols(R2a, LC, 16 * rt + i, 32 * kb, gq),
                              frag_cols(R2a, LC, 16 * rt + i, 32 * kb + 16, gq)), bo, dU[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) U[rt] -= a[rt];
  }
  // Dv = T^T dU
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb) {
    const HL8 bu = hl_of(dU[2 * kb], dU[2 * kb + 1]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      if (kb >= rt / 2)
        Dv[rt] = mma3(hl_of(frag_cols(R2b, LC, 16 * rt + i, 32 * kb, gq),
                            frag_cols(R2b, LC, 16 * rt + i, 32 * kb + 16, gq)), bu, Dv[rt]);
  }
  lds_barrier();  // every wave is done with Wk, Kh, P and T
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hl_put(H0, 16 * rt + 4 * gq + e, cw + i, U[rt][e]);
      hl_put(H1, 16 * rt + 4 * gq + e, cw + i, Dv[rt][e]);
    }
  lds_barrier();

  // ---- phase 2: dP = lower_incl(dO U^T), its 10 lower tiles over the waves
  // (the first k-block's rows of S and dH for the products after it go out
  // first, to arrive meanwhile)
  f32x4 s0 = frag_rows(S, D, cw + i, 0, gq), s1 = frag_rows(S, D, cw + i, 16, gq);
  f32x4 h0v = frag_rows(dH, D, cw + i, 0, gq), h1v = frag_rows(dH, D, cw + i, 16, gq);
  // this wave's columns of Kh and Qt, k running over tokens (for the products
  // with dP and dA, and the element-wise stage, whose rows are these)
  f32x4 fk[4], fq[4];
#pragma unroll
  for (int kb = 0; kb < C / 16; ++kb) {
    fk[kb] = frag_cols(Rp + R::KH, D, cw + i, 16 * kb, gq);
    fq[kb] = frag_cols(Rp + R::QT, D, cw + i, 16 * kb, gq);
  }
  for (int t = w; t < 10; t += kThreads / 64) {
    int ta, tb;
    low_tile(t, ta, tb);
    f32x4 acc = z4;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) acc = mma3(hl_lds(H3, 16 * ta + i, kb, gq), hl_lds(H0, 16 * tb + i, kb, gq), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      R2a[(16 * ta + 4 * gq + e) * LC + 16 * tb + i] = (ta > tb || 4 * gq + e >= i) ? acc[e] : 0.f;
  }
  // key columns cw .. cw + 15: Dk = -Dv S^T, dQt = dO S^T, dKh = U dH^T
  // diag(gamma) (the products with dP wait for its tiles).
  // dgamma-last of key channel c = cw + i is sum_j dH_cj S_next_cj, with
  // S_next = diag(gamma)(S + Kh^T U):
  //   gamma_c <dH_c, S_c> + sum_r Kh_rc (U dH^T diag(gamma))_rc,
  // the first sum over the j of this lane's row fragments here, the second
  // over its rows once Kh's columns are in (phase 4), without reading S_next.
  f32x4 Dk[4] = {z4, z4, z4, z4}, dQt[4] = {z4, z4, z4, z4}, dKh[4] = {z4, z4, z4, z4};
  float dgl = 0.f;
#pragma unroll 2
  for (int kb = 0; kb < D / 32; ++kb) {
    // S^T[value][key] = S[key][value] and dH[key][value] along rows
    dgl += h0v[0] * s0[0] + h0v[1] * s0[1] + h0v[2] * s0[2] + h0v[3] * s0[3] + h1v[0] * s1[0] + h1v[1] * s1[1] +
           h1v[2] * s1[2] + h1v[3] * s1[3];
    const HL8 bs = hl_of(s0, s1), bh = hl_of(h0v, h1v);
    if (kb + 1 < D / 32) {  // the next k-block's rows, in flight during this one's products
      s0 = frag_rows(S, D, cw + i, 32 * kb + 32, gq);
      s1 = frag_rows(S, D, cw + i, 32 * kb + 48, gq);
      h0v = frag_rows(dH, D, cw + i, 32 * kb + 32, gq);
      h1v = frag_rows(dH, D, cw + i, 32 * kb + 48, gq);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Dk[rt] = mma3(hl_lds(H1, 16 * rt + i, kb, gq), bs, Dk[rt]);
      dQt[rt] = mma3(hl_lds(H3, 16 * rt + i, kb, gq), bs, dQt[rt]);
      dKh[rt] = mma3(hl_lds(H0, 16 * rt + i, kb, gq), bh, dKh[rt]);
    }
  }
  {
    dgl *= gc;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Dk[rt] = -Dk[rt];
      dKh[rt] = dKh[rt] * gc;
    }
  }
  lds_barrier();  // dP complete; U no longer read
  // Wk and Wv as rows, for phase 3's planes (in flight during the products below)
  constexpr int NW = C * D / 4 / kThreads;
  f32x4 wkr[NW], wvr[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int x = tid + j * kThreads, r = x / (D / 4), c4 = 4 * (x % (D / 4));
    wkr[j] = *(const f32x4*)&Rp[R::WK + r * D + c4];
    wvr[j] = *(const f32x4*)&Rp[R::WV + r * D + c4];
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) hl_put(H0, 16 * rt + 4 * gq + e, cw + i, Dk[rt][e]);
  // dgamma-last's second sum, while dKh is still U dH^T diag(gamma)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
    dgl += fk[rt][0] * dKh[rt][0] + fk[rt][1] * dKh[rt][1] + fk[rt][2] * dKh[rt][2] + fk[rt][3] * dKh[rt][3];
  // dQt += dP Kh, dKh += dP^T Qt
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb) {
    const HL8 bk = hl_of(fk[2 * kb], fk[2 * kb + 1]), bq = hl_of(fq[2 * kb], fq[2 * kb + 1]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (kb <= rt / 2)
        dQt[rt] = mma3(hl_of(frag_rows(R2a, LC, 16 * rt + i, 32 * kb, gq),
                             frag_rows(R2a, LC, 16 * rt + i, 32 * kb + 16, gq)), bk, dQt[rt]);
      if (kb >= rt / 2)
        dKh[rt] = mma3(hl_of(frag_cols(R2a, LC, 16 * rt + i, 32 * kb, gq),
                             frag_cols(R2a, LC, 16 * rt + i, 32 * kb + 16, gq)), bq, dKh[rt]);
    }
  }
  lds_barrier();  // Dk complete; dO and dP no longer read

  // ---- phase 3: dA = strict_lower(-Dk Wk^T - Dv Wv^T), lower tiles over the waves
  float dbr;  // dbeta of row tid / 8 (in lanes tid % 8 == 0)
  f32x4 fkt[4];  // this wave's columns of Kt, for phase 4 and the element-wise stage
#pragma unroll
  for (int kb = 0; kb < C / 16; ++kb) fkt[kb] = frag_cols(Rp + R::KT, D, cw + i, 16 * kb, gq);
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int x = tid + j * kThreads, r = x / (D / 4), c4 = 4 * (x % (D / 4));
    hl_put4(H3, r, c4, wkr[j]);
    hl_put4(H4, r, c4, wvr[j]);
  }
  lds_barrier();  // Wk and Wv planes complete
  for (int t = w; t < 10; t += kThreads / 64) {
    int ta, tb;
    low_tile(t, ta, tb);
    f32x4 acc = z4;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      acc = mma3(hl_lds(H0, 16 * ta + i, kb, gq), hl_lds(H3, 16 * tb + i, kb, gq), acc);
      acc = mma3(hl_lds(H1, 16 * ta + i, kb, gq), hl_lds(H4, 16 * tb + i, kb, gq), acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      R2b[(16 * ta + 4 * gq + e) * LC + 16 * tb + i] = (ta > tb || 4 * gq + e > i) ? -acc[e] : 0.f;
  }
  lds_barrier();
  // dbeta_r = <Dk_r, Kt_r> + <Dv_r, V_r> + sum_{s < r} dA_rs Abar_rs (Dk in R0,
  // Dv in R1, dA in R2b), 8 neighbouring lanes per row.  Loads go out before
  // any of this kernel's stores from here on: loads and stores share one
  // in-order completion counter, so a load issued after stores also waits
  // for them.
  {
    const int r = tid / 8, part = tid % 8;
    f32x4 a4 = z4;  // columns 16 part .. 16 part + 15, four at a time
    f32x4 vv[4], kt[4];
    float ab[C / 8];  // Abar_rs, s = part + 8 j (the whole row: every load in bounds, issued at once)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c4 = 16 * part + 4 * j;
      vv[j] = vrows.ld4(r, c4);
      kt[j] = *(const f32x4*)&Rp[R::KT + r * D + c4];
    }
#pragma unroll
    for (int j = 0; j < C / 8; ++j) ab[j] = Rp[R::AB + r * C + part + 8 * j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c4 = 16 * part + 4 * j;
      a4 += hl_get4(H0, r, c4) * kt[j] + hl_get4(H1, r, c4) * vv[j];
    }
    float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    // (a select, not a branch: loads under a branch would wait one by one)
#pragma unroll
    for (int j = 0; j < C / 8; ++j) {
      const float x = R2b[r * LC + part + 8 * j] * ab[j];
      acc += part + 8 * j < r ? x : 0.f;
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) acc += __shfl_xor(acc, m);
    dbr = acc;
  }

  // ---- phase 4: E = Dk + dA Kh, dKh += dA^T diag(beta) Kt (key columns)
  f32x4 E[4], brow[4];  // brow: beta of rows 16 rt + 4 gq + e (phase 4 and the element-wise stage)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    E[rt] = Dk[rt];
    brow[rt] = *(const f32x4*)(bet + 16 * rt + 4 * gq);
  }
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb) {
    const HL8 bk = hl_of(fk[2 * kb], fk[2 * kb + 1]);
    const HL8 bt = hl_of(fkt[2 * kb] * brow[2 * kb], fkt[2 * kb + 1] * brow[2 * kb + 1]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (kb <= rt / 2)
        E[rt] = mma3(hl_of(frag_rows(R2b, LC, 16 * rt + i, 32 * kb, gq),
                           frag_rows(R2b, LC, 16 * rt + i, 32 * kb + 16, gq)), bk, E[rt]);
      if (kb >= rt / 2)
        dKh[rt] = mma3(hl_of(frag_cols(R2b, LC, 16 * rt + i, 32 * kb, gq),
                             frag_cols(R2b, LC, 16 * rt + i, 32 * kb + 16, gq)), bt, dKh[rt]);
    }
  }
  // ---- element-wise, key column c of this lane, rows 16 rt + 4 gq + e
  const int c = cw + i;
  // Qt, Kt and Kh at this lane's elements are fq, fkt and fk (row 16 rt +
  // 4 gq + e is element e of fragment rt).  The log-decays are loaded here,
  // before any store: which rows pass the floor (bit 4 rt + e), and Gamma,
  // summed in the order of the record pass (so the two agree to the bit):
  // within each group of 8 rows (lane groups gq = 2 p', 2 p' + 1 of a
  // tile) the rows in order, a running sum handed from the even lane group
  // to the odd one, then the groups' totals in order
  f32x4 gm[4];
  uint32_t keep = 0;
  {
    const GateRows<T> grows(g, gate, pos.tok0, len, H, h, D);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) gm[rt][e] = grows.ld(16 * rt + 4 * gq + e, c);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * gq + e;
        const float gv = gm[rt][e];
        if (r < len && gv >= g_floor) keep |= 1u << (4 * rt + e);
        gm[rt][e] = r < len ? fmaxf(gv, g_floor) : 0.f;
      }
  }
  {
    float run[4], prev[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 sum[4];
    // round 0 settles the even lane groups, round 1 the odd ones
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        run[rt] = prev[rt];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          run[rt] += gm[rt][e];
          sum[rt][e] = run[rt];
        }
      }
      if (s2 == 0)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const float up = __shfl_up(run[rt], 16);
          prev[rt] = (gq & 1) ? up : 0.f;
        }
    }
    // the groups' totals come from lane groups 1 and 3
    float off = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float t0 = __shfl(run[rt], 16 + i), t1 = __shfl(run[rt], 48 + i);
      const float off1 = off + t0;
      gm[rt] = (gq < 2 ? off : off1) + sum[rt];
      off = off1 + t1;
    }
  }
  dgl += __shfl_xor(dgl, 16);  // dgamma-last: the four lane groups' parts
  dgl += __shfl_xor(dgl, 32);
  // beta of the rows this thread writes out below (r = tid / 32 + 16 j)
  float bv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bv[j] = bet[tid / (D / 4) + 16 * j];
  // dq, dk and dg go out as whole rows: staged in R0 (Dk is no longer read),
  // Q2 over H4 (Wv's planes neither) and R3
  float* const Q2 = R2a;
  lds_barrier();  // every wave is past the dbeta pass and phase 4
  f32x4 dG[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + 4 * gq + e;
      const float G = gm[rt][e];
      const float ep = __expf(G), ei = __expf(-G);
      const float dqt = dQt[rt][e], dkt = brow[rt][e] * E[rt][e], dkh = dKh[rt][e];
      dG[rt][e] = dqt * fq[rt][e] + dkt * fkt[rt][e] - dkh * fk[rt][e];
      R0[r * LX + c] = dqt * ep;
      Q2[r * LX + c] = dkt * ep + dkh * ei;
    }
  // dg_r = sum_{s >= r} dGamma_s + dgamma-last, masked by the floor.  A lane
  // holds rows 4 gq .. 4 gq + 3 of each row tile: the sums of the later row
  // tiles, of the later lane groups in the same tile, then its own rows.
  // The masked values go to R3 (dO is no longer read): dg itself with the
  // per-channel gate, the terms of the channel sums below with the per-head one.
  {
    float tot[4], after[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float s = dG[rt][0] + dG[rt][1] + dG[rt][2] + dG[rt][3];
      const float v0 = __shfl(s, i), v1 = __shfl(s, 16 + i), v2 = __shfl(s, 32 + i), v3 = __shfl(s, 48 + i);
      tot[rt] = v0 + v1 + v2 + v3;
      after[rt] = (gq < 1 ? v1 : 0.f) + (gq < 2 ? v2 : 0.f) + (gq < 3 ? v3 : 0.f);
    }
    float later = dgl;
#pragma unroll
    for (int rt = 3; rt >= 0; --rt) {
      float run = later + after[rt];
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const int r = 16 * rt + 4 * gq + e;
        run += dG[rt][e];
        R3[r * LX + c] = (keep >> (4 * rt + e)) & 1u ? run : 0.f;
      }
      later += tot[rt];
    }
  }
  lds_barrier();  // the staged rows are complete
  // whole rows out, four channels a thread and step: dq, dk, dv = diag(beta)
  // Dv (R1) and the per-channel dg
  for (int j = 0; j < 4; ++j) {
    const int x = tid + kThreads * j, r = x / (D / 4), c4 = 4 * (x % (D / 4));
    if (r < len) {
      const int64_t o = ((pos.tok0 + r) * H + h) * D + c4;
      st4(dq + o, *(const f32x4*)&R0[r * LX + c4]);
      st4(dk + o, *(const f32x4*)&Q2[r * LX + c4]);
      const int po = r * LH + hl_pos(c4);  // Dv's four elements from its planes
      const uint2 vh = *(const uint2*)(H1 + po), vl = *(const uint2*)(H1 + PLANE + po);
      const f32x4 dvr = {__uint_as_float(vh.x << 16) + __uint_as_float(vl.x << 16),
                         __uint_as_float(vh.x & 0xffff0000u) + __uint_as_float(vl.x & 0xffff0000u),
                         __uint_as_float(vh.y << 16) + __uint_as_float(vl.y << 16),
                         __uint_as_float(vh.y & 0xffff0000u) + __uint_as_float(vl.y & 0xffff0000u)};
      st4(dv + o, bv[j] * dvr);
      if (gate == kGateChannel) st4(dg + o, *(const f32x4*)&R3[r * LX + c4]);
    }
  }
  {
    const int r = tid / 8, part = tid % 8;
    if (gate == kGateHead) {
      // per-head dg_r: the channel sum of R3's row
      float hg = 0.f;
      for (int c2 = part; c2 < D; c2 += 8) hg += R3[r * LX + c2];
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) hg += __shfl_xor(hg, m);
      if (part == 0 && r < len) stx(dg + (pos.tok0 + r) * H + h, hg);
    }
    if (part == 0 && r < len) dbeta[(pos.tok0 + r) * H + h] = dbr;
  }
}

template <typename T, int D>
int launch_bwd_typed(int n_rows, int T_per, int H, const BwdPlan& bp, float g_floor, int gate,
                     const ChunkInputs& in, const float* h0, const int32_t* cu, const void* dout, const float* dht,
                     void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0, void* ws,
                     hipStream_t stream, void* const* events, const AuxStream* aux) {
  unsigned char* w = (unsigned char*)ws;
  float* ht = (float*)(w + bp.ht_off);
  float* states = (float*)(w + bp.states_off);
  float* zero = (float*)(w + bp.zero_off);
  float* rec = (float*)(w + bp.rec_off);
  float* scr = (float*)(w + bp.scr_off);
  float* dHs = (float*)(w + bp.dh_off);
  int64_t* seqs = (int64_t*)(w + bp.seq_off);
  float* carry = bp.width > 0 ? (float*)(w + bp.carry_off) : nullptr;
  if (bp.rec_floats != (size_t)Rec<D>::FLOATS || bp.scr_floats != bwd_scr_floats(D)) return (int)hipErrorInvalidValue;
  hipError_t e;
  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord((hipEvent_t)events[i], stream) : hipSuccess;
  };
  if ((e = mark(0)) != hipSuccess) return (int)e;
  if (cu && n_rows > 0) {
    if ((e = launch_kernel(kda_bwd_seqs, dim3(1), dim3(256), stream, cu, n_rows, seqs)) != hipSuccess) return (int)e;
  }
  // forward replay: ht and the state after every full chunk.  Only the local
  // kernel reads what it writes, and it writes nothing the record and
  // state-gradient passes touch, so with a second stream it runs beside them.
  auto replay = [&](hipStream_t st) {
    return launch_chunk_forward(sizeof(T) == 2, D, n_rows, T_per, H, bp.fwd, g_floor, gate, in, h0, cu,
                                (void*)(w + bp.o_off), ht, states, 1, ws, st, nullptr);
  };
  constexpr int64_t kAll = INT64_MAX;
  const int64_t nw = bp.windows();
  auto window = [&](int64_t wi) {
    return bp.width > 0 ? Win{wi * bp.width, (wi + 1) * bp.width, bp.width} : Win{0, kAll, 0};
  };
  const dim3 gc((unsigned)bp.n_area, H);
  // at D = 128 the fused record pass (no copies of the inputs in the record)
  auto const record_kernel = [] {
    if constexpr (D == 128) return &kda_bwd_chunk_fused<T, D>;
    else return &kda_bwd_chunk<T, D>;
  }();
  auto record = [&](const Win& wn) {
    if (bp.n_area == 0) return hipSuccess;
    return launch_kernel(record_kernel, gc, dim3(kThreads), stream, (const T*)in.q, (const T*)in.k,
                         (const T*)in.v, in.g, in.beta, (const T*)dout, cu, (const int64_t*)seqs, n_rows, T_per, H,
                         g_floor, gate, rec, zero, wn);
  };
  // groups of 8 (sequence, head) pairs x D / 16 column blocks (see kda_bwd_state)
  const int64_t state_blocks = ((int64_t)n_rows * H + 7) / 8 * 8 * (D / 16);
  const size_t carry_floats = (size_t)n_rows * H * D * D;
  // window wi reads the carry that window wi + 1 wrote and writes the other one
  auto state = [&](const Win& wn, int64_t wi, int64_t lo, int64_t hi) {
    const float* cin = carry ? carry + (size_t)((wi + 1) & 1) * carry_floats : nullptr;
    float* cout = carry ? carry + (size_t)(wi & 1) * carry_floats : nullptr;
    return launch_kernel(kda_bwd_state<T, D>, dim3((unsigned)state_blocks), dim3(512), stream, (const float*)rec,
                         (const T*)dout, dht, cu, (const int64_t*)seqs, n_rows, T_per, H, lo, hi, wn, dHs, dh0, cin,
                         cout);
  };
  // the fused local kernel at D = 128 (one column tile per wave), the
  // scratch version otherwise
  auto const local_kernel = [] {
    if constexpr (D == 128) return &kda_bwd_local_fused<T, D>;
    else return &kda_bwd_local<T, D>;
  }();
  // A single fixed-length sequence has its chunks [lo, hi) at consecutive
  // area slots, so the grid covers just those; otherwise the whole area.
  auto local = [&](hipStream_t st, const Win& wn, int64_t lo, int64_t hi) {
    if (bp.n_area == 0) return hipSuccess;
    int64_t a0 = 0, count = bp.n_area;
    if (!cu && n_rows == 1) {
      const int64_t nc = (T_per + C - 1) / C, top = hi < nc ? hi : nc;
      if (top <= lo) return hipSuccess;
      a0 = lo - wn.lo;
      count = top - lo;
    }
    return launch_kernel(local_kernel, dim3((unsigned)count, H), dim3(kThreads), st, (const T*)in.q,
                         (const T*)in.k, (const T*)in.v, (const T*)dout, in.g, cu, (const int64_t*)seqs, n_rows, T_per, H, g_floor, gate,
                         (const float*)rec, h0, (const float*)ht, (const float*)states, (const float*)zero,
                         (const float*)dHs, scr, (T*)dq, (T*)dk, (T*)dv, (T*)dg, dbeta, lo, hi, wn, a0);
  };
  if (!aux) {
    const int rc = replay(stream);
    if (rc != 0) return rc;
    // windows from the last chunks to the first; with several windows the
    // stage events bracket the first window's passes
    for (int64_t wi = nw - 1; wi >= 0; --wi) {
      const Win wn = window(wi);
      const bool first = wi == nw - 1;
      if (first && (e = mark(1)) != hipSuccess) return (int)e;
      if ((e = record(wn)) != hipSuccess) return (int)e;
      if (first && (e = mark(2)) != hipSuccess) return (int)e;
      if ((e = state(wn, wi, wn.lo, wn.hi)) != hipSuccess) return (int)e;
      if (first && (e = mark(3)) != hipSuccess) return (int)e;
      if ((e = local(stream, wn, wn.lo, wn.hi)) != hipSuccess) return (int)e;
    }
    return (int)mark(4);
  }
  // Second stream.  The state-gradient pass runs one workgroup per (pair, 16
  // columns) and leaves most CUs idle at small batch; the second stream fills
  // them: first with the replay, forked after the first record pass (the
  // replay is off the critical path), then with local gradients.
  const hipStream_t side = (hipStream_t)aux->stream;
  const hipEvent_t fork = (hipEvent_t)aux->fork, join = (hipEvent_t)aux->join;
  if ((e = record(window(nw - 1))) != hipSuccess) return (int)e;
  if ((e = hipEventRecord(fork, stream)) != hipSuccess) return (int)e;
  if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return (int)e;
  const int rc = replay(side);
  if (rc != 0) return rc;
  if ((e = hipEventRecord(join, side)) != hipSuccess) return (int)e;  // replay done
  // Every window the same way: the walk in up to `most` launches over
  // ranges [b_i, b_{i+1}) of the window's chunks (of the average sequence
  // with one window), the last one open-ended; the local gradients of each
  // range but the first go to the side stream once its walk is done, those
  // of the first follow on the call's stream.  Windows share one area, so a
  // window ends with the call's stream waiting for the side stream's local
  // gradients before the next window's record pass overwrites it.
  const int64_t per_seq = cu ? (T_per + (int64_t)C * n_rows - 1) / ((int64_t)C * (n_rows > 0 ? n_rows : 1))
                             : (T_per + C - 1) / C;
  for (int64_t wi = nw - 1; wi >= 0; --wi) {
    const Win wn = window(wi);
    if (wi < nw - 1 && (e = record(wn)) != hipSuccess) return (int)e;
    const int64_t span = bp.width > 0 ? (wn.hi < bp.span ? wn.hi : bp.span) - wn.lo : per_seq;
    const int most = span <= kBwdShortSpan ? 2 : kBwdParts;
    const int parts = span < most ? (int)span : most;
    auto bound = [&](int i) { return i >= parts ? wn.hi : wn.lo + span * i / parts; };
    if (parts >= 2) {
      if ((e = state(wn, wi, bound(parts - 1), wn.hi)) != hipSuccess) return (int)e;
      for (int i = parts - 1; i >= 1; --i) {
        // the event is recorded again: a wait holds the state of the record it saw
        if ((e = hipEventRecord(fork, stream)) != hipSuccess) return (int)e;
        if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return (int)e;
        if ((e = local(side, wn, bound(i), bound(i + 1))) != hipSuccess) return (int)e;
        if ((e = state(wn, wi, bound(i - 1), bound(i))) != hipSuccess) return (int)e;
      }
    } else if ((e = state(wn, wi, wn.lo, wn.hi)) != hipSuccess) {
      return (int)e;
    }
    // join was last recorded after the replay (first window) or waited for
    // already (later windows)
    if ((e = hipStreamWaitEvent(stream, join, 0)) != hipSuccess) return (int)e;
    if ((e = local(stream, wn, wn.lo, parts >= 2 ? bound(1) : wn.hi)) != hipSuccess) return (int)e;
    if (parts >= 2) {
      if ((e = hipEventRecord(join, side)) != hipSuccess) return (int)e;  // the side's local gradients
      if ((e = hipStreamWaitEvent(stream, join, 0)) != hipSuccess) return (int)e;
    }
  }
  return (int)hipSuccess;
}

}  // namespace

static_assert(bwd_rec_floats(64) == (size_t)Rec<64>::FLOATS && bwd_rec_floats(128) == (size_t)Rec<128>::FLOATS,
              "record layout agrees with the host plan");
static_assert(bwd_scr_floats(64) == (size_t)Scr<64>::FLOATS && bwd_scr_floats(128) == 0,
              "scratch layout agrees with the host plan (none for the fused kernel at D = 128)");
static_assert(Rec<128>::FLOATS % 4 == 0 && Rec<64>::FLOATS % 4 == 0 && Scr<128>::FLOATS % 4 == 0 &&
                  Scr<64>::FLOATS % 4 == 0 && Rec<128>::GAM % 4 == 0 && Rec<128>::BET % 4 == 0 &&
                  Rec<64>::GAM % 4 == 0 && Rec<64>::BET % 4 == 0,
              "16-byte aligned operand rows");

int launch_chunk_backward(int is_bf16, int d, int n_rows, int T, int H, const BwdPlan& bp, float g_floor, int gate,
                          const ChunkInputs& in, const float* h0, const int32_t* cu, const void* dout,
                          const float* dht, void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0,
                          void* ws, void* stream, void* const* events, const AuxStream* aux) {
  hipStream_t s = (hipStream_t)stream;
  if (is_bf16 && d == 64)
    return launch_bwd_typed<bf16_t, 64>(n_rows, T, H, bp, g_floor, gate, in, h0, cu, dout, dht, dq, dk, dv, dg,
                                        dbeta, dh0, ws, s, events, aux);
  if (is_bf16 && d == 128)
    return launch_bwd_typed<bf16_t, 128>(n_rows, T, H, bp, g_floor, gate, in, h0, cu, dout, dht, dq, dk, dv, dg,
                                         dbeta, dh0, ws, s, events, aux);
  if (!is_bf16 && d == 64)
    return launch_bwd_typed<float, 64>(n_rows, T, H, bp, g_floor, gate, in, h0, cu, dout, dht, dq, dk, dv, dg,
                                       dbeta, dh0, ws, s, events, aux);
  return (int)hipErrorInvalidValue;
}

}  // namespace kda
