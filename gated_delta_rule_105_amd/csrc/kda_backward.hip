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
//   Dk   = T^T (-dU S^T),   Dv = T^T dU
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
//                   quantities above that do not involve the state), fp32.
//   kda_bwd_state : one workgroup per (sequence, head, 16 state columns):
//                   dS walked backward over the chunks (column j of dS only
//                   needs column j of dH and dO), writing every chunk's dH.
//   kda_bwd_local : one workgroup per (chunk, head): everything else.
// Every product runs on fp32 MFMA (v_mfma_f32_16x16x4f32); a wave owns one
// 16x16 output tile at a time and reads its operands straight from memory
// (records and scratch are L2-resident while a workgroup works on them).
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int C = kChunk;

__device__ __forceinline__ float ldx(const float* p) { return *p; }
__device__ __forceinline__ float ldx(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void stx(float* p, float x) { *p = x; }
__device__ __forceinline__ void stx(bf16_t* p, float x) { *p = f32_to_bf16(x); }

// Four consecutive-k values of one operand row: k stride `s` elements.
__device__ __forceinline__ f32x4 ld4(const float* p, int s) {
  if (s == 1) return *(const f32x4*)p;
  return (f32x4){p[0], p[s], p[2 * s], p[3 * s]};
}

// One 16x16 tile: acc += sum_k A(i, k) B(k, j) over k < K (K % 16 == 0),
// A(i, k) = A[i * ai + k * ak], B(k, j) = B[k * bk + j * bj]; A and B point
// at the tile's first row / column.  bs: per-k scale of B, or null.  The
// lane layout is the one of kda_device.h: lane 16 g + i supplies row i of A
// and column i of B at k = k0 + 4 g + e in issue e, and holds D[4 g + r][i].
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const float* A, int ai, int ak, const float* B, int bk,
                                          int bj, const float* bs, int K, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const float* pa = A + i * ai + 4 * g * ak;
  const float* pb = B + i * bj + 4 * g * bk;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const f32x4 a = ld4(pa + k0 * ak, ak);
    f32x4 b = ld4(pb + k0 * bk, bk);
    if (bs) {
      const f32x4 s = *(const f32x4*)(bs + k0 + 4 * g);
      b = (f32x4){b[0] * s[0], b[1] * s[1], b[2] * s[2], b[3] * s[3]};
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  }
  return acc;
}

// Operand views for one product: A is M x K, B is K x N.
struct MatA {
  const float* p;
  int ai, ak;
  __device__ const float* at(int i) const { return p + i * ai; }
};
struct MatB {
  const float* p;
  int bk, bj;
  const float* bs;
  __device__ const float* at(int j) const { return p + j * bj; }
};
__device__ __forceinline__ MatA rows(const float* p, int ld) { return MatA{p, ld, 1}; }      // X, X[i][k]
__device__ __forceinline__ MatA trans(const float* p, int ld) { return MatA{p, 1, ld}; }     // X^T, X[k][i]
__device__ __forceinline__ MatB krows(const float* p, int ld, const float* s = nullptr) {    // X, X[k][j]
  return MatB{p, ld, 1, s};
}
__device__ __forceinline__ MatB kcols(const float* p, int ld) { return MatB{p, 1, ld, nullptr}; }  // X^T, X[j][k]

// Mask of a stored tile element (row r, column c).
enum Mask { kFull = 0, kLowerIncl = 1, kStrictLower = 2 };

// out[r][c] = alpha * (A1 B1 + A2 B2)[r][c] (+ out[r][c] when acc_in), then
// column scale cs[c] if given, masked; M x N, tiles split over the waves.
// A2 may be null (one product).  out rows have stride ldo.
__device__ void gemm(float* out, int ldo, int M, int N, float alpha, bool acc_in, Mask mask, const float* cs,
                     const MatA& A1, const MatB& B1, int K1, const MatA* A2, const MatB* B2, int K2, int wave,
                     int nwaves, int lane) {
  const int tn = N / 16, tiles = (M / 16) * tn;
  const int i = lane & 15, g = lane >> 4;
  for (int t = wave; t < tiles; t += nwaves) {
    const int r0 = (t / tn) * 16, c0 = (t % tn) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile_mma(acc, A1.at(r0), A1.ai, A1.ak, B1.at(c0), B1.bk, B1.bj, B1.bs, K1, lane);
    if (A2) acc = tile_mma(acc, A2->at(r0), A2->ai, A2->ak, B2->at(c0), B2->bk, B2->bj, B2->bs, K2, lane);
    const int c = c0 + i;
    const float sc = cs ? cs[c] : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + 4 * g + e;
      float* dst = out + r * ldo + c;
      float x = alpha * acc[e];
      if (acc_in) x += *dst;
      x *= sc;
      const bool keep = mask == kFull || (mask == kLowerIncl ? r >= c : r > c);
      *dst = keep ? x : 0.f;
    }
  }
}

// Floats of one (chunk, head) record at key/value width D: Qt, Kt, Kh, V,
// dO, Wk, Wv ([C][D] each, rows past the chunk's end zero), P, T, Abar
// ([C][C]), gamma [D], beta [C] (0 past the end).
template <int D> struct Rec {
  static constexpr int QT = 0, KT = C * D, KH = 2 * C * D, VV = 3 * C * D, DO = 4 * C * D, WK = 5 * C * D,
                       WV = 6 * C * D, PM = 7 * C * D, TM = PM + C * C, AB = TM + C * C, GAM = AB + C * C,
                       BET = GAM + D, FLOATS = BET + C;
};
// Floats of one (chunk, head) scratch area of kda_bwd_local: U (then Dk),
// dU (then E = Dk + dA Kh), dWk (then dGamma), Dv, dQt, dKh ([C][D] each),
// dP, dA ([C][C]), dgamma-last [D].
template <int D> struct Scr {
  static constexpr int U = 0, DU = C * D, DWK = 2 * C * D, DV = 3 * C * D, DQT = 4 * C * D, DKH = 5 * C * D,
                       DP = 6 * C * D, DA = DP + C * C, DGL = DA + C * C, FLOATS = DGL + D;
};

// Chunk `slot` of the call (slots count the chunks of all sequences in
// order) as sequence n, chunk m of nc, tokens [tok0, tok0 + len), and the
// first prefix-state slot of its sequence (full chunks of the earlier
// sequences).  Returns false past the last chunk.
struct ChunkPos {
  int n, m, nc, len;
  int64_t tok0, st0;
};
__device__ bool chunk_pos(int64_t slot, const int32_t* cu, int n_rows, int T_per, ChunkPos* p) {
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
  int64_t base = 0, st0 = 0;
  for (int n = 0; n < n_rows; ++n) {
    const int64_t L = (int64_t)cu[n + 1] - cu[n];
    const int64_t nc = (L + C - 1) / C;
    if (slot < base + nc) {
      p->n = n;
      p->m = (int)(slot - base);
      p->nc = (int)nc;
      p->tok0 = (int64_t)cu[n] + (int64_t)p->m * C;
      p->len = (int)min((int64_t)C, L - (int64_t)p->m * C);
      p->st0 = st0;
      return true;
    }
    base += nc;
    st0 += L / C;
  }
  return false;
}

// Same position, found once per workgroup by thread 0 and shared via LDS.
__device__ bool chunk_pos_shared(int64_t slot, const int32_t* cu, int n_rows, int T_per, ChunkPos* sh) {
  __shared__ int ok;
  if (threadIdx.x == 0) ok = chunk_pos(slot, cu, n_rows, T_per, sh) ? 1 : 0;
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
__global__ void __launch_bounds__(512) kda_bwd_chunk(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const void* __restrict__ g,
                                                     const float* __restrict__ beta, const T* __restrict__ dout,
                                                     const int32_t* __restrict__ cu, int n_rows, int T_per, int H,
                                                     float g_floor, int gate, float* __restrict__ rec,
                                                     float* __restrict__ zero_state) {
  typedef Rec<D> R;
  __shared__ ChunkPos pos;
  __shared__ float As[C][C + 1];  // diag(beta) Abar
  __shared__ float Ts[C][C + 1];  // T
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int h = blockIdx.y;
  const int64_t slot = blockIdx.x;
  if (slot == 0 && h == 0)
    for (int x = tid; x < D * D; x += blockDim.x) zero_state[x] = 0.f;
  if (!chunk_pos_shared(slot, cu, n_rows, T_per, &pos)) return;
  float* Rp = rec + (slot * H + h) * (int64_t)R::FLOATS;
  const bool bf = sizeof(T) == 2;
  const int len = pos.len;

  // element-wise: one thread per key channel walks the rows (prefix sum)
  if (tid < D) {
    const int c = tid;
    float G = 0.f;
    for (int r = 0; r < C; ++r) {
      float qv = 0.f, kv = 0.f;
      if (r < len) {
        const int64_t th = (pos.tok0 + r) * H + h;
        G += fmaxf(gate_at(g, gate, bf, th, D, c), g_floor);
        qv = ldx(q + th * D + c);
        kv = ldx(k + th * D + c);
      }
      const float e = __expf(G), ei = __expf(-G);
      Rp[R::QT + r * D + c] = qv * e;
      Rp[R::KT + r * D + c] = kv * e;
      Rp[R::KH + r * D + c] = kv * ei;
    }
    Rp[R::GAM + c] = __expf(G);
  } else if (tid < 2 * D) {
    const int c = tid - D;
    for (int r = 0; r < C; ++r) {
      const int64_t th = (pos.tok0 + r) * H + h;
      Rp[R::VV + r * D + c] = r < len ? ldx(v + th * D + c) : 0.f;
      Rp[R::DO + r * D + c] = r < len ? ldx(dout + th * D + c) : 0.f;
    }
  } else if (tid < 2 * D + C) {
    const int r = tid - 2 * D;
    Rp[R::BET + r] = r < len ? beta[(pos.tok0 + r) * H + h] : 0.f;
  }
  __syncthreads();

  // Abar = strict_lower(Kt Kh^T), P = lower_incl(Qt Kh^T)
  gemm(Rp + R::AB, C, C, C, 1.f, false, kStrictLower, nullptr, rows(Rp + R::KT, D), kcols(Rp + R::KH, D), D,
       nullptr, nullptr, 0, wave, nw, lane);
  gemm(Rp + R::PM, C, C, C, 1.f, false, kLowerIncl, nullptr, rows(Rp + R::QT, D), kcols(Rp + R::KH, D), D,
       nullptr, nullptr, 0, wave, nw, lane);
  __syncthreads();
  for (int x = tid; x < C * C; x += blockDim.x) {
    const int r = x / C, s = x % C;
    As[r][s] = Rp[R::BET + r] * Rp[R::AB + x];
  }
  __syncthreads();
  // T = (I + A)^{-1}, A strictly lower: column s by forward substitution,
  // T[r][s] = -sum_{s <= m < r} A[r][m] T[m][s] for r > s, T[s][s] = 1
  if (tid < C) {
    const int s = tid;
    for (int r = 0; r < s; ++r) Ts[r][s] = 0.f;
    Ts[s][s] = 1.f;
    for (int r = s + 1; r < C; ++r) {
      float acc = 0.f;
      for (int m = s; m < r; ++m) acc += As[r][m] * Ts[m][s];
      Ts[r][s] = -acc;
    }
  }
  __syncthreads();
  for (int x = tid; x < C * C; x += blockDim.x) Rp[R::TM + x] = Ts[x / C][x % C];
  __syncthreads();
  // Wk = T diag(beta) Kt, Wv = T diag(beta) V
  gemm(Rp + R::WK, D, C, D, 1.f, false, kFull, nullptr, rows(Rp + R::TM, C), krows(Rp + R::KT, D, Rp + R::BET), C,
       nullptr, nullptr, 0, wave, nw, lane);
  gemm(Rp + R::WV, D, C, D, 1.f, false, kFull, nullptr, rows(Rp + R::TM, C), krows(Rp + R::VV, D, Rp + R::BET), C,
       nullptr, nullptr, 0, wave, nw, lane);
}

// ---------------------------------------------------------------------------
// Reverse pass over the chunks of one sequence for 16 columns of dS.
template <int D>
__global__ void __launch_bounds__(256) kda_bwd_state(const float* __restrict__ rec, const float* __restrict__ dht,
                                                     const int32_t* __restrict__ cu, int n_rows, int T_per, int H,
                                                     float* __restrict__ dHs, float* __restrict__ dh0) {
  typedef Rec<D> R;
  constexpr int NCB = D / 16;
  __shared__ __align__(16) float dH[D][16];
  __shared__ __align__(16) float dU[C][16];
  __shared__ __align__(16) float gam[D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int pair = blockIdx.x / NCB, cb = blockIdx.x % NCB;
  const int n = pair / H, h = pair % H;
  if (n >= n_rows) return;
  const int j0 = cb * 16;
  // this sequence's chunks and the slot of its first one
  int64_t base = 0, nc;
  if (cu) {
    for (int m = 0; m < n; ++m) base += ((int64_t)cu[m + 1] - cu[m] + C - 1) / C;
    nc = ((int64_t)cu[n + 1] - cu[n] + C - 1) / C;
  } else {
    nc = (T_per + C - 1) / C;
    base = (int64_t)n * nc;
  }
  const int64_t sd = ((int64_t)n * H + h) * D * D;
  for (int x = tid; x < D * 16; x += blockDim.x) {
    const int c = x / 16, j = x % 16;
    dH[c][j] = dht ? dht[sd + c * D + j0 + j] : 0.f;
  }
  for (int64_t m = nc - 1; m >= 0; --m) {
    const int64_t slot = base + m;
    const float* Rp = rec + (slot * H + h) * (int64_t)R::FLOATS;
    float* dHo = dHs + (slot * H + h) * (int64_t)D * D;
    for (int x = tid; x < D; x += blockDim.x) gam[x] = Rp[R::GAM + x];
    __syncthreads();  // dH and gamma ready
    for (int x = tid; x < D * 16; x += blockDim.x) {
      const int c = x / 16, j = x % 16;
      dHo[c * D + j0 + j] = dH[c][j];
    }
    // dU = P^T dO + Kh diag(gamma) dH                          [C x 16]
    {
      const MatA a1 = trans(Rp + R::PM, C), a2 = rows(Rp + R::KH, D);
      const MatB b1 = krows(Rp + R::DO + j0, D), b2 = krows(&dH[0][0], 16, gam);
      gemm(&dU[0][0], 16, C, 16, 1.f, false, kFull, nullptr, a1, b1, C, &a2, &b2, D, wave, nw, lane);
    }
    __syncthreads();  // dU ready; every wave is done reading dH
    // dH <- diag(gamma) dH + Qt^T dO - Wk^T dU                  [D x 16]
    {
      const int tiles = D / 16;
      const int i = lane & 15, g = lane >> 4;
      for (int t = wave; t < tiles; t += nw) {
        const int r0 = t * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = tile_mma(acc, Rp + R::QT + r0, 1, D, Rp + R::DO + j0, D, 1, nullptr, C, lane);
        f32x4 neg = {0.f, 0.f, 0.f, 0.f};
        neg = tile_mma(neg, Rp + R::WK + r0, 1, D, &dU[0][0], 16, 1, nullptr, C, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = r0 + 4 * g + e;
          dH[r][i] = gam[r] * dH[r][i] + acc[e] - neg[e];  // this lane's own element only
        }
      }
    }
    __syncthreads();
  }
  if (dh0)
    for (int x = tid; x < D * 16; x += blockDim.x) {
      const int c = x / 16, j = x % 16;
      dh0[sd + c * D + j0 + j] = dH[c][j];
    }
}

// ---------------------------------------------------------------------------
// Local gradients of one chunk.
template <typename T, int D>
__global__ void __launch_bounds__(512) kda_bwd_local(
    const T* __restrict__ q, const T* __restrict__ k, const void* __restrict__ g, const int32_t* __restrict__ cu,
    int n_rows, int T_per, int H, float g_floor, int gate, const float* __restrict__ rec,
    const float* __restrict__ h0, const float* __restrict__ ht, const float* __restrict__ states,
    const float* __restrict__ zero_state, const float* __restrict__ dHs, float* __restrict__ scr,
    T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv, T* __restrict__ dg, float* __restrict__ dbeta) {
  typedef Rec<D> R;
  typedef Scr<D> W;
  __shared__ ChunkPos pos;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int h = blockIdx.y;
  const int64_t slot = blockIdx.x;
  if (!chunk_pos_shared(slot, cu, n_rows, T_per, &pos)) return;
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
  gemm(Wp + W::U, D, C, D, -1.f, false, kFull, nullptr, rows(Rp + R::WK, D), krows(S, D), D, nullptr, nullptr, 0,
       wave, nw, lane);
  {
    const MatA a1 = trans(Rp + R::PM, C), a2 = rows(Rp + R::KH, D);
    const MatB b1 = krows(Rp + R::DO, D), b2 = krows(dH, D, gam);
    gemm(Wp + W::DU, D, C, D, 1.f, false, kFull, nullptr, a1, b1, C, &a2, &b2, D, wave, nw, lane);
  }
  // dgamma-last: sum_j dH_cj S_next_cj per channel
  for (int c = tid; c < D; c += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < D; ++j) acc += dH[c * D + j] * Sn[c * D + j];
    Wp[W::DGL + c] = acc;
  }
  __syncthreads();
  for (int x = tid; x < C * D; x += blockDim.x) Wp[W::U + x] += Rp[R::WV + x];
  __syncthreads();
  // 2: dP = lower_incl(dO U^T); dWk = -dU S^T; Dv = T^T dU; dQt = dO S^T;
  //    dKh = U dH^T diag(gamma)
  gemm(Wp + W::DP, C, C, C, 1.f, false, kLowerIncl, nullptr, rows(Rp + R::DO, D), kcols(Wp + W::U, D), D, nullptr,
       nullptr, 0, wave, nw, lane);
  gemm(Wp + W::DWK, D, C, D, -1.f, false, kFull, nullptr, rows(Wp + W::DU, D), kcols(S, D), D, nullptr, nullptr, 0,
       wave, nw, lane);
  gemm(Wp + W::DV, D, C, D, 1.f, false, kFull, nullptr, trans(Rp + R::TM, C), krows(Wp + W::DU, D), C, nullptr,
       nullptr, 0, wave, nw, lane);
  gemm(Wp + W::DQT, D, C, D, 1.f, false, kFull, nullptr, rows(Rp + R::DO, D), kcols(S, D), D, nullptr, nullptr, 0,
       wave, nw, lane);
  gemm(Wp + W::DKH, D, C, D, 1.f, false, kFull, gam, rows(Wp + W::U, D), kcols(dH, D), D, nullptr, nullptr, 0,
       wave, nw, lane);
  __syncthreads();
  // 3: Dk = T^T dWk (into U); dQt += dP Kh; dKh += dP^T Qt
  gemm(Wp + W::U, D, C, D, 1.f, false, kFull, nullptr, trans(Rp + R::TM, C), krows(Wp + W::DWK, D), C, nullptr,
       nullptr, 0, wave, nw, lane);
  gemm(Wp + W::DQT, D, C, D, 1.f, true, kFull, nullptr, rows(Wp + W::DP, C), krows(Rp + R::KH, D), C, nullptr,
       nullptr, 0, wave, nw, lane);
  gemm(Wp + W::DKH, D, C, D, 1.f, true, kFull, nullptr, trans(Wp + W::DP, C), krows(Rp + R::QT, D), C, nullptr,
       nullptr, 0, wave, nw, lane);
  __syncthreads();
  // 4: dA = strict_lower(-Dk Wk^T - Dv Wv^T)
  {
    const MatA a1 = rows(Wp + W::U, D), a2 = rows(Wp + W::DV, D);
    const MatB b1 = kcols(Rp + R::WK, D), b2 = kcols(Rp + R::WV, D);
    gemm(Wp + W::DA, C, C, C, -1.f, false, kStrictLower, nullptr, a1, b1, D, &a2, &b2, D, wave, nw, lane);
  }
  __syncthreads();
  // 5: E = Dk + dA Kh (into dU); dKh += dA^T diag(beta) Kt
  gemm(Wp + W::DU, D, C, D, 1.f, false, kFull, nullptr, rows(Wp + W::DA, C), krows(Rp + R::KH, D), C, nullptr,
       nullptr, 0, wave, nw, lane);
  gemm(Wp + W::DKH, D, C, D, 1.f, true, kFull, nullptr, trans(Wp + W::DA, C), krows(Rp + R::KT, D, bet), C,
       nullptr, nullptr, 0, wave, nw, lane);
  __syncthreads();
  for (int x = tid; x < C * D; x += blockDim.x) Wp[W::DU + x] += Wp[W::U + x];
  __syncthreads();

  // 6: element-wise.  dbeta per row; dv; then per channel the prefix sums
  // of the gate again (same order as the record), dq, dk, dGamma.
  const bool bf = sizeof(T) == 2;
  const int len = pos.len;
  if (tid < C) {
    const int r = tid;
    float acc = 0.f;
    for (int c = 0; c < D; ++c)
      acc += Wp[W::U + r * D + c] * Rp[R::KT + r * D + c] + Wp[W::DV + r * D + c] * Rp[R::VV + r * D + c];
    for (int s = 0; s < r; ++s) acc += Wp[W::DA + r * C + s] * Rp[R::AB + r * C + s];
    if (r < len) dbeta[(pos.tok0 + r) * H + h] = acc;
  }
  for (int x = tid; x < len * D; x += blockDim.x) {
    const int r = x / D, c = x % D;
    stx(dv + ((pos.tok0 + r) * H + h) * D + c, bet[r] * Wp[W::DV + x]);
  }
  float* dG = Wp + W::DWK;  // dGamma, then the masked dg per channel
  if (tid < D) {
    const int c = tid;
    float G = 0.f;
    for (int r = 0; r < C; ++r) {
      if (r < len) G += fmaxf(gate_at(g, gate, bf, (pos.tok0 + r) * H + h, D, c), g_floor);
      const float e = __expf(G), ei = __expf(-G);
      const int x = r * D + c;
      const float dqt = Wp[W::DQT + x], dkt = bet[r] * Wp[W::DU + x], dkh = Wp[W::DKH + x];
      dG[x] = dqt * Rp[R::QT + x] + dkt * Rp[R::KT + x] - dkh * Rp[R::KH + x];
      if (r < len) {
        const int64_t o = ((pos.tok0 + r) * H + h) * D + c;
        stx(dq + o, dqt * e);
        stx(dk + o, dkt * e + dkh * ei);
      }
    }
    // reverse prefix sum; the chunk-end decay belongs to the last row
    float acc = Wp[W::DGL + c];
    for (int r = C - 1; r >= 0; --r) {
      acc += dG[r * D + c];
      float out = 0.f;
      if (r < len) {
        const float graw = gate_at(g, gate, bf, (pos.tok0 + r) * H + h, D, c);
        out = graw >= g_floor ? acc : 0.f;
      }
      dG[r * D + c] = out;
      if (gate == kGateChannel && r < len) stx(dg + ((pos.tok0 + r) * H + h) * D + c, out);
    }
  }
  if (gate == kGateHead) {
    __syncthreads();
    if (tid < len) {
      const int r = tid;
      const float graw = gate_at(g, gate, bf, (pos.tok0 + r) * H + h, D, 0);
      float acc = 0.f;
      // per-channel sums before the mask: the mask is the head's own
      for (int c = 0; c < D; ++c) acc += dG[r * D + c];
      stx(dg + (pos.tok0 + r) * H + h, graw >= g_floor ? acc : 0.f);
    }
  }
}

template <typename T, int D>
int launch_bwd_typed(int n_rows, int T_per, int H, const BwdPlan& bp, float g_floor, int gate,
                     const ChunkInputs& in, const float* h0, const int32_t* cu, const void* dout, const float* dht,
                     void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0, void* ws,
                     hipStream_t stream, void* const* events) {
  unsigned char* w = (unsigned char*)ws;
  float* ht = (float*)(w + bp.ht_off);
  float* states = (float*)(w + bp.states_off);
  float* zero = (float*)(w + bp.zero_off);
  float* rec = (float*)(w + bp.rec_off);
  float* scr = (float*)(w + bp.scr_off);
  float* dHs = (float*)(w + bp.dh_off);
  if (bp.rec_floats != (size_t)Rec<D>::FLOATS || bp.scr_floats != (size_t)Scr<D>::FLOATS)
    return (int)hipErrorInvalidValue;
  hipError_t e;
  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord((hipEvent_t)events[i], stream) : hipSuccess;
  };
  if ((e = mark(0)) != hipSuccess) return (int)e;
  // forward replay: ht and the state after every full chunk
  int rc = launch_chunk_forward(sizeof(T) == 2, D, n_rows, T_per, H, bp.fwd, g_floor, gate, in, h0, cu,
                                (void*)(w + bp.o_off), ht, states, 1, ws, stream, nullptr);
  if (rc != 0) return rc;
  if ((e = mark(1)) != hipSuccess) return (int)e;
  const dim3 gc((unsigned)bp.n_slots, H);
  if (bp.n_slots > 0) {
    hipLaunchKernelGGL((kda_bwd_chunk<T, D>), gc, dim3(512), 0, stream, (const T*)in.q, (const T*)in.k,
                       (const T*)in.v, in.g, in.beta, (const T*)dout, cu, n_rows, T_per, H, g_floor, gate, rec, zero);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  if ((e = mark(2)) != hipSuccess) return (int)e;
  hipLaunchKernelGGL((kda_bwd_state<D>), dim3((unsigned)(n_rows * H * (D / 16))), dim3(256), 0, stream,
                     (const float*)rec, dht, cu, n_rows, T_per, H, dHs, dh0);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if ((e = mark(3)) != hipSuccess) return (int)e;
  if (bp.n_slots > 0) {
    hipLaunchKernelGGL((kda_bwd_local<T, D>), gc, dim3(512), 0, stream, (const T*)in.q, (const T*)in.k, in.g, cu,
                       n_rows, T_per, H, g_floor, gate, (const float*)rec, h0, (const float*)ht,
                       (const float*)states, (const float*)zero, (const float*)dHs, scr, (T*)dq, (T*)dk, (T*)dv,
                       (T*)dg, dbeta);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  return (int)mark(4);
}

}  // namespace

static_assert(bwd_rec_floats(64) == (size_t)Rec<64>::FLOATS && bwd_rec_floats(128) == (size_t)Rec<128>::FLOATS,
              "record layout agrees with the host plan");
static_assert(bwd_scr_floats(64) == (size_t)Scr<64>::FLOATS && bwd_scr_floats(128) == (size_t)Scr<128>::FLOATS,
              "scratch layout agrees with the host plan");
static_assert(Rec<128>::FLOATS % 4 == 0 && Rec<64>::FLOATS % 4 == 0 && Scr<128>::FLOATS % 4 == 0 &&
                  Scr<64>::FLOATS % 4 == 0 && Rec<128>::GAM % 4 == 0 && Rec<128>::BET % 4 == 0 &&
                  Rec<64>::GAM % 4 == 0 && Rec<64>::BET % 4 == 0,
              "16-byte aligned operand rows");

int launch_chunk_backward(int is_bf16, int d, int n_rows, int T, int H, const BwdPlan& bp, float g_floor, int gate,
                          const ChunkInputs& in, const float* h0, const int32_t* cu, const void* dout,
                          const float* dht, void* dq, void* dk, void* dv, void* dg, float* dbeta, float* dh0,
                          void* ws, void* stream, void* const* events) {
  hipStream_t s = (hipStream_t)stream;
  if (is_bf16 && d == 64)
    return launch_bwd_typed<bf16_t, 64>(n_rows, T, H, bp, g_floor, gate, in, h0, cu, dout, dht, dq, dk, dv, dg,
                                        dbeta, dh0, ws, s, events);
  if (is_bf16 && d == 128)
    return launch_bwd_typed<bf16_t, 128>(n_rows, T, H, bp, g_floor, gate, in, h0, cu, dout, dht, dq, dk, dv, dg,
                                         dbeta, dh0, ws, s, events);
  if (!is_bf16 && d == 64)
    return launch_bwd_typed<float, 64>(n_rows, T, H, bp, g_floor, gate, in, h0, cu, dout, dht, dq, dk, dv, dg,
                                       dbeta, dh0, ws, s, events);
  return (int)hipErrorInvalidValue;
}

}  // namespace kda
