// Chunked KDA forward for gfx950: a chunk-local kernel and a state-pass kernel.
//
// Chunk algebra (per sequence and head; chunk rows r = 0..63, state S entering
// the chunk, g floored, Gamma = running sum of g over the chunk's rows):
//   Kt = K e^{Gamma}, Kh = K e^{-Gamma}, Qt = Q e^{Gamma}, Kb = K e^{Gamma_L - Gamma}
//   A  = strict_lower(diag(beta) Kt Kh^T),   T = (I + A)^{-1}
//   Wk = T diag(beta) Kt,   Wv = T diag(beta) V,   P = lower_incl(Qt Kh^T)
//   U  = Wv - Wk S,   O = Qt S + P U,   S <- diag(e^{Gamma_L}) S + Kb^T U
// This is the recurrence S_t = (I - b k k^T) diag(a) S_{t-1} + b k v^T,
// o_t = S_t^T q_t unrolled over one chunk.  Sources: the chunk-parallel,
// inter-chunk recurrence with blocked matrix products is named in "Kimi K3
// 深度拆解" (chenxutan.com), 4.2 "线性注意力与 Delta Rule"; the lower bound on
// the log-decay, which keeps e^{-Gamma} finite so that the diagonal block is a
// dense product too, in "3 分钟看懂 Kimi K3" (landx.limxdynamics.com),
// "第一条主线", Figure 3, and "Kimi K3 发布 47 页技术报告" (163.com), 01.
// With the floor f and 64-token chunks every factor lies in [e^{64 f}, e^{-64 f}].
//
// Kernel 1 (kda_chunk_local): one workgroup per (chunk, head), all chunks in
// parallel.  Everything that does not depend on the incoming state: Gamma,
// A and P (MFMA), T by a blocked triangular inverse in LDS (fp32), Wk and Wv
// (MFMA).  Results go to the workspace already cut into MFMA fragments.
// Kernel 2 (kda_state_pass): one wave per (sequence, head, 16 value columns).
// Columns of S, U and O are independent, so waves never talk to each other.
// The wave walks its sequence's chunks in order, holding its 16 columns of S
// in fp32 accumulator registers; S is rounded to the operand type only as an
// MFMA input.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename T, int D> struct LocalSmem {
  static constexpr int C = 64;
  static constexpr int LDT = D + 16 / (int)sizeof(T);   // [64][D] arrays, elements
  static constexpr int LDC = C + 16 / (int)sizeof(T);   // [D][64] arrays, elements
  static constexpr int LDF = C + 4;                     // fp32 [64][64] arrays
  static constexpr int SZ_ROW = 64 * LDT * (int)sizeof(T);
  static constexpr int SZ_F = 64 * LDF * 4;
  static constexpr int REG = ((SZ_ROW > SZ_F ? SZ_ROW : SZ_F) + 15) / 16 * 16;
  static constexpr int SZ_COL = (D * LDC * (int)sizeof(T) + 15) / 16 * 16;
  static constexpr int NP = 256 / D;                    // token parts in the Gamma scan
  static constexpr int R_Q = 0, R_K = REG, R_G = 2 * REG;   // byte offsets
  static constexpr int R_KTT = 3 * REG, R_VT = 3 * REG + SZ_COL;
  static constexpr int R_TOT = 3 * REG + 2 * SZ_COL;         // fp32 [NP][D]
  static constexpr int R_BETA = R_TOT + NP * D * 4;          // fp32 [64]
  static constexpr int BYTES = R_BETA + 64 * 4;
};

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p) { return Elem<T>::to_f32(*p); }
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p) { return *p; }

// Locate global chunk `gc`: sequence start, chunk's first packed token, length.
__device__ __forceinline__ bool find_chunk(const int32_t* cu, int n_rows, int T, int64_t gc,
                                           int64_t& tok0, int& len) {
  if (!cu) {
    const int64_t per = (T + 63) / 64;
    if (per == 0) return false;
    const int64_t n = gc / per, j = gc % per;
    if (n >= n_rows) return false;
    tok0 = n * (int64_t)T + 64 * j;
    len = (int)min((int64_t)64, (int64_t)T - 64 * j);
    return true;
  }
  int64_t base = 0;
  for (int n = 0; n < n_rows; ++n) {
    const int L = cu[n + 1] - cu[n];
    const int64_t nch = (L + 63) / 64;
    if (gc < base + nch) {
      const int64_t j = gc - base;
      tok0 = cu[n] + 64 * j;
      len = (int)min((int64_t)64, (int64_t)L - 64 * j);
      return true;
    }
    base += nch;
  }
  return false;
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
kda_chunk_local(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                const T* __restrict__ g, const float* __restrict__ beta,
                const int32_t* __restrict__ cu, int n_rows, int T_per, int H, float g_floor,
                uint8_t* __restrict__ ws) {
  typedef ChunkLayout<T, D> L;
  typedef LocalSmem<T, D> M;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = L::KB, NKD = L::NKD, NKC = L::NKC, NP = M::NP, PL = 64 / NP;
  constexpr int LDT = M::LDT, LDC = M::LDC, LDF = M::LDF;
  __shared__ __attribute__((aligned(16))) unsigned char smem[M::BYTES];

  const int64_t gc = blockIdx.x;
  const int h = blockIdx.y;
  int64_t tok0;
  int len;
  if (!find_chunk(cu, n_rows, T_per, gc, tok0, len)) return;  // uniform over the block

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, idx = lane & 15, gq = lane >> 4;
  uint8_t* wsc = ws + ((size_t)gc * H + h) * L::BYTES;

  T* sQ = (T*)(smem + M::R_Q);      // Qt = q e^{Gamma}          [64][LDT]
  T* sK = (T*)(smem + M::R_K);      // Kh = k e^{-Gamma}         [64][LDT]
  T* sG = (T*)(smem + M::R_G);      // beta Kt                    [64][LDT]
  T* sKtT = (T*)(smem + M::R_KTT);  // (beta Kt)^T                [D][LDC]
  T* sVT = (T*)(smem + M::R_VT);    // (beta V)^T                 [D][LDC]
  float* sTot = (float*)(smem + M::R_TOT);
  float* sBeta = (float*)(smem + M::R_BETA);

  // ---- phase 1: beta and per-part sums of the floored log-decay ----------
  if (tid < 64) sBeta[tid] = tid < len ? beta[(tok0 + tid) * H + h] : 0.f;
  const int c = tid % D, part = tid / D, s0 = part * PL;
  auto at = [&](int s, int dd) -> size_t { return ((size_t)(tok0 + s) * H + h) * dd + c; };
  float gf[PL];
  float tot = 0.f;
#pragma unroll
  for (int s = 0; s < PL; ++s) {
    float x = (s0 + s < len) ? ld_f32(g + at(s0 + s, D)) : 0.f;
    x = x < g_floor ? g_floor : x;  // NaN stays NaN
    gf[s] = x;
    tot += x;
  }
  sTot[part * D + c] = tot;
  __syncthreads();

  // ---- phase 2: Gamma, decay factors and all element-wise operands -------
  float off = 0.f, gl = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float t = sTot[p * D + c];
    off += p < part ? t : 0.f;
    gl += t;
  }
  {
    float gam = off;
    float kbar[16];
    T bufK[16 / sizeof(T)], bufV[16 / sizeof(T)];
    constexpr int VW = 16 / sizeof(T);
#pragma unroll
    for (int s = 0; s < PL; ++s) {
      const int r = s0 + s;
      const bool live = r < len;
      const float qv = live ? ld_f32(q + at(r, D)) : 0.f;
      const float kv = live ? ld_f32(k + at(r, D)) : 0.f;
      const float vv = live ? ld_f32(v + at(r, D)) : 0.f;
      const float b = sBeta[r];
      gam += gf[s];
      const float e = __expf(gam), ei = __expf(-gam), eb = __expf(gl - gam);
      sQ[r * LDT + c] = Elem<T>::from_f32(qv * e);
      sK[r * LDT + c] = Elem<T>::from_f32(kv * ei);
      const T bkt = Elem<T>::from_f32(b * kv * e);
      sG[r * LDT + c] = bkt;
      bufK[s % VW] = bkt;
      bufV[s % VW] = Elem<T>::from_f32(b * vv);
      if (s % VW == VW - 1) {
        *(uint4*)(sKtT + c * LDC + r - (VW - 1)) = *(const uint4*)bufK;
        *(uint4*)(sVT + c * LDC + r - (VW - 1)) = *(const uint4*)bufV;
      }
      kbar[s % 16] = kv * eb;
      if (s % 16 == 15) {
        // Kb^T fragment pieces: rows c, k over this 16-token group
        const int s16 = s0 + s - 15, kb = s16 / KB, half = (s16 % KB) / 16;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          T piece[4];
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) piece[e4] = Elem<T>::from_f32(kbar[4 * gg + e4]);
          uint8_t* dst = wsc + L::KBT + (((size_t)(c / 16) * NKC + kb) * 64 + (c % 16) + 16 * gg) * 16 +
                         4 * half * sizeof(T);
          if (sizeof(T) == 2)
            *(uint2*)dst = *(const uint2*)piece;
          else
            *(uint4*)dst = *(const uint4*)piece;
        }
      }
    }
    if (part == 0) ((float*)(wsc + L::GL))[c] = __expf(gl);
  }
  __syncthreads();

  // ---- phase 3: A = beta Kt Kh^T (strict lower), P = Qt Kh^T (lower) -----
  f32x4 accA[4], accP[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    accA[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    accP[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (j <= wave) {
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        const FragT bK = frag_rows(sK, LDT, 16 * j + idx, kb * KB, gq);
        accA[j] = mma(frag_rows(sG, LDT, 16 * wave + idx, kb * KB, gq), bK, accA[j]);
        accP[j] = mma(frag_rows(sQ, LDT, 16 * wave + idx, kb * KB, gq), bK, accP[j]);
      }
    }
  }
  // Qt fragments straight from LDS to the workspace
#pragma unroll
  for (int f = wave; f < 4 * NKD; f += 4) {
    const int t = f / NKD, kb = f % NKD;
    *(FragT*)(wsc + L::QT + ((size_t)f * 64 + lane) * 16) = frag_rows(sQ, LDT, 16 * t + idx, kb * KB, gq);
  }
  __syncthreads();
  float* sA = (float*)(smem + M::R_G);  // A          fp32 [64][LDF]  (reuses beta Kt)
  float* sT = (float*)(smem + M::R_K);  // (I+A)^{-1} fp32 [64][LDF]  (reuses Kh)
  T* sP = (T*)(smem + M::R_Q);          // P          [64][LDC]       (reuses Qt)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * gq + i, s = 16 * j + idx;
      if (j <= wave) sA[r * LDF + s] = s < r ? accA[j][i] : 0.f;
      sP[r * LDC + s] = Elem<T>::from_f32((j <= wave && s <= r) ? accP[j][i] : 0.f);
    }
  }
  __syncthreads();

  // ---- phase 4: T = (I + A)^{-1}, blocked 4 x 4 over 16 x 16 blocks ------
  {
    // diagonal block `wave`: forward substitution, lane idx solves column idx
    const int b0 = 16 * wave;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == idx) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) acc -= sA[(b0 + r) * LDF + b0 + m] * x[m];
      x[r] = acc;
    }
    if (gq == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(b0 + r) * LDF + b0 + idx] = x[r];
    }
    // zero the blocks right of the diagonal in this block row
    for (int e = lane; e < 16 * (48 - b0); e += 64) {
      const int r = e / (48 - b0), cc = e % (48 - b0);
      sT[(b0 + r) * LDF + b0 + 16 + cc] = 0.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    const int i = wave + d, j = wave;
    if (i < 4) {
      // X = sum_{m=j}^{i-1} A_im T_mj ;  T_ij = -T_ii X
      f32x4 X = (f32x4){0.f, 0.f, 0.f, 0.f};
      for (int m = j; m < i; ++m) {
        const f32x4 a = frag_rows(sA, LDF, 16 * i + idx, 16 * m, gq);
        f32x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = sT[(16 * m + 4 * gq + e) * LDF + 16 * j + idx];
        X = mma(a, b, X);
      }
      f32x4 Y = (f32x4){0.f, 0.f, 0.f, 0.f};
      Y = mma(frag_rows(sT, LDF, 16 * i + idx, 16 * i, gq), frag_from_acc(X), Y);
#pragma unroll
      for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * gq + r) * LDF + 16 * j + idx] = -Y[r];
    }
    __syncthreads();
  }

  // ---- phase 5: Wk = T (beta Kt), Wv = T (beta V) -------------------------
  f32x4 accW[D / 16];
  {
    FragT aT[NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) aT[kb] = Frag<T>::from_f32_rows(sT, LDF, 16 * wave + idx, kb * KB, gq);
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      f32x4 wk = (f32x4){0.f, 0.f, 0.f, 0.f}, wv = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        if (kb * KB <= 16 * wave + 15) {
          wk = mma(aT[kb], frag_rows(sKtT, LDC, 16 * ct + idx, kb * KB, gq), wk);
          wv = mma(aT[kb], frag_rows(sVT, LDC, 16 * ct + idx, kb * KB, gq), wv);
        }
      }
      accW[ct] = wk;
      T out[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = Elem<T>::from_f32(wv[i]);
      uint8_t* dst = wsc + L::WV + ((size_t)(ct * 4 + wave) * 64 + lane) * (4 * sizeof(T));
      if (sizeof(T) == 2)
        *(uint2*)dst = *(const uint2*)out;
      else
        *(uint4*)dst = *(const uint4*)out;
    }
  }
  T* sW = (T*)(smem + M::R_G);  // Wk staging [64][LDT] (reuses A)
  __syncthreads();              // every wave is done reading sA
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) sW[(16 * wave + 4 * gq + i) * LDT + 16 * ct + idx] = Elem<T>::from_f32(accW[ct][i]);
  __syncthreads();

  // ---- phase 6: Wk and P fragments to the workspace ----------------------
#pragma unroll
  for (int f = wave; f < 4 * NKD; f += 4) {
    const int t = f / NKD, kb = f % NKD;
    *(FragT*)(wsc + L::WK + ((size_t)f * 64 + lane) * 16) = frag_rows(sW, LDT, 16 * t + idx, kb * KB, gq);
  }
#pragma unroll
  for (int f = wave; f < 4 * NKC; f += 4) {
    const int t = f / NKC, kb = f % NKC;
    *(FragT*)(wsc + L::P + ((size_t)f * 64 + lane) * 16) = frag_rows(sP, LDC, 16 * t + idx, kb * KB, gq);
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
kda_state_pass(const uint8_t* __restrict__ ws, const float* h0, float* ht, T* __restrict__ o,
                const int32_t* __restrict__ cu, int n_rows, int T_per, int H) {
  typedef ChunkLayout<T, D> L;
  typedef typename Frag<T>::type FragT;
  constexpr int KB = L::KB, NKD = L::NKD, NKC = L::NKC, WPP = D / 64;
  const int n_pairs = n_rows * H;
  // XCD-aware order: consecutive block ids go to different XCDs, so all the
  // workgroups of one (sequence, head) get ids with the same residue mod 8
  // and share one XCD's L2 for the chunk operands they all read.
  const int id = blockIdx.x, xcd = id & 7, jj = id >> 3;
  const int p = (jj / WPP) * 8 + xcd, sub = jj % WPP;
  if (p >= n_pairs) return;
  const int n = p / H, h = p % H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, idx = lane & 15, gq = lane >> 4;
  const int vt = sub * 4 + wave, vcol = 16 * vt + idx;

  int64_t tok0, chunk0;
  int len;
  if (cu) {
    chunk0 = 0;
    for (int m = 0; m < n; ++m) chunk0 += (cu[m + 1] - cu[m] + 63) / 64;
    tok0 = cu[n];
    len = cu[n + 1] - cu[n];
  } else {
    tok0 = (int64_t)n * T_per;
    len = T_per;
    chunk0 = (int64_t)n * ((T_per + 63) / 64);
  }

  f32x4 S[D / 16];
  const size_t sbase = (size_t)p * D * D;
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[ct][i] = h0 ? h0[sbase + (size_t)(16 * ct + 4 * gq + i) * D + vcol] : 0.f;

  const int nch = (len + 63) / 64;
  for (int jc = 0; jc < nch; ++jc) {
    const uint8_t* base = ws + ((size_t)(chunk0 + jc) * H + h) * L::BYTES;
    const int clen = min(64, len - 64 * jc);
    auto frag = [&](size_t off, int f) -> FragT { return *(const FragT*)(base + off + ((size_t)f * 64 + lane) * 16); };

    FragT SB[NKD];
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) SB[kb] = Frag<T>::from_acc(S, kb);

    f32x4 U[4], O[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 ws_ = (f32x4){0.f, 0.f, 0.f, 0.f}, qs = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        ws_ = mma(frag(L::WK, t * NKD + kb), SB[kb], ws_);
        qs = mma(frag(L::QT, t * NKD + kb), SB[kb], qs);
      }
      const T* wvp = (const T*)(base + L::WV + ((size_t)(vt * 4 + t) * 64 + lane) * (4 * sizeof(T)));
#pragma unroll
      for (int i = 0; i < 4; ++i) U[t][i] = ld_f32(wvp + i) - ws_[i];
      O[t] = qs;
    }
    FragT UB[NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) UB[kb] = Frag<T>::from_acc(U, kb);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb)
        if (kb * KB <= 16 * t + 15) O[t] = mma(frag(L::P, t * NKC + kb), UB[kb], O[t]);
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      const f32x4 gl = *(const f32x4*)(base + L::GL + (size_t)(16 * ct + 4 * gq) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[ct][i] *= gl[i];
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) S[ct] = mma(frag(L::KBT, ct * NKC + kb), UB[kb], S[ct]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * gq + i;
        if (r < clen) o[((size_t)(tok0 + 64 * jc + r) * H + h) * D + vcol] = Elem<T>::from_f32(O[t][i]);
      }
  }
  if (ht) {
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) ht[sbase + (size_t)(16 * ct + 4 * gq + i) * D + vcol] = S[ct][i];
  }
}

template <typename T, int D>
static int launch_typed(int n_rows, int T_per, int H, int64_t n_chunks, float g_floor, const void* q,
                        const void* k, const void* v, const void* g, const float* beta, const float* h0,
                        const int32_t* cu, void* o, float* ht, void* ws, hipStream_t stream) {
  if (n_chunks > 0) {
    hipLaunchKernelGGL((kda_chunk_local<T, D>), dim3((unsigned)n_chunks, H), dim3(256), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)g, beta, cu, n_rows, T_per, H,
                       g_floor, (uint8_t*)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  const int64_t pairs = (int64_t)n_rows * H;
  const int64_t blocks = (pairs + 7) / 8 * 8 * (D / 64);
  hipLaunchKernelGGL((kda_state_pass<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint8_t*)ws, h0, ht, (T*)o, cu, n_rows, T_per, H);
  return (int)hipGetLastError();
}

size_t chunk_bytes(int is_bf16, int d) {
  if (is_bf16) {
    if (d == 64) return ChunkLayout<bf16_t, 64>::BYTES;
    if (d == 128) return ChunkLayout<bf16_t, 128>::BYTES;
  } else {
    if (d == 64) return ChunkLayout<float, 64>::BYTES;
  }
  return 0;
}

int launch_chunk_forward(int is_bf16, int d, int n_rows, int T, int H, int64_t n_chunks, float g_floor,
                         const void* q, const void* k, const void* v, const void* g, const float* beta,
                         const float* h0, const int32_t* cu, void* o, float* ht, void* ws, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (is_bf16 && d == 64)
    return launch_typed<bf16_t, 64>(n_rows, T, H, n_chunks, g_floor, q, k, v, g, beta, h0, cu, o, ht, ws, s);
  if (is_bf16 && d == 128)
    return launch_typed<bf16_t, 128>(n_rows, T, H, n_chunks, g_floor, q, k, v, g, beta, h0, cu, o, ht, ws, s);
  if (!is_bf16 && d == 64)
    return launch_typed<float, 64>(n_rows, T, H, n_chunks, g_floor, q, k, v, g, beta, h0, cu, o, ht, ws, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace kda
