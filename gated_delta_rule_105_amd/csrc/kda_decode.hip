// KDA decode step for gfx950: one new token per sequence, state in place.
//
// For each (sequence n, head h), with S the d x d fp32 state (rows = key
// channels c, columns = value channels j):
//   a_c = exp(max(g_c, floor));  w_j = sum_c a_c S_cj k_c;  z_j = sum_c a_c S_cj q_c
//   u_j = beta (v_j - w_j);      S_cj <- a_c S_cj + k_c u_j
//   o_j = z_j + (q . k) u_j      (= S_new^T q)
// i.e. the gated delta rule for a single token ("Kimi K3 深度拆解"
// (chenxutan.com), 4.2 "线性注意力与 Delta Rule"; per-channel gate from
// "Kimi K3 技術報告" (akiraxclaw.com), "長度"); its cost does not depend on the
// context length ("Kimi K3：预训练规模与推理算力" (studioglobal.ai), "KDA 与 Gated MLA").
//
// The step is bound by HBM: the state is read once and written once
// (2 * 4 d^2 bytes per (n, h)); everything else is a few hundred bytes.
// One workgroup owns one (n, h) tile, so the in-place write needs no
// synchronisation beyond the workgroup.  At d = 128 the workgroup has 1024
// threads, each holding a 4-column strip of 4 rows (16-byte non-temporal
// loads, all issued before any arithmetic): the most bytes in flight per CU
// of the launch shapes measured (256 to 1024 threads, one or two tiles per
// workgroup), and non-temporal loads and stores keep the stream out of the
// caches, which held up best when the state is larger than the last-level
// cache.  Column sums over rows are reduced by cross-lane shuffles inside a
// wave and through LDS across waves.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename T>
__device__ __forceinline__ float ldf(const T* p);
template <>
__device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldf<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <int D> struct DecodeShape {
  static constexpr int NTH = D == 128 ? 1024 : 256;  // threads per tile
};

template <typename T, int D>
__global__ void __launch_bounds__(DecodeShape<D>::NTH)
kda_decode(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
           const T* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
           T* __restrict__ o, float g_floor, int gate) {
  constexpr int NTH = DecodeShape<D>::NTH;
  constexpr int CPR = D / 4;         // float4 columns per row
  constexpr int RP = NTH / CPR;      // rows per pass (row groups)
  constexpr int NI = D / RP;         // passes
  constexpr int NWV = NTH / 64;      // waves
  static_assert(RP * CPR == NTH && NI * RP == D && CPR <= 64, "tile layout");
  __shared__ float sA[D], sK[D], sQ[D];
  __shared__ f32x4 sW[NWV][CPR], sZ[NWV][CPR];
  __shared__ float sQK;

  const size_t nh = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cg = tid % CPR, rg = tid / CPR;
  f32x4* S = (f32x4*)(state + nh * D * D);

  // issue the whole strip's loads first; then the gate, key and query into
  // LDS, q.k in wave 0, and this thread's v and beta (that order measured
  // fastest: vector-memory waits retire in issue order)
  f32x4 s[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) s[i] = __builtin_nontemporal_load(&S[(rg + RP * i) * CPR + cg]);

  if (tid < D) {
    // one log-decay per channel, one per head for every channel, or none
    float gg = gate == kGateChannel ? ldf(g + nh * D + tid) : gate == kGateHead ? ldf(g + nh) : 0.f;
    gg = gg < g_floor ? g_floor : gg;  // NaN stays NaN
    sA[tid] = __expf(gg);
    sK[tid] = ldf(k + nh * D + tid);
    sQ[tid] = ldf(q + nh * D + tid);
  }
  if (wave == 0) {
    float qk = 0.f;
    for (int c = lane; c < D; c += 64) qk += ldf(q + nh * D + c) * ldf(k + nh * D + c);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) qk += __shfl_xor(qk, off, 64);
    if (lane == 0) sQK = qk;
  }
  const float b = beta[nh];
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = ldf(v + nh * D + 4 * cg + e);
  __syncthreads();

  // w = S'^T k and z = S'^T q with S' = diag(a) S, partial over this strip
  f32x4 w = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = rg + RP * i;
    const float a = sA[c], kc = sK[c], qc = sQ[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[i][e] *= a;
      w[e] += s[i][e] * kc;
      z[e] += s[i][e] * qc;
    }
  }
  // reduce over the row groups of this wave (lanes cg, cg + CPR, ...)
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] += __shfl_xor(w[e], off, 64);
      z[e] += __shfl_xor(z[e], off, 64);
    }
  if (lane < CPR) {
    sW[wave][cg] = w;
    sZ[wave][cg] = z;
  }
  __syncthreads();
  // u and o for this thread's 4 columns (each thread sums the NWV partials
  // itself: no further barrier)
  f32x4 u, oz;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float ww = 0.f, zz = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWV; ++wv) {
      ww += sW[wv][cg][e];
      zz += sZ[wv][cg][e];
    }
    u[e] = b * (vv[e] - ww);
    oz[e] = zz + sQK * u[e];
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float kc = sK[rg + RP * i];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[i][e] += kc * u[e];
    __builtin_nontemporal_store(s[i], &S[(rg + RP * i) * CPR + cg]);
  }
  // o after the state stores (measured faster than before them)
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[nh * D + 4 * cg + e] = Elem<T>::from_f32(oz[e]);
  }
}

template <typename T, int D>
static int launch_typed(int N, int H, float g_floor, int gate, const void* q, const void* k, const void* v,
                        const void* g, const float* beta, float* state, void* o, hipStream_t s) {
  const size_t blocks = (size_t)N * H;
  if (blocks == 0) return 0;
  return (int)launch_kernel(kda_decode<T, D>, dim3((unsigned)blocks), dim3(DecodeShape<D>::NTH), s, (const T*)q,
                            (const T*)k, (const T*)v, (const T*)g, beta, state, (T*)o, g_floor, gate);
}

int launch_decode_step(int is_bf16, int d, int N, int H, float g_floor, int gate, const void* q, const void* k,
                       const void* v, const void* g, const float* beta, float* state, void* o,
                       void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (is_bf16 && d == 64) return launch_typed<bf16_t, 64>(N, H, g_floor, gate, q, k, v, g, beta, state, o, s);
  if (is_bf16 && d == 128) return launch_typed<bf16_t, 128>(N, H, g_floor, gate, q, k, v, g, beta, state, o, s);
  if (!is_bf16 && d == 64) return launch_typed<float, 64>(N, H, g_floor, gate, q, k, v, g, beta, state, o, s);
  if (!is_bf16 && d == 128) return launch_typed<float, 128>(N, H, g_floor, gate, q, k, v, g, beta, state, o, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace kda
