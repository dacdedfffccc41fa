// Microbenchmarks of the device's own peaks (gfx950), beside which the
// roofline figures quote the vendor's nominal ones: dense bf16 and fp32 MFMA
// throughput and HBM read bandwidth.  A measurement aid, built as its own
// library (libkda_peaks.so); nothing on the KDA path calls it.
//
// The MFMA loops run on register operands only: each wave issues eight
// independent accumulation chains back to back (enough to keep the matrix
// core busy across an MFMA's latency), and every thread writes one float of
// its results, so that the work cannot be dropped.  The read sweep sums a
// buffer with 16-byte non-temporal loads, grid-stride, one float a thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"

namespace {

using kda::bf16x8;
using kda::f32x4;

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) peak_bf16(float* __restrict__ out, int iters) {
  const float t = (float)(threadIdx.x & 63) * 1e-3f;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(t + 0.25f * e);
    b[e] = (__bf16)(0.5f - t + 0.125f * e);
  }
  // distinct starting values: identical chains would let the compiler merge
  // them, and it then shifted their accumulators against one another
  f32x4 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = (f32x4){t + j, t - j, 2.f * t + j, (float)j};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) peak_f32(float* __restrict__ out, int iters) {
  const float a = (float)(threadIdx.x & 63) * 1e-3f, b = 0.5f - a;
  f32x4 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = (f32x4){a + j, a - j, 2.f * a + j, (float)j};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) peak_read(const f32x4* __restrict__ src, int64_t n4, float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n4; x += stride)
    s += __builtin_nontemporal_load(src + x);
  out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

extern "C" {

// FLOP of one MFMA chain step: v_mfma_f32_16x16x32_bf16 (kind 0) or
// v_mfma_f32_16x16x4f32 (kind 1), and the MFMA issues per thread and iteration.
long long kda_peak_flop_per_mfma(int kind) { return kind == 0 ? 2LL * 16 * 16 * 32 : 2LL * 16 * 16 * 4; }
int kda_peak_chains(void) { return kChains; }

// n_wg workgroups of 256 threads (four waves) run `iters` iterations of the
// chains; out holds n_wg * 256 floats.  Returns the launch's hipError_t.
int kda_peak_mfma(int kind, int n_wg, int iters, float* out, void* stream) {
  if (n_wg <= 0 || iters <= 0 || !out || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
  return (int)kda::launch_kernel(kind == 0 ? peak_bf16 : peak_f32, dim3(n_wg), dim3(256), (hipStream_t)stream, out,
                                 iters);
}

// Sums n4 16-byte elements of src with n_wg workgroups of 256 threads; out
// holds n_wg * 256 floats.
int kda_peak_read(const void* src, long long n4, int n_wg, float* out, void* stream) {
  if (!src || !out || n4 <= 0 || n_wg <= 0 || ((uintptr_t)src & 15)) return (int)hipErrorInvalidValue;
  return (int)kda::launch_kernel(peak_read, dim3(n_wg), dim3(256), (hipStream_t)stream, (const f32x4*)src,
                                 (int64_t)n4, out);
}

}  // extern "C"
