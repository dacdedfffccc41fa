// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4).
//
// MFMA operand convention used throughout (checked against the hardware):
// for a 16x16 output tile and a k-block of KB indices, lane l = 16*g + i
// (i = l % 16, g = l / 16) supplies
//     A-fragment: row i of A,    k = 16*(e/4) + 4*g + e%4  for element e
//     B-fragment: column i of B, the same k for element e
// and receives D[4*g + r][i] in accumulator register r (r = 0..3).
//   bf16: v_mfma_f32_16x16x32_bf16, KB = 32, 8 elements (16 bytes) per lane.
//   fp32: v_mfma_f32_16x16x4f32 issued 4 times (element e in issue e),
//         KB = 16, 4 elements (16 bytes) per lane.
// The hardware's own order of k inside a lane is a permutation of the one
// above; a sum over k is invariant under any permutation applied to both
// operands, so the convention only has to be the same for A and B.
// Its payoff: an accumulator tile (rows 4g..4g+3 of column i in lane l) is
// already a B-fragment whose k runs over the tile's rows, so an output can
// feed the next product without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace kda {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint16_t bf16_t;  // storage type of bf16 tensors in memory

// ---- scalar conversions -------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats to two bf16 in one instruction (v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays NaN); a in the low half
__device__ __forceinline__ bf16x2 f32x2_to_bf16x2(float a, float b) {
  return __builtin_convertvector((f32x2){a, b}, bf16x2);
}
// Single halves are read from the packed 32-bit word: bit-casting one lane
// of a bf16 vector to an integer returned the other lane with this compiler.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return (bf16_t)__builtin_bit_cast(uint32_t, f32x2_to_bf16x2(f, 0.f));
}

// Element-type traits: storage type, fragment type, k-block of one MMA step.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int KB = 16;
  typedef f32x4 frag;
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ float from_f32(float x) { return x; }
};
template <> struct Elem<bf16_t> {
  static constexpr int KB = 32;
  typedef bf16x8 frag;
  __device__ static __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ bf16_t from_f32(float x) { return f32_to_bf16(x); }
};

// ---- MMA on one 16x16 tile over one k-block ----------------------------
__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x4& a, const f32x4& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
  return c;
}

// ---- fragments ----------------------------------------------------------
// A- or B-fragment from a row-major array X[row][k] (k contiguous, row
// stride `ld` elements): this lane's row, k-block starting at k0.
__device__ __forceinline__ f32x4 frag_rows(const float* X, int ld, int row, int k0, int g) {
  const float* p = X + row * ld + k0 + 4 * g;
  return *(const f32x4*)p;
}
__device__ __forceinline__ bf16x8 frag_rows(const bf16_t* X, int ld, int row, int k0, int g) {
  const bf16_t* p = X + row * ld + k0 + 4 * g;
  bf16x4 lo = *(const bf16x4*)p;
  bf16x4 hi = *(const bf16x4*)(p + 16);
  return (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// bf16 fragment read from an fp32 row-major array (rounded on the fly)
__device__ __forceinline__ bf16x8 frag_rows_f32_to_bf16(const float* X, int ld, int row, int k0, int g) {
  const float* p = X + row * ld + k0 + 4 * g;
  const f32x4 lo = *(const f32x4*)p;
  const f32x4 hi = *(const f32x4*)(p + 16);
  const bf16x2 a = f32x2_to_bf16x2(lo[0], lo[1]), b = f32x2_to_bf16x2(lo[2], lo[3]);
  const bf16x2 c = f32x2_to_bf16x2(hi[0], hi[1]), d = f32x2_to_bf16x2(hi[2], hi[3]);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// B-fragment from accumulator tiles whose rows run over k.
__device__ __forceinline__ f32x4 frag_from_acc(const f32x4& t0) { return t0; }
__device__ __forceinline__ bf16x8 frag_from_acc(const f32x4& t0, const f32x4& t1) {
  const bf16x2 a = f32x2_to_bf16x2(t0[0], t0[1]), b = f32x2_to_bf16x2(t0[2], t0[3]);
  const bf16x2 c = f32x2_to_bf16x2(t1[0], t1[1]), d = f32x2_to_bf16x2(t1[2], t1[3]);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Uniform view over the two element types for kernels templated on T.
template <typename T> struct Frag;
template <> struct Frag<float> {
  typedef f32x4 type;
  // fragment over k-block kb from accumulator tiles acc[], where tile j
  // covers k = 16 j .. 16 j + 15
  __device__ static __forceinline__ f32x4 from_acc(const f32x4* acc, int kb) { return acc[kb]; }
  __device__ static __forceinline__ f32x4 from_f32_rows(const float* X, int ld, int row, int k0, int g) {
    return frag_rows(X, ld, row, k0, g);
  }
};
template <> struct Frag<bf16_t> {
  typedef bf16x8 type;
  __device__ static __forceinline__ bf16x8 from_acc(const f32x4* acc, int kb) {
    return frag_from_acc(acc[2 * kb], acc[2 * kb + 1]);
  }
  __device__ static __forceinline__ bf16x8 from_f32_rows(const float* X, int ld, int row, int k0, int g) {
    return frag_rows_f32_to_bf16(X, ld, row, k0, g);
  }
};

// ---- launches ---------------------------------------------------------------
// Enqueue `kernel` and return the status of this launch itself: the
// arguments are converted to the kernel's parameter types and handed to
// hipLaunchKernel, whose return value is the launch's own (unlike
// hipGetLastError(), which also reports errors that earlier, unrelated HIP
// calls left on the calling thread).
template <typename K, typename Tup, size_t... I>
hipError_t launch_tuple(K kernel, dim3 grid, dim3 block, hipStream_t stream, Tup& vals, std::index_sequence<I...>) {
  void* ptrs[] = {(void*)&std::get<I>(vals)...};
  return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, stream);
}
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "one argument per kernel parameter");
  std::tuple<std::decay_t<KArgs>...> vals(std::forward<Args>(args)...);
  return launch_tuple(kernel, grid, block, stream, vals, std::index_sequence_for<KArgs...>{});
}

}  // namespace kda
