// Chunk rows of the KDA inputs, global memory -> registers (gfx950), shared
// by the forward sweeps (which fetch a chunk ahead) and the backward's record
// pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ---- chunk inputs: global -> registers --------------------------------------
// Thread (channel pair cp = tid % (D / 2), part = tid / (D / 2)) holds rows
// 8 part .. 8 part + 7 of channels 2 cp, 2 cp + 1: one 32-bit word of a bf16
// pair (fp32: two floats) per row and tensor, so that one wave's load covers
// whole rows and the prefix sums over a part's rows stay in one thread.
// Each tensor of a chunk is one buffer resource whose range ends with the
// chunk's last row: rows past the chunk's end (a sequence's last chunk) read
// as zeros, with no branch, and every lane's offsets are 32-bit.  gate: g
// per channel, one per (token, head) (replicated over the channels when
// used), or none.  MX: q, k and v arrive as e4m3 bytes (two per pair) with
// their 32-channel block's scale byte, decoded to bf16 when used.  NT: the
// loads are non-temporal (the last read of the inputs).
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 family
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
template <typename T> struct PairT;
template <> struct PairT<bf16_t> {
  typedef uint32_t word;
  __device__ static __forceinline__ float lo(word w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(word w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static __forceinline__ word pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(a, b));
  }
  __device__ static __forceinline__ word splat(word x) { return (x & 0xffffu) | (x << 16); }
  template <int AUX>
  __device__ static __forceinline__ word load(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, AUX);
  }
  template <int AUX>
  __device__ static __forceinline__ word load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
  }
};
template <> struct PairT<float> {
  typedef f32x2 word;
  __device__ static __forceinline__ float lo(word w) { return w[0]; }
  __device__ static __forceinline__ float hi(word w) { return w[1]; }
  __device__ static __forceinline__ word pack(float a, float b) { return (f32x2){a, b}; }
  __device__ static __forceinline__ word splat(word x) { return (f32x2){x[0], x[0]}; }
  template <int AUX>
  __device__ static __forceinline__ word load(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, AUX));
  }
  template <int AUX>
  __device__ static __forceinline__ word load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (f32x2){__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX)), 0.f};
  }
};

template <typename T, int D, bool WITH_Q, bool MX, bool NT> struct Raw {
  typedef PairT<T> PW;
  typedef typename PW::word word;
  static constexpr int NPR = D / 2, ES = (int)sizeof(T);
  static_assert(!MX || sizeof(T) == 2, "MXFP8 inputs feed the bf16 path");
  word q[WITH_Q ? 8 : 1], k[8], v[8], g[8];  // MX: q, k, v hold two e4m3 bytes in the low half
  uint32_t qs[MX && WITH_Q ? 8 : 1], ks[MX ? 8 : 1], vs[MX ? 8 : 1];
  float beta;

  // chunk rows tok0 .. tok0 + clen - 1 (clen >= 1) of head h
  __device__ __forceinline__ void load(const ChunkInputs& in, int64_t tok0, int clen, int H, int h, int tid,
                                       int gate) {
    constexpr int aux = NT ? 2 : 0;                    // non-temporal
    const int cp = tid % NPR, part = tid / NPR;
    const size_t row0 = (size_t)tok0 * H + h;          // first (token, head) row of the chunk
    const uint32_t rs = (uint32_t)H * D;               // row stride, elements
    const uint32_t span = (uint32_t)(clen - 1) * rs + D;  // elements from row0 * D to the chunk's end
    const uint32_t off0 = (uint32_t)(8 * part) * rs + 2 * cp;
    // beta first: loads complete in issue order, so once the chunk's other
    // inputs have arrived beta has too, and its use needs no wait of its own
    const __amdgpu_buffer_rsrc_t rb = rsrc(in.beta + row0, ((uint32_t)(clen - 1) * H + 1) * 4);
    beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)tid * H * 4, 0, aux));
    if (MX) {
      const uint32_t sspan = span / 32;
      const __amdgpu_buffer_rsrc_t rk = rsrc((const uint8_t*)in.k + row0 * D, span);
      const __amdgpu_buffer_rsrc_t rv = rsrc((const uint8_t*)in.v + row0 * D, span);
      const __amdgpu_buffer_rsrc_t rks = rsrc(in.ks + row0 * D / 32, sspan);
      const __amdgpu_buffer_rsrc_t rvs = rsrc(in.vs + row0 * D / 32, sspan);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t off = off0 + (uint32_t)s * rs;
        k[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rk, off, 0, aux);
        v[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, off, 0, aux);
        ks[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rks, off / 32, 0, aux);
        vs[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rvs, off / 32, 0, aux);
      }
      if constexpr (WITH_Q) {
        const __amdgpu_buffer_rsrc_t rq = rsrc((const uint8_t*)in.q + row0 * D, span);
        const __amdgpu_buffer_rsrc_t rqs = rsrc(in.qs + row0 * D / 32, sspan);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint32_t off = off0 + (uint32_t)s * rs;
          q[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rq, off, 0, aux);
          qs[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rqs, off / 32, 0, aux);
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t rk = rsrc((const T*)in.k + row0 * D, span * ES);
      const __amdgpu_buffer_rsrc_t rv = rsrc((const T*)in.v + row0 * D, span * ES);
      // per-row steps as the uniform offset
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        k[s] = PW::template load<aux>(rk, off0 * ES, s * rs * ES);
        v[s] = PW::template load<aux>(rv, off0 * ES, s * rs * ES);
      }
      if constexpr (WITH_Q) {
        const __amdgpu_buffer_rsrc_t rq = rsrc((const T*)in.q + row0 * D, span * ES);
#pragma unroll
        for (int s = 0; s < 8; ++s) q[s] = PW::template load<aux>(rq, off0 * ES, s * rs * ES);
      }
    }
    // g is filled by loads in every mode, without a gate from an empty range
    // (zeros): a plain register write there would make the compiler wait for
    // every load in flight (the next chunk's inputs included) before it
    if (gate == kGateHead) {
      const __amdgpu_buffer_rsrc_t rgt = rsrc((const T*)in.g + row0, ((uint32_t)(clen - 1) * H + 1) * ES);
#pragma unroll
      for (int s = 0; s < 8; ++s) g[s] = PW::template load1<aux>(rgt, (uint32_t)(8 * part + s) * H * ES);
    } else {
      const bool ch = gate == kGateChannel;
      const __amdgpu_buffer_rsrc_t rgt = rsrc(ch ? (const void*)((const T*)in.g + row0 * D) : in.k, ch ? span * ES : 0u);
#pragma unroll
      for (int s = 0; s < 8; ++s) g[s] = PW::template load<aux>(rgt, off0 * ES, s * rs * ES);
    }
  }
  // the pair (2 cp, 2 cp + 1) of row s as operand words
  __device__ static __forceinline__ word dec(word w, uint32_t s) {
    if constexpr (MX) {
      const float sc = __uint_as_float(s ? s << 23 : 0x00400000u);  // 2^(s - 127)
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, sc, false));
    } else {
      return w;
    }
  }
  __device__ __forceinline__ word qw(int s) const { return dec(q[WITH_Q ? s : 0], MX && WITH_Q ? qs[s] : 0u); }
  __device__ __forceinline__ word kw(int s) const { return dec(k[s], MX ? ks[s] : 0u); }
  __device__ __forceinline__ word vw(int s) const { return dec(v[s], MX ? vs[s] : 0u); }
};


// ---- one chunk's rows of an input, read by any element ----------------------
// Rows tok0 .. tok0 + len - 1 (len >= 1) of head h of a [tokens, H, D]
// tensor as one buffer resource: element (r, c) at byte offset
// (r H D + c) sizeof(T), and a read past the last row returns zeros, with no
// branch.
template <typename T> struct ChunkRows {
  __amdgpu_buffer_rsrc_t r;
  uint32_t rs;  // row stride, bytes
  __device__ __forceinline__ ChunkRows(const T* x, int64_t tok0, int len, int H, int h, int D)
      : r(rsrc(x + (tok0 * H + h) * D, ((uint32_t)(len - 1) * H * D + D) * sizeof(T))),
        rs((uint32_t)H * D * sizeof(T)) {}
  // the bits of elements c .. c + 3 of row row (c % 4 == 0; bf16: the low
  // two words), to be widened by to_f32x4 where they are used
  __device__ __forceinline__ uint4 raw4(int row, int c) const {
    const uint32_t off = (uint32_t)row * rs + (uint32_t)c * sizeof(T);
    if constexpr (sizeof(T) == 2) {
      const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
      return make_uint4(u.x, u.y, 0u, 0u);
    } else {
      return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
  }
  __device__ static __forceinline__ f32x4 to_f32x4(const uint4& u) {
    if constexpr (sizeof(T) == 2)
      return (f32x4){__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u)};
    else
      return __builtin_bit_cast(f32x4, u);
  }
  // elements c .. c + 3 of row row (c % 4 == 0)
  __device__ __forceinline__ f32x4 ld4(int row, int c) const {
    const uint32_t off = (uint32_t)row * rs + (uint32_t)c * sizeof(T);
    if constexpr (sizeof(T) == 2) {
      const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
      return (f32x4){__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u)};
    } else {
      return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
  }
};
// The log-decays of one chunk: per channel ([tokens, H, D]), one per
// (token, head) ([tokens, H], the same for every channel), or none (zeros:
// an empty range).
template <typename T> struct GateRows {
  __amdgpu_buffer_rsrc_t r;
  uint32_t rs, cs;  // row and channel strides, bytes
  __device__ __forceinline__ GateRows(const void* g, int gate, int64_t tok0, int len, int H, int h, int D) {
    const T* x = (const T*)g;
    if (gate == kGateChannel) {
      r = rsrc(x + (tok0 * H + h) * D, ((uint32_t)(len - 1) * H * D + D) * sizeof(T));
      rs = (uint32_t)H * D * sizeof(T);
      cs = sizeof(T);
    } else {
      r = gate == kGateHead ? rsrc(x + tok0 * H + h, ((uint32_t)(len - 1) * H + 1) * sizeof(T)) : rsrc(g, 0u);
      rs = (uint32_t)H * sizeof(T);
      cs = 0;
    }
  }
  __device__ __forceinline__ float ld(int row, int c) const {
    const uint32_t off = (uint32_t)row * rs + (uint32_t)c * cs;
    if constexpr (sizeof(T) == 2)
      return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16);
    else
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
};

}  // namespace kda
