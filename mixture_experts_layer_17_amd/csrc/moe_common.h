// Shared device helpers for libmoe's gfx950 kernels: element types, 16-byte
// vector access, bf16 rounding and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// bfloat16 is carried as its raw 16-bit pattern in memory.
struct bf16_t {
  uint16_t bits;
};

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_v;
// 16 bytes as a native vector (HIP's uint4 is a struct whose copies become
// memcpy and can pin arrays of it to scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_v;

// float -> bfloat16, round to nearest even (inputs are finite; NaN is kept a
// NaN by forcing a mantissa bit).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Element traits: how many bytes a "k-chunk" of 8 consecutive elements
// occupies, and how to convert.
template <typename T> struct elem;

template <> struct elem<float> {
  static constexpr int bytes = 4;
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};

template <> struct elem<bf16_t> {
  static constexpr int bytes = 2;
  __device__ static float to_f32(bf16_t v) { return bf16_bits_to_f32(v.bits); }
  __device__ static bf16_t from_f32(float v) { return bf16_t{f32_to_bf16_bits(v)}; }
};

// A chunk of 8 consecutive elements along K held by one lane: 16 bytes for
// bf16, 32 bytes for float.
template <typename T> struct chunk8;
template <> struct chunk8<bf16_t> { u32x4 v; };
template <> struct chunk8<float> { u32x4 lo, hi; };

template <typename T>
__device__ __forceinline__ chunk8<T> load_chunk(const T* p);
template <>
__device__ __forceinline__ chunk8<bf16_t> load_chunk<bf16_t>(const bf16_t* p) {
  chunk8<bf16_t> c;
  c.v = *reinterpret_cast<const u32x4*>(p);
  return c;
}
template <>
__device__ __forceinline__ chunk8<float> load_chunk<float>(const float* p) {
  chunk8<float> c;
  c.lo = reinterpret_cast<const u32x4*>(p)[0];
  c.hi = reinterpret_cast<const u32x4*>(p)[1];
  return c;
}

// The same load with the non-temporal hint, for rows read once (the expert
// outputs the combine sums, the per-slot input gradients).
template <typename T>
__device__ __forceinline__ chunk8<T> load_chunk_stream(const T* p) {
  chunk8<T> c;
  if constexpr (sizeof(T) == 2) {
    c.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else {
    c.lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    c.hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
  }
  return c;
}

template <typename T>
__device__ __forceinline__ chunk8<T> zero_chunk() {
  chunk8<T> c;
  if constexpr (sizeof(T) == 2) {
    c.v = u32x4{0u, 0u, 0u, 0u};
  } else {
    c.lo = u32x4{0u, 0u, 0u, 0u};
    c.hi = u32x4{0u, 0u, 0u, 0u};
  }
  return c;
}

// acc += A(16 x 32) * B(32 x 16) where each lane supplies the 8 consecutive
// k values (k = 8 * (lane / 16) + s, s = 0..7) of row (lane % 16) of A and of
// column (lane % 16) of B.  The accumulator layout is the 16x16 MFMA one:
// lane holds C[4 * (lane / 16) + i][lane % 16], i = 0..3.
//
// bf16: one v_mfma_f32_16x16x32_bf16.  float: eight v_mfma_f32_16x16x4_f32,
// instruction s taking element s of every lane's chunk, so lane group g
// supplies k = 8g + s; the union over s covers the same 32 k values.  Any
// such pairing is a valid contraction as long as A and B use the same one.
__device__ __forceinline__ f32x4_v mfma_16x16x32(const chunk8<bf16_t>& a,
                                                 const chunk8<bf16_t>& b,
                                                 f32x4_v acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a.v),
                                                 __builtin_bit_cast(bf16x8_v, b.v),
                                                 acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4_v mfma_16x16x32(const chunk8<float>& a,
                                                 const chunk8<float>& b,
                                                 f32x4_v acc) {
  const float* af0 = reinterpret_cast<const float*>(&a.lo);
  const float* af1 = reinterpret_cast<const float*>(&a.hi);
  const float* bf0 = reinterpret_cast<const float*>(&b.lo);
  const float* bf1 = reinterpret_cast<const float*>(&b.hi);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af0[s], bf0[s], acc, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af1[s], bf1[s], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + expf(-z));
}

// Wave-wide (64 lanes) reductions.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace moe
