// Device helpers for the gfx950 kernels: vector types, MFMA wrappers, conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// D(32x32) += A(32x16) B(16x32), bf16 operands, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32]; D register i of lane l
// is row 8*(i/4) + 4*(l/32) + i%4, column l%32.
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                 0);
}
// D(16x16) += A(16x32) B(32x16), fp16 operands. Lane l supplies A[l%16][8*(l/16) .. +8] and
// B[8*(l/16) .. +8][l%16]; D register r of lane l is row 4*(l/16) + r, column l%16.
__device__ __forceinline__ f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu));
}

// bits [s, s+32) of the 64-bit value hi:lo (0 <= s < 32)
__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t s) {
  return __builtin_amdgcn_alignbit(hi, lo, s);
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Two floats -> packed bf16 / fp16 pair (round to nearest even), one instruction on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}

// Number of positive decision boundaries below |z| turned into a code: for z > 0 the code
// is L/2 + count, for z <= 0 its mirror L-1 - (L/2 + count). Equals #{k : t_k < z} except
// exactly on a boundary. `p` holds the positive boundaries already scaled by (||x|| + eps).
// The count is taken by binary search over the sorted boundaries (b-1 compares).
template <int BITS>
__device__ __forceinline__ uint32_t quantize_scaled(float z, const float* p) {
  constexpr uint32_t H = 1u << (BITS - 1);
  const float a = fabsf(z);
  uint32_t u;
  if constexpr (BITS == 2) {
    u = H + (a > p[0] ? 1u : 0u);
  } else if constexpr (BITS == 3) {
    const bool c1 = a > p[1];
    const bool c2 = a > (c1 ? p[2] : p[0]);
    u = H + (c1 ? 2u : 0u) + (c2 ? 1u : 0u);
  } else {
    const bool c1 = a > p[3];
    const float lo = c1 ? p[4] : p[0], hi = c1 ? p[6] : p[2];
    const bool c2 = a > (c1 ? p[5] : p[1]);
    const bool c3 = a > (c2 ? hi : lo);
    u = H + (c1 ? 4u : 0u) + (c2 ? 2u : 0u) + (c3 ? 1u : 0u);
  }
  return z > 0.0f ? u : (u ^ (2u * H - 1u));
}

}  // namespace tq
