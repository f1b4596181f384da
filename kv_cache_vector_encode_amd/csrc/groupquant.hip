// Affine group quantization of value vectors (KV Cache API page, quantize_values /
// dequantize_values): per group of 32 consecutive elements, zero = min, scale = max((max - min)
// / (2^b - 1), 1e-12), q = clamp(round_half_even((x - zero) / scale), 0, 2^b - 1); scale and
// zero kept in float16; x_hat = q * scale + zero. Every step is an IEEE float32 operation on
// the page, so the kernels use correctly rounded float32 division and no fused multiply-add:
// codes, metadata and reconstructions equal the float32 definition bit for bit.
//
// Encode: one thread owns one group: it reads the group's 32 elements with 16-byte loads,
// reduces min / max, quantizes, and writes the 32 codes (4*b bytes, the LSB-first bitstream of
// the key codes) and the two float16 values. Threads are laid out along the flattened groups,
// so a wave covers 64 consecutive groups.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {

constexpr int kGqGroup = 32;

struct GqEncKArgs {
  const void* x;
  int64_t x_row_stride;   // elements
  uint8_t* packed;
  uint16_t* scales;
  uint16_t* zeros;
  int64_t n_groups;       // n * d / 32
  int32_t groups_per_row;
};

template <int IN>
__device__ __forceinline__ void gq_load(const void* x, int64_t off, float (&v)[kGqGroup]) {
  if constexpr (IN == TQ_F32) {
#pragma unroll
    for (int k = 0; k < kGqGroup / 4; ++k) {
      const u32x4 q = *(const u32x4*)((const float*)x + off + 4 * k);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * k + c] = __uint_as_float(q[c]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kGqGroup / 8; ++k) {
      const u32x4 q = *(const u32x4*)((const uint16_t*)x + off + 8 * k);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[8 * k + 2 * c] = IN == TQ_BF16 ? bf16_lo_to_f32(q[c]) : f16_bits_to_f32(q[c]);
        v[8 * k + 2 * c + 1] = IN == TQ_BF16 ? bf16_hi_to_f32(q[c]) : f16_bits_to_f32(q[c] >> 16);
      }
    }
  }
}

template <int BITS, int IN>
__global__ void __launch_bounds__(256) gq_encode_kernel(GqEncKArgs a) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= a.n_groups) return;
  const int64_t row = gi / a.groups_per_row;
  const int g = (int)(gi - row * a.groups_per_row);
  float v[kGqGroup];
  gq_load<IN>(a.x, row * a.x_row_stride + g * kGqGroup, v);
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int k = 1; k < kGqGroup; ++k) {
    mn = fminf(mn, v[k]);
    mx = fmaxf(mx, v[k]);
  }
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  const float scale = fmaxf(__fdiv_rn(__fsub_rn(mx, mn), LEVELS), 1e-12f);
  constexpr int NW = kGqGroup * BITS / 32;   // packed dwords per group
  uint32_t pk[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) pk[w] = 0u;
#pragma unroll
  for (int k = 0; k < kGqGroup; ++k) {
    const float t = __fdiv_rn(__fsub_rn(v[k], mn), scale);
    const float r = fminf(fmaxf(rintf(t), 0.f), LEVELS);
    const uint32_t q = (uint32_t)r;
    const int pos = k * BITS;
    pk[pos >> 5] |= q << (pos & 31);
    if ((pos & 31) + BITS > 32) pk[(pos >> 5) + 1] |= q >> (32 - (pos & 31));
  }
  uint32_t* dst = (uint32_t*)(a.packed + gi * (kGqGroup * BITS / 8));
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int w = 0; w < NW; w += 4) *(u32x4*)(dst + w) = u32x4{pk[w], pk[w + 1], pk[w + 2], pk[w + 3]};
  } else if constexpr (NW == 2) {
    *(u32x2*)dst = u32x2{pk[0], pk[1]};
  } else {
#pragma unroll
    for (int w = 0; w < NW; ++w) dst[w] = pk[w];
  }
  a.scales[gi] = (uint16_t)f32_to_f16_bits(scale);
  a.zeros[gi] = (uint16_t)f32_to_f16_bits(mn);
}

struct GqDecKArgs {
  const uint8_t* packed;
  const uint16_t* scales;
  const uint16_t* zeros;
  void* out;
  int64_t n_groups;
};

// Decode: four threads per group, each producing 8 consecutive outputs, so that consecutive
// threads write consecutive 16-byte pieces (fully coalesced stores).
template <int BITS, int OUT>
__global__ void __launch_bounds__(256) gq_decode_kernel(GqDecKArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gi = t >> 2;
  const int q4 = (int)(t & 3);
  if (gi >= a.n_groups) return;
  constexpr int NW = kGqGroup * BITS / 32;
  uint32_t pk[NW];
  const uint32_t* src = (const uint32_t*)(a.packed + gi * (kGqGroup * BITS / 8));
#pragma unroll
  for (int w = 0; w < NW; ++w) pk[w] = src[w];
  const float s = f16_bits_to_f32(a.scales[gi]), z = f16_bits_to_f32(a.zeros[gi]);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pos = (8 * q4 + e) * BITS;   // q4 is not a compile-time value: index by cases
    uint32_t q = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w == (pos >> 5)) q = pk[w] >> (pos & 31);
    if ((pos & 31) + BITS > 32) {
#pragma unroll
      for (int w = 1; w < NW; ++w)
        if (w == (pos >> 5) + 1) q |= pk[w] << (32 - (pos & 31));
    }
    q &= (1u << BITS) - 1u;
    o[e] = __fadd_rn(__fmul_rn((float)q, s), z);   // a product then a sum, as on the page
  }
  if constexpr (OUT == TQ_F32) {
    float* dst = (float*)a.out + gi * kGqGroup + 8 * q4;
    *(u32x4*)dst = u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
    *(u32x4*)(dst + 4) =
        u32x4{__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])};
  } else {
    uint16_t* dst = (uint16_t*)a.out + gi * kGqGroup + 8 * q4;
    uint32_t w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      w[c] = OUT == TQ_BF16 ? pack_bf16x2(o[2 * c], o[2 * c + 1]) : pack_f16x2(o[2 * c], o[2 * c + 1]);
    *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
  }
}

template <int BITS>
static hipError_t gq_enc_in(const GqLaunch& L, const GqEncKArgs& k, dim3 grid) {
  switch (L.dtype) {
    case TQ_F32: hipLaunchKernelGGL((gq_encode_kernel<BITS, TQ_F32>), grid, dim3(256), 0, L.stream, k); break;
    case TQ_BF16: hipLaunchKernelGGL((gq_encode_kernel<BITS, TQ_BF16>), grid, dim3(256), 0, L.stream, k); break;
    default: hipLaunchKernelGGL((gq_encode_kernel<BITS, TQ_F16>), grid, dim3(256), 0, L.stream, k);
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t gq_dec_out(const GqLaunch& L, const GqDecKArgs& k, dim3 grid) {
  switch (L.dtype) {
    case TQ_F32: hipLaunchKernelGGL((gq_decode_kernel<BITS, TQ_F32>), grid, dim3(256), 0, L.stream, k); break;
    case TQ_BF16: hipLaunchKernelGGL((gq_decode_kernel<BITS, TQ_BF16>), grid, dim3(256), 0, L.stream, k); break;
    default: hipLaunchKernelGGL((gq_decode_kernel<BITS, TQ_F16>), grid, dim3(256), 0, L.stream, k);
  }
  return hipGetLastError();
}

hipError_t launch_gq(const GqLaunch& L) {
  const int64_t n_groups = L.n * (L.d / kGqGroup);
  if (n_groups == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_groups + 255) / 256));
  if (L.encode) {
    GqEncKArgs k;
    k.x = L.x;
    k.x_row_stride = L.x_row_stride;
    k.packed = L.packed;
    k.scales = L.scales;
    k.zeros = L.zeros;
    k.n_groups = n_groups;
    k.groups_per_row = L.d / kGqGroup;
    switch (L.bits) {
      case 2: return gq_enc_in<2>(L, k, grid);
      case 3: return gq_enc_in<3>(L, k, grid);
      case 4: return gq_enc_in<4>(L, k, grid);
      default: return gq_enc_in<8>(L, k, grid);
    }
  }
  const dim3 dgrid((unsigned)((4 * n_groups + 255) / 256));   // four threads per group
  GqDecKArgs k;
  k.packed = L.packed;
  k.scales = L.scales;
  k.zeros = L.zeros;
  k.out = L.out;
  k.n_groups = n_groups;
  switch (L.bits) {
    case 2: return gq_dec_out<2>(L, k, dgrid);
    case 3: return gq_dec_out<3>(L, k, dgrid);
    case 4: return gq_dec_out<4>(L, k, dgrid);
    default: return gq_dec_out<8>(L, k, dgrid);
  }
}

}  // namespace tq
