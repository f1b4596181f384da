// Encode and decode with a Hadamard rotation as an O(d log d) fast Walsh-Hadamard transform.
//
// Method: Turbo Attention PyPI page, "The codec", Hadamard rotation row (the rotation is a
// Walsh-Hadamard transform, here after a seeded sign per channel, so that a few large channels
// are smeared over all coordinates before quantization; the query side uses the same
// rotation). With Pi = H_d diag(s) / sqrt(d) (H_d Sylvester's
// +-1 matrix, H[i][j] = (-1)^popcount(i & j)), the encode of the KV Cache API page
// (TurboQuantCompressorMSE.compress) becomes y = H (s o x) / (sqrt(d) (n + 1e-8)) and its decode
// (decompress) x_hat = (n / sqrt(d)) s o (H c[idx]), since H is symmetric. No matrix is read:
// the transform is log2(d) stages of butterflies in float32, exact to a few float32 roundings
// per stage (~1e-7 of the norm), so codes meet the 1e-5 boundary window and the decode the
// rounding bar with no hi/lo operand splits.
//
// Layout: lane j of a vector's group of L = d/32 lanes owns coordinates 32j .. 32j+31, a
// 64-byte run of a bf16 row, so a wave holds 64/L vectors whose rows are contiguous. Butterfly
// stages 1..16 run inside the lane, stages 32.. across the lanes of the group (shuffles); the
// transform keeps natural order, so lane j ends holding outputs 32j .. 32j+31. The encode
// quantizes them with the same one-subtraction table as the MFMA encode (one boundary per
// bin, the code in the carry) and stores the lane's 32 codes as 4*bits contiguous bytes of the
// packed row; the decode stages its 16-bit outputs in LDS so that each store instruction writes
// 1 KiB of consecutive rows.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {

template <int D>
struct WhtGeo {
  static constexpr int EPL = 32;          // coordinates per lane
  static constexpr int L = D / EPL;       // lanes per vector (2, 4, 8)
  static constexpr int VPW = 64 / L;      // vectors per wave
};
constexpr int kWhtWaves = 4;

// x ^ y across lanes (xor mask m < 8, within a group of 8 lanes): DPP quad permutes for 1 and 2,
// a swizzle for 4
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int iv = __float_as_int(v);
  int r;
  if constexpr (M == 1)
    r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  else if constexpr (M == 2)
    r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  else
    r = __builtin_amdgcn_ds_swizzle(iv, 0x101F);               // and 0x1F, xor 4 (32-lane mode)
  return __int_as_float(r);
}

// Fast Walsh-Hadamard transform of a vector held as 32 floats in each of the group's L lanes
// (lane j = lane % L holds coordinates 32j ..): natural order in, natural order out, unscaled.
template <int LPV>
__device__ __forceinline__ void fwht32(float (&v)[32], int j) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  // across lanes: the lane with the bit clear keeps a + b, the other b' - a' (its own value is
  // the upper operand): v = fma(v, +-1, partner)
  auto stage = [&](auto mk) {
    constexpr int M = decltype(mk)::value;
    const float sg = (j & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = fmaf(v[i], sg, lane_xor<M>(v[i]));
  };
  if constexpr (LPV >= 2) stage(std::integral_constant<int, 1>{});
  if constexpr (LPV >= 4) stage(std::integral_constant<int, 2>{});
  if constexpr (LPV >= 8) stage(std::integral_constant<int, 4>{});
}

template <int LPV>
__device__ __forceinline__ float group_sum(float s) {
  if constexpr (LPV >= 2) s += lane_xor<1>(s);
  if constexpr (LPV >= 4) s += lane_xor<2>(s);
  if constexpr (LPV >= 8) s += lane_xor<4>(s);
  return s;
}

// signs of lane j's 32 coordinates from row 0 of the float32 rotation (Pi[0][c] = s_c / sqrt(d)):
// bit e set when s_{32j+e} = -1
__device__ __forceinline__ uint32_t sign_mask(const float* row0) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const f32x4 v = *(const f32x4*)(row0 + 4 * q);
#pragma unroll
    for (int c = 0; c < 4; ++c) m |= (v[c] < 0.f ? 1u : 0u) << (4 * q + c);
  }
  return m;
}

struct WhtEncArgs {
  const void* x;
  int64_t x_row_stride;     // elements
  uint8_t* packed;
  float* norms;
  const int64_t* slot;
  const float* pi;          // float32 rotations, rotation r at pi + r * pi_stride
  int64_t pi_stride;
  uint8_t* sink;            // where masked lanes store (>= 64 x 16 bytes of codes + 64 norms)
  int64_t n, vpr;
  float lut_scale, lut_off, inv_sqrt_d;
  int32_t norm_correct;
  uint32_t lut[kLutBins];
  float csq[kMaxLevels];
};

template <int D, int BITS, int IN, bool SLOT>
__global__ void __launch_bounds__(kWhtWaves * 64) encode_wht_kernel(WhtEncArgs a) {
  using Geo = WhtGeo<D>;
  constexpr int LPV = Geo::L, VPW = Geo::VPW;
  constexpr int ELEM = IN == TQ_F32 ? 4 : 2;
  constexpr int NRAW = 32 * ELEM / 16;          // 16-byte loads per lane
  constexpr int ROW = D * BITS / 8;             // packed bytes per vector
  __shared__ uint32_t lut[2 * kLutBins];   // entries at 128 + bin, repeated below
  __shared__ float csq[kMaxLevels];

  const int r = blockIdx.y;
  const int64_t v_begin = a.vpr ? (int64_t)r * a.vpr : 0;
  const int64_t v_end = a.vpr ? min(a.n, v_begin + a.vpr) : a.n;
  const int64_t ngroup = (v_end - v_begin + VPW - 1) / VPW;
  if (ngroup <= 0) return;   // uniform per workgroup: no thread is left at the barrier below
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vsub = lane / LPV, j = lane % LPV;

  // Every load and store is issued unconditionally (masked lanes read row v_begin and write the
  // sink): the memory counter is in order, and a branch around an access would make the wait for
  // a prefetched load also wait for the stores issued after it.
  auto fetch = [&](int64_t g, u32x4 (&raw)[NRAW]) -> int64_t {
    const int64_t v = v_begin + g * VPW + vsub;
    const bool ok = v < v_end;
    const int64_t vs = ok ? v : v_begin;
    const uint8_t* xp = (const uint8_t*)a.x + (vs * a.x_row_stride + 32 * j) * ELEM;
#pragma unroll
    for (int k = 0; k < NRAW; ++k) raw[k] = *(const u32x4*)(xp + 16 * k);
    if constexpr (SLOT) {
      const int64_t s = a.slot[vs];
      return ok ? s : -1;
    } else {
      return ok ? v : -1;
    }
  };
  const int64_t gstride = (int64_t)gridDim.x * kWhtWaves;
  int64_t g = (int64_t)blockIdx.x * kWhtWaves + wave;
  u32x4 rawn[NRAW];
  // the first group's loads go out before the table copies and the sign reads
  int64_t rown = fetch(g, rawn);
  {
    const char* ka = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    const uint32_t* klut = (const uint32_t*)(ka + offsetof(WhtEncArgs, lut));
    const float* kcsq = (const float*)(ka + offsetof(WhtEncArgs, csq));
    for (int i = threadIdx.x; i < 2 * kLutBins; i += blockDim.x) lut[i] = klut[i & (kLutBins - 1)];
    if (threadIdx.x < kMaxLevels) csq[threadIdx.x] = kcsq[threadIdx.x];
  }
  const uint32_t smask = sign_mask(a.pi + r * a.pi_stride + 32 * j);
  __syncthreads();
  wait_vmem_all();

  for (; g < ngroup; g += gstride) {
    u32x4 raw[NRAW];
#pragma unroll
    for (int k = 0; k < NRAW; ++k) raw[k] = rawn[k];
    const int64_t row = rown;
    rown = fetch(g + gstride, rawn);   // past the end this reads row v_begin, unused

    // ---- s o x in float32, the sum of squares (two chains of 16 per lane), the transform
    float v[32];
    if constexpr (IN == TQ_F32) {
#pragma unroll
      for (int e = 0; e < 32; ++e) v[e] = __uint_as_float(raw[e / 4][e % 4] ^ (((smask >> e) & 1u) << 31));
    } else {
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const uint32_t p = raw[w / 4][w % 4];
        if constexpr (IN == TQ_BF16) {
          // bf16 -> f32 is a shift; the sign flips ride on the bf16 sign bits
          const uint32_t sw = (((smask >> (2 * w)) & 1u) << 15) | (((smask >> (2 * w + 1)) & 1u) << 31);
          const uint32_t q = p ^ sw;
          v[2 * w] = __uint_as_float(q << 16);
          v[2 * w + 1] = __uint_as_float(q & 0xffff0000u);
        } else {
          v[2 * w] = __uint_as_float(__float_as_uint(f16_bits_to_f32(p)) ^ (((smask >> (2 * w)) & 1u) << 31));
          v[2 * w + 1] = __uint_as_float(__float_as_uint(f16_bits_to_f32(p >> 16)) ^ (((smask >> (2 * w + 1)) & 1u) << 31));
        }
      }
    }
    float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      ss0 = fmaf(v[e], v[e], ss0);
      ss1 = fmaf(v[e + 1], v[e + 1], ss1);
    }
    const float nrm = sqrtf(group_sum<LPV>(ss0 + ss1));
    fwht32<LPV>(v, j);

    // ---- quantize: f = y * s + o with y = z / (sqrt(d) (n + 1e-8)), code in the carry of
    //      bits(f) - entry (the table of the MFMA encode); pack LSB-first, code e at bit e*BITS
    const float fs = a.lut_scale * a.inv_sqrt_d / (nrm + 1e-8f);
    const float foff = a.lut_off;
    uint32_t pk[BITS];
#pragma unroll
    for (int w = 0; w < BITS; ++w) pk[w] = 0u;
    float cs0 = 0.f, cs1 = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float f = fmaf(v[e], fs, foff);
      const uint32_t code = (__float_as_uint(f) - lut[(__float_as_uint(f) >> 16) & 255u]) >> 24;
      const int pos = e * BITS;
      pk[pos >> 5] |= code << (pos & 31);
      if ((pos & 31) + BITS > 32) pk[(pos >> 5) + 1] |= code >> (32 - (pos & 31));
      if (a.norm_correct) {
        if (e & 1)
          cs1 += csq[code];
        else
          cs0 += csq[code];
      }
    }
    // norm correction (Turbo Attention page, "The codec", Norms row): n / ||c[idx]||
    float nst = nrm;
    if (a.norm_correct) nst = nrm / sqrtf(group_sum<LPV>(cs0 + cs1));

    // ---- store: the lane's 4*BITS bytes of the packed row (consecutive lanes, consecutive bytes)
    const bool ok = row >= 0;
    uint8_t* dst = ok ? a.packed + row * ROW + j * (4 * BITS) : a.sink + 16 * lane;
    if constexpr (BITS == 4) {
      *(u32x4*)dst = u32x4{pk[0], pk[1], pk[2], pk[3]};
    } else if constexpr (BITS == 2) {
      *(u32x2*)dst = u32x2{pk[0], pk[1]};
    } else {
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      *(u32x3*)dst = u32x3{pk[0], pk[1], pk[2]};
    }
    float* np = ok && j == 0 ? a.norms + row : (float*)(a.sink + 4096) + lane;
    *np = nst;
  }
}

struct WhtDecArgs {
  const uint8_t* packed;
  const float* norms;
  const int64_t* slot;
  void* out;
  const float* pi;
  int64_t pi_stride;
  const uint8_t* zero;      // zeros that masked lanes load (>= 16 bytes)
  uint8_t* sink;            // where masked lanes store (>= 64 x 16 bytes)
  int64_t n, vpr;
  float inv_sqrt_d;
  float cent[kMaxLevels];   // centroids in float32
};

template <int D, int BITS, int OUT, bool SLOT>
__global__ void __launch_bounds__(kWhtWaves * 64) decode_wht_kernel(WhtDecArgs a) {
  using Geo = WhtGeo<D>;
  constexpr int LPV = Geo::L, VPW = Geo::VPW;
  constexpr int ROW = D * BITS / 8;
  constexpr int E = OUT == TQ_F32 ? 4 : 2;       // output bytes per element
  constexpr int LB = 32 * E;                     // output bytes per lane
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  __shared__ float cent[kMaxLevels];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWhtWaves][64 * LB];

  const int r = blockIdx.y;
  const int64_t v_begin = a.vpr ? (int64_t)r * a.vpr : 0;
  const int64_t v_end = a.vpr ? min(a.n, v_begin + a.vpr) : a.n;
  const int64_t ngroup = (v_end - v_begin + VPW - 1) / VPW;
  if (ngroup <= 0) return;   // uniform per workgroup: no thread is left at the barrier below
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vsub = lane / LPV, j = lane % LPV;
  uint8_t* stg = &stage[wave][0];

  auto row_of = [&](int64_t g) -> int64_t {
    const int64_t v = v_begin + g * VPW + vsub;
    const bool ok = g < ngroup && v < v_end;
    if constexpr (SLOT) {
      const int64_t s = a.slot[ok ? v : v_begin];
      return ok ? s : -1;
    } else {
      return ok ? v : -1;
    }
  };
  auto fetch = [&](int64_t row, uint32_t (&cw)[BITS], float& nrm) {
    const uint8_t* src = row >= 0 ? a.packed + row * ROW + j * (4 * BITS) : a.zero;
    if constexpr (BITS == 4) {
      const u32x4 q = *(const u32x4*)src;
      cw[0] = q[0]; cw[1] = q[1]; cw[2] = q[2]; cw[3] = q[3];
    } else if constexpr (BITS == 2) {
      const u32x2 q = *(const u32x2*)src;
      cw[0] = q[0]; cw[1] = q[1];
    } else {
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 q = *(const u32x3*)src;
      cw[0] = q[0]; cw[1] = q[1]; cw[2] = q[2];
    }
    nrm = *(row >= 0 ? a.norms + row : (const float*)a.zero);
  };
  const int64_t gstride = (int64_t)gridDim.x * kWhtWaves;
  int64_t g = (int64_t)blockIdx.x * kWhtWaves + wave;
  uint32_t cwn[BITS];
  float nrmn;
  fetch(row_of(g), cwn, nrmn);
  int64_t row_nn = row_of(g + gstride);
  {
    const float* kc = (const float*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(WhtDecArgs, cent));
    if (threadIdx.x < kMaxLevels) cent[threadIdx.x] = kc[threadIdx.x];
  }
  const uint32_t smask = sign_mask(a.pi + r * a.pi_stride + 32 * j);
  __syncthreads();
  wait_vmem_all();

  for (; g < ngroup; g += gstride) {
    uint32_t cw[BITS];
#pragma unroll
    for (int w = 0; w < BITS; ++w) cw[w] = cwn[w];
    const float nrm = nrmn;
    const int64_t gbase = v_begin + g * VPW;
    fetch(row_nn, cwn, nrmn);
    row_nn = row_of(g + 2 * gstride);

    float v[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int pos = e * BITS;
      uint32_t code = cw[pos >> 5] >> (pos & 31);
      if ((pos & 31) + BITS > 32) code |= cw[(pos >> 5) + 1] << (32 - (pos & 31));
      v[e] = cent[code & MASK];
    }
    fwht32<LPV>(v, j);
    // x_hat = (n / sqrt(d)) s o z, rounded to the output type
    const float sc = nrm * a.inv_sqrt_d;
    u32x4 ch[LB / 16];
    if constexpr (OUT == TQ_F32) {
#pragma unroll
      for (int e = 0; e < 32; ++e)
        ch[e / 4][e % 4] = __float_as_uint(v[e] * sc) ^ (((smask >> e) & 1u) << 31);
    } else {
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const float lo = __uint_as_float(__float_as_uint(v[2 * w] * sc) ^ (((smask >> (2 * w)) & 1u) << 31));
        const float hi = __uint_as_float(__float_as_uint(v[2 * w + 1] * sc) ^ (((smask >> (2 * w + 1)) & 1u) << 31));
        ch[w / 4][w % 4] = OUT == TQ_BF16 ? pack_bf16x2(lo, hi) : pack_f16x2(lo, hi);
      }
    }
    // the wave's VPW rows are one contiguous block of 64 * LB bytes with lane l's LB bytes at
    // 64... l * LB: staged in LDS (16-byte chunks XOR-swizzled by lane so that the 64 lanes'
    // writes spread over banks) and stored 1 KiB per instruction
    constexpr uint32_t NC = LB / 16;             // 16-byte chunks per lane
#pragma unroll
    for (uint32_t c = 0; c < NC; ++c) *(u32x4*)(stg + 16 * (lane * NC + (c ^ (lane & (NC - 1))))) = ch[c];
    uint8_t* tbase = (uint8_t*)a.out + gbase * (int64_t)(D * E);
#pragma unroll
    for (uint32_t k = 0; k < NC; ++k) {
      const uint32_t off = 1024u * k + 16u * lane;        // byte offset in the wave's block
      const uint32_t ln = off / LB, c = (off % LB) / 16;  // the lane and chunk that hold it
      const u32x4 q = *(const u32x4*)(stg + 16 * (ln * NC + (c ^ (ln & (NC - 1)))));
      const int64_t vv = gbase + ln / LPV;
      uint8_t* dst = vv < v_end ? tbase + off : a.sink + 16 * lane;
      __builtin_nontemporal_store(q, (u32x4*)dst);
    }
  }
}

// ---- launchers ---------------------------------------------------------------------------

template <int D, int BITS, int IN, bool SLOT>
static hipError_t launch_enc_wht_t(const EncodeLaunch& L) {
  using Geo = WhtGeo<D>;
  WhtEncArgs k;
  k.x = L.x;
  k.x_row_stride = L.x_row_stride;
  k.packed = L.packed;
  k.norms = L.norms;
  k.slot = L.slot_mapping;
  k.pi = L.rot->f32(0);
  k.pi_stride = (int64_t)(L.rot->f32_stride / sizeof(float));
  k.sink = L.rot->sink();
  k.n = L.n;
  k.vpr = L.vectors_per_rot;
  k.lut_scale = L.lv.lut.scale;
  k.lut_off = L.lv.lut.offset;
  k.inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
  k.norm_correct = L.norm_correct ? 1 : 0;
  for (int i = 0; i < kLutBins; ++i) k.lut[i] = L.lv.lut.entry[i];
  for (int i = 0; i < kMaxLevels; ++i) k.csq[i] = L.lv.centroid_sq[i];
  const int64_t per_rot = L.vectors_per_rot ? L.vectors_per_rot : L.n;
  const int nrot = L.vectors_per_rot ? (int)((L.n + L.vectors_per_rot - 1) / L.vectors_per_rot) : 1;
  const int64_t groups = (per_rot + Geo::VPW - 1) / Geo::VPW;
  const int cu = device_cu_count(L.rot->device);
  int64_t bx = ((int64_t)cu * 4 + nrot - 1) / nrot;   // 16 waves per CU
  const int64_t need = (groups + kWhtWaves - 1) / kWhtWaves;
  if (bx > need) bx = need;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL((encode_wht_kernel<D, BITS, IN, SLOT>), dim3((unsigned)bx, (unsigned)nrot), dim3(kWhtWaves * 64),
                     0, L.stream, k);
  return hipGetLastError();
}

template <int D, int BITS, int OUT, bool SLOT>
static hipError_t launch_dec_wht_t(const DecodeLaunch& L) {
  using Geo = WhtGeo<D>;
  WhtDecArgs k;
  k.packed = L.packed;
  k.norms = L.norms;
  k.slot = L.slot_mapping;
  k.out = L.out;
  k.pi = L.rot->f32(0);
  k.pi_stride = (int64_t)(L.rot->f32_stride / sizeof(float));
  k.zero = L.rot->zero();
  k.sink = L.rot->sink();
  k.n = L.n;
  k.vpr = L.vectors_per_rot;
  k.inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
  for (int i = 0; i < kMaxLevels; ++i) k.cent[i] = L.lv.centroid_f32[i];
  const int64_t per_rot = L.vectors_per_rot ? L.vectors_per_rot : L.n;
  const int nrot = L.vectors_per_rot ? (int)((L.n + L.vectors_per_rot - 1) / L.vectors_per_rot) : 1;
  const int64_t groups = (per_rot + Geo::VPW - 1) / Geo::VPW;
  const int cu = device_cu_count(L.rot->device);
  int64_t bx = ((int64_t)cu * 2 + nrot - 1) / nrot;   // 8 waves per CU (the decode is bound by its stores)
  const int64_t need = (groups + kWhtWaves - 1) / kWhtWaves;
  if (bx > need) bx = need;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL((decode_wht_kernel<D, BITS, OUT, SLOT>), dim3((unsigned)bx, (unsigned)nrot), dim3(kWhtWaves * 64),
                     0, L.stream, k);
  return hipGetLastError();
}

template <int D, int BITS>
static hipError_t enc_wht_in(const EncodeLaunch& L) {
  const bool s = L.slot_mapping != nullptr;
  switch (L.x_dtype) {
    case TQ_F32: return s ? launch_enc_wht_t<D, BITS, TQ_F32, true>(L) : launch_enc_wht_t<D, BITS, TQ_F32, false>(L);
    case TQ_BF16: return s ? launch_enc_wht_t<D, BITS, TQ_BF16, true>(L) : launch_enc_wht_t<D, BITS, TQ_BF16, false>(L);
    default: return s ? launch_enc_wht_t<D, BITS, TQ_F16, true>(L) : launch_enc_wht_t<D, BITS, TQ_F16, false>(L);
  }
}

template <int D, int BITS>
static hipError_t dec_wht_out(const DecodeLaunch& L) {
  const bool s = L.slot_mapping != nullptr;
  switch (L.out_dtype) {
    case TQ_F32: return s ? launch_dec_wht_t<D, BITS, TQ_F32, true>(L) : launch_dec_wht_t<D, BITS, TQ_F32, false>(L);
    case TQ_BF16: return s ? launch_dec_wht_t<D, BITS, TQ_BF16, true>(L) : launch_dec_wht_t<D, BITS, TQ_BF16, false>(L);
    default: return s ? launch_dec_wht_t<D, BITS, TQ_F16, true>(L) : launch_dec_wht_t<D, BITS, TQ_F16, false>(L);
  }
}

template <int D>
static hipError_t enc_wht_bits(const EncodeLaunch& L) {
  switch (L.bits) {
    case 2: return enc_wht_in<D, 2>(L);
    case 3: return enc_wht_in<D, 3>(L);
    default: return enc_wht_in<D, 4>(L);
  }
}

template <int D>
static hipError_t dec_wht_bits(const DecodeLaunch& L) {
  switch (L.bits) {
    case 2: return dec_wht_out<D, 2>(L);
    case 3: return dec_wht_out<D, 3>(L);
    default: return dec_wht_out<D, 4>(L);
  }
}

hipError_t launch_encode_wht(const EncodeLaunch& L) {
  switch (L.rot->d) {
    case 64: return enc_wht_bits<64>(L);
    case 128: return enc_wht_bits<128>(L);
    default: return enc_wht_bits<256>(L);
  }
}

hipError_t launch_decode_wht(const DecodeLaunch& L) {
  switch (L.rot->d) {
    case 64: return dec_wht_bits<64>(L);
    case 128: return dec_wht_bits<128>(L);
    default: return dec_wht_bits<256>(L);
  }
}

}  // namespace tq
