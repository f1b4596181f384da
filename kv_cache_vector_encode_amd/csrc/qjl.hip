// QJL key encode: the MSE encode at the codebook's width plus a 1-bit sketch of the residual.
//
// Method (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv, TurboQuantCompressorV2
// .compress): n = ||x||; codes of y = Pi x / (n + 1e-8) against the codebook (max(b - 1, 1)
// bits); k_mse = n Pi^T c[idx]; r = x - k_mse; store n, the codes, ||r|| and the signs of S r,
// a zero projection counting as +1.
//
// Rotated domain. r_rot = Pi r = Pi x - n c[idx] has ||r_rot|| = ||r||, and
// S r = (S Pi^T) r_rot = M r_rot. The first half of the kernel is the encode kernel's pass: a
// wave owns 32 vectors and lane (v, hh) ends up holding rotated coordinates hh*d/2 + 16t + i of
// vector v in accumulator register i of output tile t. From those registers it forms r_rot and
// its bf16 hi / lo split, which is directly the B operand of a second 32x32x16 product: the
// operand of K block kb is coordinates hh*d/2 + 8kb + e (e < 8), i.e. registers 8(kb%2)..+8 of
// tile kb/2, so M's tiles use the same row and column orders as Pi's and nothing moves between
// lanes. The projections come out in the same layout, so lane (v, hh) holds sign bits
// hh*d/2 .. hh*d/2 + d/2 of vector v: a contiguous d/16-byte piece of the row.
//
// Precision: M r_rot takes three bf16 passes (M_hi r_hi + M_lo r_hi + M_hi r_lo, ~2^-16
// relative), so a sign can differ from the float64 definition only for a projection within a
// few 1e-6 of zero relative to ||S_i|| ||r||.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {

struct QjlKArgs {
  const u32x4* frag;       // Pi tiles (hi, lo) of rotation r at frag + r * frag_stride (u32x4 units)
  const u32x4* mfrag;      // M = S Pi^T tiles (hi, lo), same layout
  int64_t frag_stride, mfrag_stride;
  const void* x;
  int64_t x_row_stride;    // elements
  uint8_t* packed;
  float* norms;
  uint8_t* signs;
  float* rnorms;
  const int64_t* slot;
  uint8_t* sink;           // masked lanes store here (codes, norms, signs, residual norms)
  int64_t n, vpr;
  float lut_scale, lut_off;
  uint32_t lut[kLutBins];
  float cf[kMaxLevels];    // centroids in float32
};

template <int D, int BITS>
struct QjlGeo {
  static constexpr int T = D / 32;                 // output tiles
  static constexpr int KB = D / 16;                // K blocks
  static constexpr int HALF = D / 2;               // coordinates per lane
  static constexpr int ROW = D * BITS / 8;         // packed bytes per vector
  static constexpr int CHUNK = HALF * BITS / 8;    // packed bytes per lane
  static constexpr int CHUNK_DW = CHUNK / 4;
  static constexpr int SROW = D / 8;               // sign bytes per vector
  static constexpr int SCHUNK_DW = D / 64;         // sign words per lane
  static constexpr int FRAG_U4 = 2 * T * KB * 64;  // hi and lo tiles of one matrix
  // Pi and M tiles both sit in LDS up to d = 128 (2 x 64 KiB at d = 128: one 8-wave workgroup
  // per CU); d = 256 reads them from L2.
  static constexpr bool LDS = (D <= 128);
  static constexpr int WG_PER_CU = D == 64 ? 2 : 1;
};
// Waves per workgroup and per SIMD: d = 256 needs the whole register file of a SIMD (the residual
// operands alone take 128 registers), so one 4-wave workgroup per CU there.
template <int D>
constexpr int qjl_waves() { return D == 256 ? 4 : 8; }
template <int D>
constexpr int qjl_wpe() { return D == 64 ? 4 : D == 128 ? 2 : 1; }

// Masked-lane store offsets inside the sink (bytes)
constexpr int kSinkCodes = 0, kSinkNorms = 4096, kSinkSigns = 4352, kSinkRnorms = 5376;

template <int D, int BITS, int IN, bool SLOT>
__global__ void __launch_bounds__(qjl_waves<D>() * 64) __attribute__((amdgpu_waves_per_eu(qjl_wpe<D>())))
qjl_encode_kernel(QjlKArgs a) {
  using Geo = QjlGeo<D, BITS>;
  constexpr int T = Geo::T, KB = Geo::KB, HALF = Geo::HALF;
  constexpr bool SPLIT_X = (IN != TQ_BF16);
  extern __shared__ u32x4 smem[];
  __shared__ uint32_t lut[2 * kLutBins];   // entries at 128 + bin, repeated below
  __shared__ float cf[kMaxLevels];

  const int r = blockIdx.y;
  const u32x4* gp = a.frag + (int64_t)r * a.frag_stride;
  const u32x4* gm = a.mfrag + (int64_t)r * a.mfrag_stride;
  if constexpr (Geo::LDS) {
    for (int i = threadIdx.x; i < Geo::FRAG_U4; i += blockDim.x) {
      smem[i] = gp[i];
      smem[Geo::FRAG_U4 + i] = gm[i];
    }
  }
  {
    // tables straight from the kernel-argument segment (`a` is the only argument)
    const char* ka = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    const uint32_t* klut = (const uint32_t*)(ka + offsetof(QjlKArgs, lut));
    for (int i = threadIdx.x; i < 2 * kLutBins; i += blockDim.x) lut[i] = klut[i & (kLutBins - 1)];
    const float* kcf = (const float*)(ka + offsetof(QjlKArgs, cf));
    if (threadIdx.x < kMaxLevels) cf[threadIdx.x] = kcf[threadIdx.x];
  }
  __syncthreads();
  const char* pbase = Geo::LDS ? (const char*)smem : (const char*)gp;
  const char* mbase = Geo::LDS ? (const char*)(smem + Geo::FRAG_U4) : (const char*)gm;

  const int64_t v_begin = a.vpr ? (int64_t)r * a.vpr : 0;
  const int64_t v_end = a.vpr ? min(a.n, v_begin + a.vpr) : a.n;
  const int64_t ntile = (v_end - v_begin + 31) / 32;
  if (ntile <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vl = lane & 31, hh = lane >> 5;

  // Inputs: lane (v, hh) reads elements 16kb + 8hh .. +7 (K block kb) with 16-byte loads, in the
  // column order of Pi's encode tiles; bf16 tiles are prefetched one tile ahead. Every access is
  // unconditional (masked lanes read row v_begin and write the sink), as in the encode kernel.
  constexpr int ELEM = IN == TQ_F32 ? 4 : 2;
  constexpr int NRAW = HALF * ELEM / 16;
  constexpr int PER = ELEM / 2;          // 16-byte loads per K block
  constexpr bool PREFETCH = (IN == TQ_BF16) && D <= 128;
  constexpr int WAVES = qjl_waves<D>();
  const int64_t wstride = (int64_t)gridDim.x * WAVES;
  auto fetch = [&](int64_t tl, u32x4 (&raw)[NRAW]) -> int64_t {
    const int64_t v = v_begin + tl * 32 + vl;
    const bool ok = v < v_end;
    const int64_t vs = ok ? v : v_begin;
    const uint8_t* xp = (const uint8_t*)a.x + (vs * a.x_row_stride + 8 * hh) * ELEM;
#pragma unroll
    for (int k = 0; k < NRAW; ++k) raw[k] = *(const u32x4*)(xp + (k / PER) * 32 * PER + (k % PER) * 16);
    if constexpr (SLOT) {
      const int64_t s = a.slot[vs];
      return ok ? s : -1;
    } else {
      return ok ? v : -1;
    }
  };
  // tiles go to waves wave-major (as in the encode): an uneven last round is spread over every
  // workgroup instead of falling to a subset of them
  int64_t tile = (int64_t)wave * gridDim.x + blockIdx.x;
  u32x4 xr[NRAW];
  int64_t rown = -1;
  if (PREFETCH) {
    rown = fetch(tile, xr);
    wait_vmem_all();
  }

  for (; tile < ntile; tile += wstride) {
    u32x4 xh[KB], xl[SPLIT_X ? KB : 1];
    int64_t row;
    if constexpr (PREFETCH) {
#pragma unroll
      for (int k = 0; k < NRAW; ++k) xh[k] = xr[k];
      row = rown;
      rown = fetch(tile + wstride, xr);   // past the end this reads row v_begin, unused
    } else {
      row = fetch(tile, xr);
    }

    // ---- norm and the B operands of the rotation
    float ss0 = 0.f, ss1 = 0.f;
    if constexpr (IN == TQ_BF16) {
      if constexpr (!PREFETCH) {
#pragma unroll
        for (int k = 0; k < NRAW; ++k) xh[k] = xr[k];
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        ss0 = dot2_bf16(xh[kb][0], xh[kb][0], ss0);
        ss1 = dot2_bf16(xh[kb][1], xh[kb][1], ss1);
        ss0 = dot2_bf16(xh[kb][2], xh[kb][2], ss0);
        ss1 = dot2_bf16(xh[kb][3], xh[kb][3], ss1);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float v[8];
        if constexpr (IN == TQ_F32) {
          const u32x4 p0 = xr[2 * kb], p1 = xr[2 * kb + 1];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            v[c] = __uint_as_float(p0[c]);
            v[4 + c] = __uint_as_float(p1[c]);
          }
        } else {
          const u32x4 p = xr[kb];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            v[2 * c] = f16_bits_to_f32(p[c]);
            v[2 * c + 1] = f16_bits_to_f32(p[c] >> 16);
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t h0 = f32_to_bf16_bits(v[2 * c]), h1 = f32_to_bf16_bits(v[2 * c + 1]);
          uint32_t l0 = f32_to_bf16_bits(v[2 * c] - bf16_bits_to_f32(h0));
          uint32_t l1 = f32_to_bf16_bits(v[2 * c + 1] - bf16_bits_to_f32(h1));
          xh[kb][c] = h0 | (h1 << 16);
          xl[kb][c] = l0 | (l1 << 16);
          ss0 = fmaf(v[2 * c], v[2 * c], ss0);
          ss1 = fmaf(v[2 * c + 1], v[2 * c + 1], ss1);
        }
      }
    }
    float ss = ss0 + ss1;
    ss += wave_xor(ss, 32);
    const float nrm = sqrtf(ss);
    const float fs = a.lut_scale / (nrm + 1e-8f);
    const float foff = a.lut_off;

    // ---- stage 1: rotate, quantize, pack; residual r_rot = Pi x - n c[idx] as bf16 hi / lo
    //      B operands rh / rl of the sketch product (K block kb = registers 8(kb%2).. of tile kb/2)
    uint32_t aoff = (uint32_t)lane * 16u;
    asm volatile("" : "+v"(aoff));
    uint32_t pk[Geo::CHUNK_DW];
#pragma unroll
    for (int w = 0; w < Geo::CHUNK_DW; ++w) pk[w] = 0u;
    u32x4 rh[KB], rl[KB];
    float rr0 = 0.f, rr1 = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      asm volatile("" : "+v"(aoff));
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (!Geo::LDS && kb % 4 == 0 && kb > 0) asm volatile("" : "+v"(aoff));
        const u32x4 ahi = *(const u32x4*)(pbase + aoff + ((0 * T + t) * KB + kb) * 1024);
        const u32x4 alo = *(const u32x4*)(pbase + aoff + ((1 * T + t) * KB + kb) * 1024);
        acc = mfma32_bf16(ahi, xh[kb], acc);
        acc = mfma32_bf16(alo, xh[kb], acc);
        if constexpr (SPLIT_X) acc = mfma32_bf16(ahi, xl[kb], acc);
      }
      float rv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float f = fmaf(acc[i], fs, foff);
        const uint32_t code = (__float_as_uint(f) - lut[(__float_as_uint(f) >> 16) & 255u]) >> 24;
        const int pos = (16 * t + i) * BITS;
        pk[pos >> 5] |= code << (pos & 31);
        if ((pos & 31) + BITS > 32) pk[(pos >> 5) + 1] |= code >> (32 - (pos & 31));
        rv[i] = fmaf(-nrm, cf[code], acc[i]);
        if (i & 1)
          rr1 = fmaf(rv[i], rv[i], rr1);
        else
          rr0 = fmaf(rv[i], rv[i], rr0);
        if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int w = (16 * t * BITS) >> 5; w <= ((16 * t + 16) * BITS - 1) >> 5; ++w)
        asm volatile("" : "+v"(pk[w]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float v0 = rv[8 * j + 2 * c], v1 = rv[8 * j + 2 * c + 1];
          const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
          const uint32_t l0 = f32_to_bf16_bits(v0 - bf16_bits_to_f32(h0));
          const uint32_t l1 = f32_to_bf16_bits(v1 - bf16_bits_to_f32(h1));
          rh[2 * t + j][c] = h0 | (h1 << 16);
          rl[2 * t + j][c] = l0 | (l1 << 16);
        }
    }
    float rr = rr0 + rr1;
    rr += wave_xor(rr, 32);
    const float rnrm = sqrtf(rr);

    // ---- stage 2: projections M r_rot, one output tile at a time; sign bit = (proj >= 0)
    uint32_t sw[Geo::SCHUNK_DW];
#pragma unroll
    for (int w = 0; w < Geo::SCHUNK_DW; ++w) sw[w] = 0u;
    uint32_t moff = (uint32_t)lane * 16u;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      asm volatile("" : "+v"(moff));
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (!Geo::LDS && kb % 4 == 0 && kb > 0) asm volatile("" : "+v"(moff));
        const u32x4 ahi = *(const u32x4*)(mbase + moff + ((0 * T + t) * KB + kb) * 1024);
        const u32x4 alo = *(const u32x4*)(mbase + moff + ((1 * T + t) * KB + kb) * 1024);
        acc = mfma32_bf16(ahi, rh[kb], acc);
        acc = mfma32_bf16(alo, rh[kb], acc);
        acc = mfma32_bf16(ahi, rl[kb], acc);
      }
      uint32_t bits = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) bits |= (acc[i] >= 0.f ? 1u : 0u) << i;
      sw[t >> 1] |= bits << (16 * (t & 1));
    }

    // ---- stores
    {
      const bool ok = row >= 0;
      uint8_t* dst = ok ? a.packed + row * Geo::ROW + hh * Geo::CHUNK : a.sink + kSinkCodes + 64 * lane;
      float* np = ok && hh == 0 ? a.norms + row : (float*)(a.sink + kSinkNorms) + lane;
      uint8_t* sd = ok ? a.signs + row * Geo::SROW + hh * (Geo::SROW / 2) : a.sink + kSinkSigns + 16 * lane;
      float* rp = ok && hh == 0 ? a.rnorms + row : (float*)(a.sink + kSinkRnorms) + lane;
      if constexpr (Geo::CHUNK % 8 == 0 && Geo::ROW % 8 == 0) {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; w += 2) *(u32x2*)(dst + 4 * w) = u32x2{pk[w], pk[w + 1]};
      } else {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; ++w) *(uint32_t*)(dst + 4 * w) = pk[w];
      }
      if constexpr (Geo::SCHUNK_DW == 4)
        *(u32x4*)sd = u32x4{sw[0], sw[1], sw[2], sw[3]};
      else if constexpr (Geo::SCHUNK_DW == 2)
        *(u32x2*)sd = u32x2{sw[0], sw[1]};
      else
        *(uint32_t*)sd = sw[0];
      *np = nrm;
      *rp = rnrm;
    }
  }
}

template <int D, int BITS, int IN, bool SLOT>
static hipError_t launch_qjl_t(const QjlEncodeLaunch& Q) {
  using Geo = QjlGeo<D, BITS>;
  const EncodeLaunch& L = Q.enc;
  QjlKArgs k;
  k.frag = (const u32x4*)L.rot->enc(0);
  k.frag_stride = (int64_t)(L.rot->enc_stride / sizeof(u32x4));
  k.mfrag = (const u32x4*)Q.qjl->frag(0);
  k.mfrag_stride = (int64_t)(Q.qjl->frag_stride / sizeof(u32x4));
  k.x = L.x;
  k.x_row_stride = L.x_row_stride;
  k.packed = L.packed;
  k.norms = L.norms;
  k.signs = Q.signs;
  k.rnorms = Q.rnorms;
  k.slot = L.slot_mapping;
  k.sink = L.rot->sink();
  k.n = L.n;
  k.vpr = L.vectors_per_rot;
  k.lut_scale = L.lv.lut.scale;
  k.lut_off = L.lv.lut.offset;
  for (int j = 0; j < kLutBins; ++j) k.lut[j] = L.lv.lut.entry[j];
  for (int j = 0; j < kMaxLevels; ++j) k.cf[j] = L.lv.centroid_f32[j];
  const int64_t per_rot = L.vectors_per_rot ? L.vectors_per_rot : L.n;
  const int nrot = L.vectors_per_rot ? (int)((L.n + L.vectors_per_rot - 1) / L.vectors_per_rot) : 1;
  const int64_t tiles = (per_rot + 31) / 32;
  const size_t lds = Geo::LDS ? 2 * Geo::FRAG_U4 * sizeof(u32x4) : 0;
  if (lds > 0) {
    hipError_t e = set_kernel_lds((const void*)qjl_encode_kernel<D, BITS, IN, SLOT>, L.rot->device, lds);
    if (e != hipSuccess) return e;
  }
  const int cu = device_cu_count(L.rot->device);
  const int64_t want = (int64_t)cu * Geo::WG_PER_CU;
  int64_t bx = (want + nrot - 1) / nrot;
  constexpr int WAVES = qjl_waves<D>();
  const int64_t need = (tiles + WAVES - 1) / WAVES;
  if (bx > need) bx = need;
  if (bx < 1) bx = 1;
  dim3 grid((unsigned)bx, (unsigned)nrot);
  hipLaunchKernelGGL((qjl_encode_kernel<D, BITS, IN, SLOT>), grid, dim3(WAVES * 64), lds, L.stream, k);
  return hipGetLastError();
}

template <int D, int BITS, int IN>
static hipError_t qjl_slot(const QjlEncodeLaunch& Q) {
  return Q.enc.slot_mapping ? launch_qjl_t<D, BITS, IN, true>(Q) : launch_qjl_t<D, BITS, IN, false>(Q);
}

template <int D, int BITS>
static hipError_t qjl_in(const QjlEncodeLaunch& Q) {
  switch (Q.enc.x_dtype) {
    case TQ_F32: return qjl_slot<D, BITS, TQ_F32>(Q);
    case TQ_BF16: return qjl_slot<D, BITS, TQ_BF16>(Q);
    default: return qjl_slot<D, BITS, TQ_F16>(Q);
  }
}

template <int D>
static hipError_t qjl_bits(const QjlEncodeLaunch& Q) {
  switch (Q.enc.bits) {
    case 1: return qjl_in<D, 1>(Q);
    case 2: return qjl_in<D, 2>(Q);
    case 3: return qjl_in<D, 3>(Q);
    default: return qjl_in<D, 4>(Q);
  }
}

hipError_t launch_qjl_encode(const QjlEncodeLaunch& Q) {
  switch (Q.enc.rot->d) {
    case 64: return qjl_bits<64>(Q);
    case 128: return qjl_bits<128>(Q);
    default: return qjl_bits<256>(Q);
  }
}

}  // namespace tq
