// Decode kernel: unpack, centroid lookup, inverse rotation and norm scaling.
//
// Method (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv, TurboQuantCompressorMSE
// .decompress): x_hat = (c[idx] Pi) * n, cast to the output dtype.
//
// Layout mirrors the encode: a wave owns 32 vectors; lane (v, hh) reads the packed chunk
// of rotated coordinates hh*d/2 .. +d/2 of vector v, turns 8 codes at a time into an fp16
// MFMA B operand, and one 32x32x16 fp16 MFMA per (output tile, K block) against prebuilt
// tiles of Pi^T (resident in LDS) leaves output coordinates hh*d/2 + 16t + i in accumulator
// register i, which are scaled by n and stored 16 at a time. fp16 operands (2^-11 relative)
// keep the decode within ~2e-4 of the float64 result, well inside the 2e-3 parity bound.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {

struct DecodeKArgs {
  const u32x4* frag;
  int64_t frag_stride;
  const uint8_t* packed;
  const float* norms;
  const int64_t* slot;
  void* out;
  int64_t n, vpr;
  uint32_t ctab[8];   // 16 fp16 centroids, two per word
};

constexpr int kDecWaves = 8;

template <int D, int BITS>
struct DecGeo {
  static constexpr int T = D / 32, KB = D / 16, HALF = D / 2;
  static constexpr int ROW = D * BITS / 8;
  static constexpr int CHUNK = HALF * BITS / 8;
  static constexpr int CHUNK_DW = CHUNK / 4;
  static constexpr int G = (CHUNK % 16 == 0 && ROW % 16 == 0) ? 16 : ((CHUNK % 8 == 0 && ROW % 8 == 0) ? 8 : 4);
  static constexpr int FRAG_U4 = T * KB * 64;
};

template <int D, int BITS, int OUT>
__global__ void __launch_bounds__(kDecWaves * 64) decode_kernel(DecodeKArgs a) {
  using Geo = DecGeo<D, BITS>;
  constexpr int T = Geo::T, KB = Geo::KB, HALF = Geo::HALF;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  extern __shared__ u32x4 smem[];
  __shared__ uint16_t ctab[16];

  const int r = blockIdx.y;
  const u32x4* gfrag = a.frag + (int64_t)r * a.frag_stride;
  for (int i = threadIdx.x; i < Geo::FRAG_U4; i += blockDim.x) smem[i] = gfrag[i];
  if (threadIdx.x < 16) ctab[threadIdx.x] = (uint16_t)(a.ctab[threadIdx.x >> 1] >> (16 * (threadIdx.x & 1)));
  __syncthreads();

  const int64_t v_begin = a.vpr ? (int64_t)r * a.vpr : 0;
  const int64_t v_end = a.vpr ? min(a.n, v_begin + a.vpr) : a.n;
  const int64_t ntile = (v_end - v_begin + 31) / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vl = lane & 31, hh = lane >> 5;

  // Two-stage prefetch: the packed row of the next tile is loaded while this tile is decoded,
  // and with a slot gather the slot index is read one tile earlier still.
  const int64_t wstride = (int64_t)gridDim.x * kDecWaves;
  auto row_of = [&](int64_t tl) -> int64_t {
    const int64_t v = v_begin + tl * 32 + vl;
    if (tl >= ntile || v >= v_end) return -1;
    return a.slot ? a.slot[v] : v;
  };
  auto fetch = [&](int64_t row, uint32_t (&cw)[Geo::CHUNK_DW], float& nrm) {
    if (row >= 0) {
      const uint8_t* src = a.packed + row * Geo::ROW + hh * Geo::CHUNK;
      if constexpr (Geo::G == 16) {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; w += 4) {
          u32x4 q = *(const u32x4*)(src + 4 * w);
          cw[w] = q[0]; cw[w + 1] = q[1]; cw[w + 2] = q[2]; cw[w + 3] = q[3];
        }
      } else if constexpr (Geo::G == 8) {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; w += 2) {
          u32x2 q = *(const u32x2*)(src + 4 * w);
          cw[w] = q[0]; cw[w + 1] = q[1];
        }
      } else {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; ++w) cw[w] = *(const uint32_t*)(src + 4 * w);
      }
      nrm = a.norms[row];
    } else {
#pragma unroll
      for (int w = 0; w < Geo::CHUNK_DW; ++w) cw[w] = 0u;
      nrm = 0.f;
    }
  };
  int64_t tile = (int64_t)blockIdx.x * kDecWaves + wave;
  uint32_t cwn[Geo::CHUNK_DW];
  float nrmn;
  fetch(row_of(tile), cwn, nrmn);
  int64_t row_nn = row_of(tile + wstride);

  for (; tile < ntile; tile += wstride) {
    const int64_t vec = v_begin + tile * 32 + vl;
    const bool valid = vec < v_end;
    uint32_t cw[Geo::CHUNK_DW];
#pragma unroll
    for (int w = 0; w < Geo::CHUNK_DW; ++w) cw[w] = cwn[w];
    const float nrm = nrmn;
    fetch(row_nn, cwn, nrmn);
    row_nn = row_of(tile + 2 * wstride);

    // ---- codes -> fp16 centroids, 8 per K block
    u32x4 bfrag[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t h2[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int pos = (8 * kb + 2 * c + s) * BITS;
          uint32_t code = (cw[pos >> 5] >> (pos & 31));
          if ((pos & 31) + BITS > 32) code |= cw[(pos >> 5) + 1] << (32 - (pos & 31));
          h2[s] = ctab[code & MASK];
        }
        bfrag[kb][c] = h2[0] | (h2[1] << 16);
      }
    }

    // ---- inverse rotation and store (an opaque offset keeps the Pi^T tiles in LDS instead of
    //      letting the compiler hoist all of them into registers)
    uint32_t aoff = (uint32_t)lane * 16u;
    asm volatile("" : "+v"(aoff));
    const bool store = valid;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = mfma32_f16(*(const u32x4*)((const char*)smem + aoff + (t * KB + kb) * 1024), bfrag[kb], acc);
      if (store) {
        const int64_t base = vec * D + hh * HALF + 16 * t;
        if constexpr (OUT == TQ_F32) {
          float* o = (float*)a.out + base;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(f32x4*)(o + 4 * q4) =
                f32x4{acc[4 * q4] * nrm, acc[4 * q4 + 1] * nrm, acc[4 * q4 + 2] * nrm, acc[4 * q4 + 3] * nrm};
        } else {
          uint32_t w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float lo = acc[2 * j] * nrm, hi = acc[2 * j + 1] * nrm;
            w[j] = OUT == TQ_BF16 ? pack_bf16x2(lo, hi) : pack_f16x2(lo, hi);
          }
          uint16_t* o = (uint16_t*)a.out + base;
          *(u32x4*)o = u32x4{w[0], w[1], w[2], w[3]};
          *(u32x4*)(o + 8) = u32x4{w[4], w[5], w[6], w[7]};
        }
      }
    }
  }
}

template <int D, int BITS, int OUT>
static hipError_t launch_decode_t(const DecodeLaunch& L) {
  using Geo = DecGeo<D, BITS>;
  DecodeKArgs k;
  k.frag = (const u32x4*)L.rot->dec(0);
  k.frag_stride = (int64_t)(L.rot->dec_stride / sizeof(u32x4));
  k.packed = L.packed;
  k.norms = L.norms;
  k.slot = L.slot_mapping;
  k.out = L.out;
  k.n = L.n;
  k.vpr = L.vectors_per_rot;
  for (int j = 0; j < 8; ++j)
    k.ctab[j] = (uint32_t)L.lv.centroid_f16[2 * j] | ((uint32_t)L.lv.centroid_f16[2 * j + 1] << 16);
  const int64_t per_rot = L.vectors_per_rot ? L.vectors_per_rot : L.n;
  const int nrot = L.vectors_per_rot ? (int)((L.n + L.vectors_per_rot - 1) / L.vectors_per_rot) : 1;
  const int64_t tiles = (per_rot + 31) / 32;
  const size_t lds = Geo::FRAG_U4 * sizeof(u32x4);
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<D, BITS, OUT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int cu = device_cu_count(L.rot->device);
  // workgroups per CU: LDS-limited at d=256 (128 KiB of tiles), else up to 3 (24 waves)
  int per_cu = (int)((160 * 1024 - 256) / lds);
  per_cu = per_cu < 1 ? 1 : (per_cu > 3 ? 3 : per_cu);
  const int64_t want = (int64_t)cu * per_cu;
  int64_t bx = (want + nrot - 1) / nrot;
  const int64_t need = (tiles + kDecWaves - 1) / kDecWaves;
  if (bx > need) bx = need;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL((decode_kernel<D, BITS, OUT>), dim3((unsigned)bx, (unsigned)nrot), dim3(kDecWaves * 64), lds,
                     L.stream, k);
  return hipGetLastError();
}

template <int D, int BITS>
static hipError_t dec_out(const DecodeLaunch& L) {
  switch (L.out_dtype) {
    case TQ_F32: return launch_decode_t<D, BITS, TQ_F32>(L);
    case TQ_BF16: return launch_decode_t<D, BITS, TQ_BF16>(L);
    default: return launch_decode_t<D, BITS, TQ_F16>(L);
  }
}

template <int D>
static hipError_t dec_bits(const DecodeLaunch& L) {
  switch (L.bits) {
    case 2: return dec_out<D, 2>(L);
    case 3: return dec_out<D, 3>(L);
    default: return dec_out<D, 4>(L);
  }
}

hipError_t launch_decode(const DecodeLaunch& L) {
  switch (L.rot->d) {
    case 64: return dec_bits<64>(L);
    case 128: return dec_bits<128>(L);
    default: return dec_bits<256>(L);
  }
}

}  // namespace tq
