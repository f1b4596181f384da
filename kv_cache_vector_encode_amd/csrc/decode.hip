// Decode kernel: unpack, centroid lookup, inverse rotation and norm scaling.
//
// Method (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv, TurboQuantCompressorMSE
// .decompress): x_hat = (c[idx] Pi) * n, cast to the output dtype.
//
// Layout mirrors the encode: a wave owns 32 vectors; lane (v, hh) reads the packed chunk
// of rotated coordinates hh*d/2 .. +d/2 of vector v, turns 8 codes at a time into an fp16
// MFMA B operand, and one 32x32x16 fp16 MFMA per (output tile, K block) against prebuilt
// tiles of Pi^T (resident in LDS) leaves output coordinates hh*d/2 + 16t + i in accumulator
// register i, which are scaled by n, staged in LDS and stored with the wave's other rows as
// one contiguous block. fp16 operands (2^-11 relative)
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
  const uint8_t* zero;   // zeros that masked lanes load (>= one packed chunk)
  uint8_t* sink;         // where masked lanes store (>= 64 lanes x 16 bytes)
  int64_t n, vpr;
  uint32_t ctab[8];   // 16 fp16 centroids, two per word
};

// Four waves per workgroup, two workgroups per CU (one where LDS allows only one: float32
// outputs at d = 128, every output type at d = 256). The decode is bound by its output
// stores; HBM write throughput drops when many waves keep scattered stores in flight, so each
// wave stages its 32 output rows in LDS and writes them as one contiguous block, 1 KiB per
// store instruction, and latency within a wave is hidden by computing two output tiles at a
// time.
constexpr int kDecWaves = 4;
constexpr int kDecWgPerCu = 2;

template <int D, int BITS>
struct DecGeo {
  static constexpr int T = D / 32, KB = D / 16, HALF = D / 2;
  static constexpr int ROW = D * BITS / 8;
  static constexpr int CHUNK = HALF * BITS / 8;
  static constexpr int CHUNK_DW = CHUNK / 4;
  static constexpr int G = (CHUNK % 16 == 0 && ROW % 16 == 0) ? 16 : ((CHUNK % 8 == 0 && ROW % 8 == 0) ? 8 : 4);
  static constexpr int FRAG_U4 = T * KB * 64;
  // Code -> centroid table: 2-bit codes go four at a time (one byte -> four fp16), 3- and 4-bit
  // codes two at a time (6 or 8 bits -> two fp16).
  static constexpr int PER_LOOKUP = BITS == 2 ? 4 : 2;
  static constexpr int TAB_N = 1 << (PER_LOOKUP * BITS);
  static constexpr int TAB_WORDS = TAB_N * PER_LOOKUP / 2;
  // Outputs are staged through LDS so that a wave's 32 output rows, one contiguous block, go
  // out as 1 KiB per store instruction (d <= 128; at d=256 the Pi^T tiles fill LDS and lanes
  // store their own 16-byte pieces).
  static constexpr bool STAGE = D <= 128;
  static constexpr size_t stage_bytes(int out_elem) { return STAGE ? (size_t)32 * D * out_elem : 0; }
  static constexpr size_t lds_bytes(int out_elem) {
    return (size_t)FRAG_U4 * 16 + (size_t)kDecWaves * stage_bytes(out_elem);
  }
};


template <int D, int BITS, int OUT, bool SLOT>
__global__ void __launch_bounds__(kDecWaves * 64) decode_kernel(DecodeKArgs a) {
  using Geo = DecGeo<D, BITS>;
  constexpr int T = Geo::T, KB = Geo::KB, HALF = Geo::HALF;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  extern __shared__ u32x4 smem[];
  __shared__ uint32_t tab[Geo::TAB_WORDS];

  const int r = blockIdx.y;
  const u32x4* gfrag = a.frag + (int64_t)r * a.frag_stride;

  const int64_t v_begin = a.vpr ? (int64_t)r * a.vpr : 0;
  const int64_t v_end = a.vpr ? min(a.n, v_begin + a.vpr) : a.n;
  const int64_t ntile = (v_end - v_begin + 31) / 32;
  if (ntile <= 0) return;   // uniform per workgroup: no thread is left at the barrier below
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vl = lane & 31, hh = lane >> 5;
  constexpr int OE = OUT == TQ_F32 ? 4 : 2;
  uint8_t* stg = (uint8_t*)(smem + Geo::FRAG_U4) + wave * Geo::stage_bytes(OE);

  // Two-stage prefetch: the packed row of the next tile is loaded while this tile is decoded,
  // and with a slot gather the slot index is read one tile earlier still. Every load and store
  // is issued unconditionally (masked lanes read the zero page and write the sink): the memory
  // counter is in order, and a branch around an access would make the wait for a prefetched
  // load also wait for the stores issued after it.
  const int64_t wstride = (int64_t)gridDim.x * kDecWaves;
  auto row_of = [&](int64_t tl) -> int64_t {
    const int64_t v = v_begin + tl * 32 + vl;
    const bool ok = tl < ntile && v < v_end;
    if constexpr (SLOT) {
      const int64_t s = a.slot[ok ? v : v_begin];
      return ok ? s : -1;
    } else {
      return ok ? v : -1;
    }
  };
  auto fetch = [&](int64_t row, uint32_t (&cw)[Geo::CHUNK_DW], float& nrm) {
    {
      const uint8_t* src = row >= 0 ? a.packed + row * Geo::ROW + hh * Geo::CHUNK : a.zero;
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
      nrm = *(row >= 0 ? a.norms + row : (const float*)a.zero);
    }
  };
  int64_t tile = (int64_t)blockIdx.x * kDecWaves + wave;
  uint32_t cwn[Geo::CHUNK_DW];
  float nrmn;
  // the first tile's loads are issued before the table copies below, so the two latencies overlap
  fetch(row_of(tile), cwn, nrmn);
  int64_t row_nn = row_of(tile + wstride);

  for (int i = threadIdx.x; i < Geo::FRAG_U4; i += blockDim.x) smem[i] = gfrag[i];
  {
    // centroids straight from the kernel-argument segment (indexing the by-value copy with a
    // lane-dependent index would go through scratch)
    const uint32_t* kc = (const uint32_t*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() +
                                           offsetof(DecodeKArgs, ctab));
    auto cent = [&](uint32_t k) -> uint32_t { return (kc[k >> 1] >> (16 * (k & 1))) & 0xffffu; };
    for (int j = threadIdx.x; j < Geo::TAB_N; j += blockDim.x) {
      if constexpr (Geo::PER_LOOKUP == 4) {
        tab[2 * j] = cent(j & MASK) | (cent((j >> BITS) & MASK) << 16);
        tab[2 * j + 1] = cent((j >> (2 * BITS)) & MASK) | (cent(j >> (3 * BITS)) << 16);
      } else {
        tab[j] = cent(j & MASK) | (cent(j >> BITS) << 16);
      }
    }
  }
  __syncthreads();
  wait_vmem_all();

  for (; tile < ntile; tile += wstride) {
    const int64_t vbase = v_begin + tile * 32;
    const int64_t vec = vbase + vl;
    uint32_t cw[Geo::CHUNK_DW];
#pragma unroll
    for (int w = 0; w < Geo::CHUNK_DW; ++w) cw[w] = cwn[w];
    const float nrm = nrmn;
    fetch(row_nn, cwn, nrmn);
    row_nn = row_of(tile + 2 * wstride);

    // ---- codes -> fp16 centroids, 8 per K block (the lane's codes 8kb .. 8kb+7)
    u32x4 bfrag[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (BITS == 2) {
        // 8 codes = 16 bits = two table bytes, four fp16 each
        const uint32_t bits16 = cw[kb >> 1] >> (16 * (kb & 1));
        const u32x2 q0 = *(const u32x2*)&tab[2 * (bits16 & 255u)];
        const u32x2 q1 = *(const u32x2*)&tab[2 * ((bits16 >> 8) & 255u)];
        bfrag[kb] = u32x4{q0[0], q0[1], q1[0], q1[1]};
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          constexpr int PB = 2 * BITS;           // bits per code pair
          const int pos = (4 * kb + c) * PB;     // compile-time after unrolling
          uint32_t idx;
          if ((pos & 31) + PB <= 32)
            idx = cw[pos >> 5] >> (pos & 31);
          else
            idx = funnel(cw[(pos >> 5) + 1], cw[pos >> 5], pos & 31);
          bfrag[kb][c] = tab[idx & ((1u << PB) - 1u)];
        }
      }
    }

    // ---- inverse rotation (an opaque offset keeps the Pi^T tiles in LDS instead of letting
    //      the compiler hoist all of them into registers)
    uint32_t aoff = (uint32_t)lane * 16u;
    asm volatile("" : "+v"(aoff));
    constexpr int E = OUT == TQ_F32 ? 4 : 2;   // output bytes per element
    constexpr int CPT = E;                     // 16-byte chunks per lane per tile (16 outputs)
    constexpr int S = 4 / CPT;                 // tiles per 64-byte run of one half vector
    f32x16 accp[2];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (t % 2 == 0) {
        // two independent accumulation chains in flight
        accp[0] = f32x16{};
        accp[1] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          accp[0] = mfma32_f16(*(const u32x4*)((const char*)smem + aoff + (t * KB + kb) * 1024), bfrag[kb], accp[0]);
          accp[1] = mfma32_f16(*(const u32x4*)((const char*)smem + aoff + ((t + 1) * KB + kb) * 1024), bfrag[kb],
                               accp[1]);
        }
      }
      const f32x16 acc = accp[t % 2];
      // scaled outputs of coordinates hh*d/2 + 16t .. +16 as CPT 16-byte chunks
      u32x4 ch[CPT];
      if constexpr (OUT == TQ_F32) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          ch[q4] = u32x4{__float_as_uint(acc[4 * q4] * nrm), __float_as_uint(acc[4 * q4 + 1] * nrm),
                         __float_as_uint(acc[4 * q4 + 2] * nrm), __float_as_uint(acc[4 * q4 + 3] * nrm)};
      } else {
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float lo = acc[2 * j] * nrm, hi = acc[2 * j + 1] * nrm;
          w[j] = OUT == TQ_BF16 ? pack_bf16x2(lo, hi) : pack_f16x2(lo, hi);
        }
        ch[0] = u32x4{w[0], w[1], w[2], w[3]};
        ch[1] = u32x4{w[4], w[5], w[6], w[7]};
      }
      if constexpr (Geo::STAGE) {
        // staged in row-major order (row v = the wave's vector v), 16-byte chunks XOR-swizzled
        // within a row by the row index so that the 32 rows written together spread over banks
        constexpr uint32_t RC = D * E / 16;                  // 16-byte chunks per output row
        constexpr uint32_t SW = RC >= 16 ? 15u : RC - 1u;
        const uint32_t c0 = hh * (HALF * E / 16) + t * CPT;
#pragma unroll
        for (int k = 0; k < CPT; ++k)
          *(u32x4*)(stg + 16 * (vl * RC + ((c0 + k) ^ (vl & SW)))) = ch[k];
      } else {
        uint8_t* dst = vec < v_end ? (uint8_t*)a.out + (vec * D + hh * HALF + 16 * t) * E : a.sink + 64 * lane;
        // (ordinary stores: non-temporal 16-byte pieces of a line measured 10x slower)
#pragma unroll
        for (int k = 0; k < CPT; ++k) *(u32x4*)(dst + 16 * k) = ch[k];
      }
    }
    if constexpr (Geo::STAGE) {
      // the tile's 32 output rows are one contiguous block: 1 KiB per store instruction
      constexpr uint32_t RB = D * E, RC = RB / 16;
      constexpr uint32_t SW = RC >= 16 ? 15u : RC - 1u;
      uint8_t* tbase = (uint8_t*)a.out + vbase * RB;
#pragma unroll
      for (uint32_t j = 0; j < 32 * RB / 1024; ++j) {
        const uint32_t off = 1024u * j + 16u * lane;
        const uint32_t rowi = off / RB, c = (off % RB) / 16;
        const u32x4 q = *(const u32x4*)(stg + 16 * (rowi * RC + (c ^ (rowi & SW))));
        uint8_t* dst = vbase + rowi < v_end ? tbase + off : a.sink + 16 * lane;
        // non-temporal: the decoded stream is far larger than the caches, and left in them as
        // dirty lines it is written back during whatever kernel runs next
        __builtin_nontemporal_store(q, (u32x4*)dst);
      }
    }
  }
}

template <int D, int BITS, int OUT, bool SLOT>
static hipError_t launch_decode_t(const DecodeLaunch& L) {
  using Geo = DecGeo<D, BITS>;
  DecodeKArgs k;
  k.frag = (const u32x4*)L.rot->dec(0);
  k.frag_stride = (int64_t)(L.rot->dec_stride / sizeof(u32x4));
  k.packed = L.packed;
  k.norms = L.norms;
  k.slot = L.slot_mapping;
  k.out = L.out;
  k.zero = L.rot->zero();
  k.sink = L.rot->sink();
  k.n = L.n;
  k.vpr = L.vectors_per_rot;
  for (int j = 0; j < 8; ++j)
    k.ctab[j] = (uint32_t)L.lv.centroid_f16[2 * j] | ((uint32_t)L.lv.centroid_f16[2 * j + 1] << 16);
  const int64_t per_rot = L.vectors_per_rot ? L.vectors_per_rot : L.n;
  const int nrot = L.vectors_per_rot ? (int)((L.n + L.vectors_per_rot - 1) / L.vectors_per_rot) : 1;
  const int64_t tiles = (per_rot + 31) / 32;
  const size_t lds = Geo::lds_bytes(OUT == TQ_F32 ? 4 : 2);
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<D, BITS, OUT, SLOT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int cu = device_cu_count(L.rot->device);
  const int64_t want = (int64_t)cu * kDecWgPerCu;
  int64_t bx = (want + nrot - 1) / nrot;
  const int64_t need = (tiles + kDecWaves - 1) / kDecWaves;
  if (bx > need) bx = need;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL((decode_kernel<D, BITS, OUT, SLOT>), dim3((unsigned)bx, (unsigned)nrot), dim3(kDecWaves * 64), lds,
                     L.stream, k);
  return hipGetLastError();
}

template <int D, int BITS, int OUT>
static hipError_t dec_slot(const DecodeLaunch& L) {
  return L.slot_mapping ? launch_decode_t<D, BITS, OUT, true>(L) : launch_decode_t<D, BITS, OUT, false>(L);
}

template <int D, int BITS>
static hipError_t dec_out(const DecodeLaunch& L) {
  switch (L.out_dtype) {
    case TQ_F32: return dec_slot<D, BITS, TQ_F32>(L);
    case TQ_BF16: return dec_slot<D, BITS, TQ_BF16>(L);
    default: return dec_slot<D, BITS, TQ_F16>(L);
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
