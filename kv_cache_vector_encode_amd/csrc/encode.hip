// Encode kernel: norm, rotation, Lloyd-Max quantization and LSB-first packing in one pass.
//
// Method (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv, TurboQuantCompressorMSE
// .compress): n = ||x||; y = Pi x / (n + 1e-8); code_i = nearest centroid of y_i; store n
// and the packed codes. Packing is the LSB-first bitstream of the same page's value packing
// (quantize_value_chunk) at a dense (d*b + 7)//8 bytes per vector (value_formula_nbytes).
//
// Layout of the work. A wave owns 32 vectors. The rotation is one 32x32x16 bf16 MFMA per
// (output tile t of 32 coordinates, K block kb of 16 inputs, pass): the B operand is the
// vectors' raw inputs (lane v + 32*hh holds inputs 16kb + 8hh .. +7 of vector v, so lanes v and
// v + 32 read the two halves of each 32-byte piece of the row: half as many cache lines per
// load instruction as d/2 contiguous inputs per lane, and measurably faster to stream), the A
// operand is a prebuilt tile of Pi whose columns follow that order and whose row order makes
// lane (v, hh) end up holding rotated coordinates hh*d/2 + 16t + i in accumulator register i. A lane therefore owns d/2 consecutive output coordinates of one
// vector, which pack into whole bytes (d/2 * b bits is a multiple of 8) with no cross-lane
// traffic, and are written with wide stores.
//
// Precision: a code must match the float64 definition except within 1e-5 of a decision
// boundary. One bf16 pass perturbs y by ~1e-4, so Pi is split into bf16 hi + lo (16
// significant bits, error ~1e-6): bf16 inputs are exact and take 2 passes; float32 and
// float16 inputs are split too and take 3 (Pi_hi x_hi + Pi_lo x_hi + Pi_hi x_lo).
//
// Quantization: one FMA maps the unnormalized Pi x to f = y * s + o in [1, 2) (y = Pi x /
// (n + 1e-8), the per-vector factor s / (n + 1e-8) computed once), and a 128-bin LDS table
// indexed by the top 7 fraction bits of f, whose bins each hold at most one decision boundary,
// gives the code base + (f > boundary) = #{k : t_k < y} as the top bits of bits(f) - entry:
// all f share one exponent, so the compare is an integer subtraction whose carry adds to the
// base stored above it. Byte 2 of bits(f) is the exponent's low bit and those 7 fraction bits,
// so one byte-select shift (SDWA) makes the table address. 2- and 3-bit codes sit in the top b
// bits and one funnel shift appends each to the packed word (4 VALU instructions per
// coordinate: fma, shift, subtract, funnel shift); 4-bit codes sit in byte 3 and a pair goes
// into its byte with two byte-select instructions. A compare chain over the 2^b - 1 boundaries
// costs 15-20.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {

struct EncodeKArgs {
  const u32x4* frag;       // rotation tiles (u32x4 units), rotation r at frag + r * frag_stride
  int64_t frag_stride;
  const void* x;
  int64_t x_row_stride;    // elements
  uint8_t* packed;
  float* norms;
  const int64_t* slot;
  uint8_t* sink;           // where masked lanes store (>= 64 x 64 bytes of codes + 64 norms)
  int64_t n, vpr;
  float lut_scale, lut_off;
  int32_t norm_correct;    // store n / ||c[idx]|| instead of n
  uint32_t lut[kLutBins];
  float csq[kMaxLevels];   // c_k^2, for the norm correction
};


template <int D, int BITS, int QS = 1>
struct EncGeo {
  static constexpr int T = D / 32;                 // output tiles
  static constexpr int KB = D / 16;                // K blocks
  static constexpr int HALF = D / 2;               // coordinates per lane
  static constexpr int TS = T / QS;                // output tiles per workgroup slice
  static constexpr int ROW = D * BITS / 8;         // packed bytes per vector
  static constexpr int CHUNK = HALF * BITS / 8;    // packed bytes per lane (its half of the row)
  static constexpr int CHUNK_S = CHUNK / QS;       // of those, the bytes of this slice
  static constexpr int CHUNK_DW = CHUNK_S / 4;
  static constexpr int G = (CHUNK_S % 16 == 0 && ROW % 16 == 0) ? 16 : ((CHUNK_S % 8 == 0 && ROW % 8 == 0) ? 8 : 4);
  static constexpr int SET_U4 = TS * KB * 64;      // one slice's tiles of one pass, u32x4 per lane
  static constexpr int FRAG_U4 = 2 * SET_U4;       // hi and lo tiles of the slice
  static constexpr bool LDS = (D <= 128) || QS > 1;
  // Occupancy plan: at d <= 128, two workgroups per CU (2 x 64 KiB of Pi tiles in LDS): bf16
  // inputs at d = 128 in 12-wave workgroups without an input prefetch (6 waves per SIMD within
  // 80 VGPRs); d = 64, and float32 / fp16 inputs, which are split in registers, in 8-wave ones
  // (4 per SIMD within 128; at d = 64 the prefetch measured 7% faster than more waves); d=256 needs up to 256 VGPRs, so one 8-wave workgroup (2 waves per SIMD), holding half of
  // Pi's output rows (128 KiB) when split in two slices, else reading Pi from L2.
  static constexpr int WG_PER_CU = D == 256 ? 1 : 2;
};
// Byte B of `word` = (byte 3 of lo) | (byte 3 of hi) << 4; for B > 0 the other bytes are kept,
// for B = 0 (written first) bytes 1-3 are cleared: two SDWA instructions (byte-select sources,
// byte-select destination), where shifting each code out of byte 3 and or-ing it into place
// takes four. The codes are < 16, so each byte 3 is one nibble.
template <int B>
__device__ __forceinline__ uint32_t nibble_pair_to_byte(uint32_t word, uint32_t lo, uint32_t hi) {
  uint32_t t;
  asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
      : "=v"(t) : "v"(hi));
  if constexpr (B == 0)
    asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
        : "=v"(word) : "v"(lo), "v"(t));
  else if constexpr (B == 1)
    asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3 src1_sel:DWORD"
        : "+v"(word) : "v"(lo), "v"(t));
  else if constexpr (B == 2)
    asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3 src1_sel:DWORD"
        : "+v"(word) : "v"(lo), "v"(t));
  else
    asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3 src1_sel:DWORD"
        : "+v"(word) : "v"(lo), "v"(t));
  return word;
}

// (byte 2 of f) * 4: the LDS byte address of its table entry (the table at address 0)
__device__ __forceinline__ uint32_t lut_addr(uint32_t f) {
  uint32_t r;
  asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
      : "=v"(r) : "v"(f));
  return r;
}
// bf16 inputs at d = 128 take more waves instead of a prefetch (see the occupancy plan)
template <int D, int IN>
constexpr bool enc_many_waves() { return D == 128 && IN == TQ_BF16; }
template <int D, int IN>
constexpr int enc_waves() { return enc_many_waves<D, IN>() ? 12 : 8; }
template <int D, int IN>
constexpr int enc_wpe() { return D == 256 ? 2 : (enc_many_waves<D, IN>() ? 6 : 4); }

// QS > 1 (d = 256): QS workgroups share each group of vectors, each computing the output tiles of
// one slice of the coordinates with that slice's rows of Pi in LDS (the dense Pi, 256 KiB as hi +
// lo, does not fit). The QS workgroups of a group are numbered 8 apart, which places them on one
// XCD, so the repeated reads of each input row hit that XCD's L2. The slice q = 0 stores the norm.
template <int D, int BITS, int IN, bool SLOT, int QS>
__global__ void __launch_bounds__((enc_waves<D, IN>() * 64))
__attribute__((amdgpu_waves_per_eu(enc_wpe<D, IN>())))
encode_kernel(EncodeKArgs a) {
  using Geo = EncGeo<D, BITS, QS>;
  constexpr int T = Geo::TS, KB = Geo::KB, HALF = Geo::HALF;
  constexpr bool SPLIT_X = (IN != TQ_BF16);
  constexpr int WAVES = enc_waves<D, IN>();
  extern __shared__ u32x4 smem[];
  // entries at words 128 .. 255 (byte 2 of an f in [1, 2) is 128 + its bin); words 0 .. 127
  // repeat them for inputs that are not finite
  __shared__ uint32_t lut[2 * kLutBins];
  __shared__ float csq[kMaxLevels];

  const int r = blockIdx.y;
  // slice q and vector-group slot of this workgroup (the slices of one slot are 8 apart)
  const int wg = blockIdx.x;
  const int q = QS == 1 ? 0 : (wg >> 3) % QS;
  const int slot_id = QS == 1 ? wg : (wg & 7) + 8 * (wg / (8 * QS));
  const int nslots = gridDim.x / QS;
  const u32x4* gfrag = a.frag + (int64_t)r * a.frag_stride;

  const int64_t v_begin = a.vpr ? (int64_t)r * a.vpr : 0;
  const int64_t v_end = a.vpr ? min(a.n, v_begin + a.vpr) : a.n;
  const int64_t ntile = (v_end - v_begin + 31) / 32;
  if (ntile <= 0) return;   // uniform per workgroup: no thread is left at the barrier below
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vl = lane & 31, hh = lane >> 5;

  // Raw inputs of one tile: lane (v, hh) reads elements 16kb + 8hh .. +7 with 16-byte loads.
  // bf16 inputs are the MFMA B operands as loaded. At d = 64 and 256 they are prefetched one
  // tile ahead, so every wave keeps a tile of loads in flight while it rotates and quantizes the
  // previous one; at d = 128 the 32 registers of a prefetch buy more: without it a SIMD holds
  // 6 waves instead of 4, which hides the load latency better (measured ~8% faster).
  // Every load and store is issued unconditionally (masked lanes read row v_begin and write
  // the sink): the memory counter is in order, and a branch around an access would make the
  // wait for a prefetched load also wait for the stores issued after it.
  constexpr int ELEM = IN == TQ_F32 ? 4 : 2;
  constexpr int NRAW = HALF * ELEM / 16;
  constexpr int PER = ELEM / 2;          // 16-byte loads per K block
  constexpr bool PREFETCH = IN == TQ_BF16 && !enc_many_waves<D, IN>();
  const int64_t wstride = (int64_t)nslots * WAVES;
  // loads tile tl's inputs and returns the packed row its codes go to (-1: none)
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
  // Tiles go to waves wave-major (tile = wave * nslots + slot, then every wstride): when the
  // tiles do not divide evenly, the waves with one more are the low-numbered waves of every
  // workgroup, so the last round keeps every CU and SIMD busy rather than a subset of workgroups
  int64_t tile = (int64_t)wave * nslots + slot_id;
  u32x4 xr[NRAW];
  int64_t rown = -1;
  // the first tile's loads are issued before the table copies below, so the two latencies overlap
  if (PREFETCH) rown = fetch(tile, xr);

  if constexpr (Geo::LDS) {
    // the slice's tiles of each pass: tiles (pass, t, kb) are stored pass-major, then t, then kb
    for (int i = threadIdx.x; i < Geo::FRAG_U4; i += blockDim.x) {
      const int pass = i / Geo::SET_U4, k = i - pass * Geo::SET_U4;
      smem[i] = gfrag[(pass * QS + q) * Geo::SET_U4 + k];
    }
  }
  {
    // read the table straight from the kernel-argument segment (the only argument is `a`, at
    // offset 0): indexing the by-value copy would spill the whole struct to scratch
    const uint32_t* klut = (const uint32_t*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() +
                                             offsetof(EncodeKArgs, lut));
    for (int i = threadIdx.x; i < 2 * kLutBins; i += blockDim.x) lut[i] = klut[i & (kLutBins - 1)];
    const float* kcsq = (const float*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() +
                                       offsetof(EncodeKArgs, csq));
    if (threadIdx.x < kMaxLevels) csq[threadIdx.x] = kcsq[threadIdx.x];
  }
  __syncthreads();
  if (PREFETCH) wait_vmem_all();
  // Tile reads go through an offset the compiler cannot prove loop-invariant; otherwise it
  // hoists every tile of Pi into registers and spills.
  const char* abase = Geo::LDS ? (const char*)smem : (const char*)gfrag;

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
      if constexpr (IN == TQ_BF16) {
#pragma unroll
        for (int k = 0; k < NRAW; ++k) xh[k] = xr[k];
      }
    }

    // ---- norm, and the MFMA B operands (bf16 hi, and lo for split inputs)
    float ss0 = 0.f, ss1 = 0.f;
    if constexpr (IN == TQ_BF16) {
      // sum of squares two elements per instruction (bf16 products are exact in fp32)
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
    ss += wave_xor(ss, 32);            // the other half of the same vector
    const float nrm = sqrtf(ss);
    // f = y * lut_scale + lut_off with y = z / (n + 1e-8): one FMA per coordinate
    const float fs = a.lut_scale / (nrm + 1e-8f);
    const float foff = a.lut_off;

    // ---- rotate tile by tile, quantize, pack into this lane's chunk
    uint32_t aoff = (uint32_t)lane * 16u;
    asm volatile("" : "+v"(aoff));
    uint32_t pk[Geo::CHUNK_DW];
#pragma unroll
    for (int w = 0; w < Geo::CHUNK_DW; ++w) pk[w] = 0u;
    uint32_t wprev = 0u;
    // 2- and 3-bit codes (table entries with the code in the top BITS bits): the lane's codes are
    // taken from its last coordinate down to its first and each is appended to `chain` by one
    // funnel shift, chain = (chain << BITS) | code; after code j, chain holds stream bits
    // [BITS*j, BITS*j + 32). A word whose first bit is code j's first bit is the chain itself; a
    // word that begins inside code j is (chain << r) | (the top r bits of code j) taken before
    // code j goes in (r = the code's bits in that word): one more funnel shift.
    constexpr bool CHAIN = BITS < 4;
    uint32_t chain = 0u;
    // tile t and coordinate i as compile-time constants: the packing's shift counts are
    // instruction immediates
    static_for<0, T>([&](auto tc) {
      constexpr int t = CHAIN ? T - 1 - decltype(tc)::value : decltype(tc)::value;
      // a fresh opaque offset per tile: the scheduler cannot pull later tiles' Pi reads ahead
      // (all 4 tiles' operands at once would not fit in registers)
      asm volatile("" : "+v"(aoff));
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // Pi tiles read from L2 (d=256) are fenced in groups of 4 K blocks for the same reason
        if (!Geo::LDS && kb % 4 == 0 && kb > 0) asm volatile("" : "+v"(aoff));
        const u32x4 ahi = *(const u32x4*)(abase + aoff + ((0 * T + t) * KB + kb) * 1024);
        const u32x4 alo = *(const u32x4*)(abase + aoff + ((1 * T + t) * KB + kb) * 1024);
        acc = mfma32_bf16(ahi, xh[kb], acc);
        acc = mfma32_bf16(alo, xh[kb], acc);
        if constexpr (SPLIT_X) acc = mfma32_bf16(ahi, xl[kb], acc);
      }
      static_for<0, 16>([&](auto ic) {
        constexpr int i = CHAIN ? 15 - decltype(ic)::value : decltype(ic)::value;
        const uint32_t fb = __float_as_uint(fmaf(acc[i], fs, foff));
        // code: byte 3 (4 bits), the top BITS bits (2 and 3 bits)
        const uint32_t w = fb - *(const uint32_t*)((const char*)lut + lut_addr(fb));
        constexpr int pos = (16 * t + i) * BITS;
        if constexpr (CHAIN) {
          if constexpr ((pos & 31) + BITS > 32) {
            constexpr int r = (pos & 31) + BITS - 32;
            pk[(pos >> 5) + 1] = __builtin_amdgcn_alignbit(chain, w, 32 - r);
          }
          chain = __builtin_amdgcn_alignbit(chain, w, 32 - BITS);
          if constexpr ((pos & 31) == 0) pk[pos >> 5] = chain;
        } else if constexpr (BITS == 4) {
          // two codes per byte: byte 3 of the odd coordinate's w goes to the high nibble and the
          // even one's to the low nibble, written straight into byte (i % 8) / 2 of the word
          if (i & 1) {
            uint32_t& word = pk[pos >> 5];
            switch ((i & 7) >> 1) {
              case 0: word = nibble_pair_to_byte<0>(word, wprev, w); break;
              case 1: word = nibble_pair_to_byte<1>(word, wprev, w); break;
              case 2: word = nibble_pair_to_byte<2>(word, wprev, w); break;
              default: word = nibble_pair_to_byte<3>(word, wprev, w); break;
            }
          }
          wprev = w;
        }
        // table reads in groups of 8: all 16 in flight at once would not fit in registers
        if constexpr ((decltype(ic)::value & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      });
      // finish this tile's packed words here: left alone, the compiler sinks the packing to the
      // store and keeps every table entry of the vector live until then
#pragma unroll
      for (int w = (16 * t * BITS) >> 5; w <= ((16 * t + 16) * BITS - 1) >> 5; ++w)
        asm volatile("" : "+v"(pk[w]));
      if constexpr (CHAIN) asm volatile("" : "+v"(chain));
    });

    // ---- norm correction (Turbo Attention page, "The codec", Norms row: the decoded key keeps
    //      the input's length): store n / ||c[idx]||, ||c[idx]||^2 summed over this lane's codes
    //      and the other half of the vector
    float nst = nrm;
    if constexpr (QS == 1) {
      if (a.norm_correct) {
        float cs0 = 0.f, cs1 = 0.f;
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
          const int pos = j * BITS;
          uint32_t code = pk[pos >> 5] >> (pos & 31);
          if ((pos & 31) + BITS > 32) code |= pk[(pos >> 5) + 1] << (32 - (pos & 31));
          const float c2 = csq[code & ((1u << BITS) - 1u)];
          if (j & 1)
            cs1 += c2;
          else
            cs0 += c2;
        }
        float cs = cs0 + cs1;
        cs += wave_xor(cs, 32);
        nst = nrm / sqrtf(cs);
      }
    }

    // ---- store: dense rows of one slice non-temporally (a wave's 32 rows are one contiguous
    //      run); slot-mapped rows, and the half rows of the d = 256 slices, with ordinary stores:
    //      a paged pool puts the KV heads of one token in different pages, and a slice writes
    //      every other half row, so those pieces stand alone in their cache lines until the
    //      cache combines them with their neighbours
    auto put = [&](auto v, auto* p) {
      if constexpr (SLOT || QS > 1)
        *p = v;
      else
        __builtin_nontemporal_store(v, p);
    };
    {
      const bool ok = row >= 0;
      uint8_t* dst = ok ? a.packed + row * Geo::ROW + hh * Geo::CHUNK + q * Geo::CHUNK_S : a.sink + 64 * lane;
      float* np = ok && hh == 0 && q == 0 ? a.norms + row : (float*)(a.sink + 4096) + lane;
      if constexpr (Geo::G == 16) {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; w += 4)
          put(u32x4{pk[w], pk[w + 1], pk[w + 2], pk[w + 3]}, (u32x4*)(dst + 4 * w));
      } else if constexpr (Geo::G == 8) {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; w += 2) put(u32x2{pk[w], pk[w + 1]}, (u32x2*)(dst + 4 * w));
      } else {
#pragma unroll
        for (int w = 0; w < Geo::CHUNK_DW; ++w) put(pk[w], (uint32_t*)(dst + 4 * w));
      }
      put(nst, np);
    }
  }
}

template <int D, int BITS, int IN, bool SLOT, int QS>
static hipError_t launch_encode_t(const EncodeLaunch& L) {
  using Geo = EncGeo<D, BITS, QS>;
  EncodeKArgs k;
  k.frag = (const u32x4*)L.rot->enc(0);
  k.frag_stride = (int64_t)(L.rot->enc_stride / sizeof(u32x4));
  k.x = L.x;
  k.x_row_stride = L.x_row_stride;
  k.packed = L.packed;
  k.norms = L.norms;
  k.slot = L.slot_mapping;
  k.sink = L.rot->sink();
  k.n = L.n;
  k.vpr = L.vectors_per_rot;
  k.lut_scale = L.lv.lut.scale;
  k.lut_off = L.lv.lut.offset;
  k.norm_correct = L.norm_correct ? 1 : 0;
  for (int j = 0; j < kMaxLevels; ++j) k.csq[j] = L.lv.centroid_sq[j];
  // 2- and 3-bit codes are packed by funnel shifts from the top bits of the difference
  for (int j = 0; j < kLutBins; ++j) k.lut[j] = BITS < 4 ? L.lv.lut.entry_top[j] : L.lv.lut.entry[j];
  const int64_t per_rot = L.vectors_per_rot ? L.vectors_per_rot : L.n;
  const int nrot = L.vectors_per_rot ? (int)((L.n + L.vectors_per_rot - 1) / L.vectors_per_rot) : 1;
  const int64_t tiles = (per_rot + 31) / 32;
  const size_t lds = Geo::LDS ? Geo::FRAG_U4 * sizeof(u32x4) : 0;
  if (lds > 0) {
    hipError_t e = set_kernel_lds((const void*)encode_kernel<D, BITS, IN, SLOT, QS>, L.rot->device, lds);
    if (e != hipSuccess) return e;
  }
  constexpr int WAVES = enc_waves<D, IN>();
  const int cu = device_cu_count(L.rot->device);
  const int64_t want = (int64_t)cu * Geo::WG_PER_CU;
  int64_t slots = (want / QS + nrot - 1) / nrot;
  const int64_t need = (tiles + WAVES - 1) / WAVES;
  if (slots > need) slots = need;
  if (slots < 1) slots = 1;
  if (QS > 1) slots = (slots + 7) / 8 * 8;   // whole groups of 8 slots: a slot's slices share an XCD
  dim3 grid((unsigned)(slots * QS), (unsigned)nrot);
  hipLaunchKernelGGL((encode_kernel<D, BITS, IN, SLOT, QS>), grid, dim3(WAVES * 64), lds, L.stream, k);
  return hipGetLastError();
}

template <int D, int BITS, int IN>
static hipError_t dispatch_slot(const EncodeLaunch& L) {
  // d = 256: two slices with Pi's rows in LDS, except for the norm correction, which needs the
  // code energies of the whole vector in one workgroup
  if constexpr (D == 256) {
    if (!L.norm_correct)
      return L.slot_mapping ? launch_encode_t<D, BITS, IN, true, 2>(L) : launch_encode_t<D, BITS, IN, false, 2>(L);
  }
  return L.slot_mapping ? launch_encode_t<D, BITS, IN, true, 1>(L) : launch_encode_t<D, BITS, IN, false, 1>(L);
}

template <int D, int BITS>
static hipError_t dispatch_in(const EncodeLaunch& L) {
  switch (L.x_dtype) {
    case TQ_F32: return dispatch_slot<D, BITS, TQ_F32>(L);
    case TQ_BF16: return dispatch_slot<D, BITS, TQ_BF16>(L);
    default: return dispatch_slot<D, BITS, TQ_F16>(L);
  }
}

template <int D>
static hipError_t dispatch_bits(const EncodeLaunch& L) {
  switch (L.bits) {
    case 2: return dispatch_in<D, 2>(L);
    case 3: return dispatch_in<D, 3>(L);
    default: return dispatch_in<D, 4>(L);
  }
}

hipError_t launch_encode(const EncodeLaunch& L) {
  if (L.rot->hadamard) return launch_encode_wht(L);
  switch (L.rot->d) {
    case 64: return dispatch_bits<64>(L);
    case 128: return dispatch_bits<128>(L);
    default: return dispatch_bits<256>(L);
  }
}

}  // namespace tq
