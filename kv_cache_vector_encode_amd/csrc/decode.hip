// Decode kernel: unpack, centroid lookup, inverse rotation and norm scaling.
//
// Method (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv, TurboQuantCompressorMSE
// .decompress): x_hat = (c[idx] Pi) * n, cast to the output dtype.
//
// Layout mirrors the encode: a wave owns 32 vectors; lane (v, hh) reads the packed chunk of
// rotated coordinates hh*d/2 .. +d/2 of vector v and turns 8 codes at a time into fp16 MFMA B
// operands; 32x32x16 fp16 MFMAs against prebuilt tiles of Pi^T (resident in LDS) leave 16
// consecutive output coordinates of one vector in a lane's accumulator (tile t, half hh:
// coordinates 32t + 16hh .. +16 of the slice), which are scaled by n, staged in LDS and stored
// 128 bytes of each of the wave's 32 rows at a time (a full cache line per row), 1 KiB per
// store instruction. With that small staging area a CU holds 12 or 16 waves at d = 128.
//
// Precision. A 16-bit output is the float64 decode rounded to nearest even, so the kernel's
// unrounded value must sit well inside a 16-bit half-ulp of the float64 one; single fp16
// operands (2^-12 relative each) leave ~3e-4 of the norm, which changes the rounding of many
// elements. Pi^T is therefore split, Pi^T = P_hi + P_lo with both parts in fp16 (2^-22
// relative). The centroid operand takes one of two forms:
//  * fp16 and float32 outputs, and 4-bit codebooks: c = c_hi + c_lo, and
//      2^19 Pi^T c ~ (2^11 P_hi)(2^8 c_hi) + (2^11 P_lo)(2^8 c_hi) + (2^11 P_hi)(2^8 c_lo),
//    three products into one fp32 accumulator (the scalings keep every low part a normal fp16
//    number; P_lo c_lo, ~2^-24 relative, is dropped): ~1.2e-7 of the vector norm per element
//    in a float emulation;
//  * bfloat16 outputs of 2- and 3-bit codebooks: one operand. A codebook has only 2^(bits-1)
//    centroid magnitudes, and the host picks a scale alpha in [1, 2) under which every
//    2^8 alpha c_k is within rho <= 2.5e-5 (relative) of an fp16 value c'_k; then
//      2^19 alpha Pi^T c ~ (2^11 P_hi) c' + (2^11 P_lo) c',
//    two products, and since every row of Pi^T has unit norm, each element is within
//    rho ||x|| of the result with exact centroids (Cauchy-Schwarz): a fifth of a bfloat16
//    half-ulp at a coordinate of typical size ||x|| / sqrt(d) at worst, and as a sum of d
//    terms of either sign typically ~1/sqrt(d) of that. The 1/alpha goes into the norm
//    multiplier.
// The A1 = 2^11 P_hi operand is read once for two products, so LDS reads grow by half a tile
// set per product, not by two.
//
// Instruction budget. On gfx950 the vector ALU and LDS instructions of a SIMD issue largely
// in series with its MFMAs (a probe that gives each wave independent fp32 FMAs next to its
// MFMA chains runs in nearly the sum of the two times), so everything around the MFMAs is
// kept to few instructions: the code -> operand tables return each 32-bit operand word
// straight into its MFMA register (hi and lo tables, one LDS read per word, no moves), a
// code pair's table offset is two ALU operations, the staging area is padded rather than
// swizzled so that every LDS address is a per-lane base plus a constant, and without a slot
// gather the packed rows are read, and every output row is written, through buffer
// resources over the tile's rows: a lane's address is a 32-bit offset from a uniform base,
// and rows past the end read as zero or are dropped by the hardware's range check.
//
// Head size 256: the two tile sets of the whole Pi^T (256 KiB) do not fit in LDS, so four
// workgroups share each group of vectors, each holding the tiles of one quarter of the output
// coordinates (64 KiB) and writing that quarter of every row. The four are numbered 8 apart,
// which places them on one XCD (workgroups are dealt to the XCDs in turn), so three of the
// four reads of each packed row hit that XCD's L2.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {

struct DecodeKArgs {
  const u32x4* frag;     // Pi^T tiles, rotation r at frag + r * frag_stride
  int64_t frag_stride;
  const uint8_t* packed;
  const float* norms;
  const int64_t* slot;
  void* out;
  const uint8_t* zero;   // zeros that masked lanes load with a slot gather (>= one packed chunk)
  int64_t n, vpr;
  float nscale;          // x_hat = acc * n * nscale
  uint32_t chi[8];       // 2^8 c_hi (or 2^8 alpha c) as fp16, two per word
  uint32_t clo[8];       // 2^8 c_lo as fp16, two per word (three-product decodes)
};

template <int D, int BITS, int OUT>
struct DecGeo {
  static constexpr int T = D / 32, KB = D / 16, HALF = D / 2;
  static constexpr int QS = D == 256 ? 4 : 1;     // output slices (workgroups per vector group)
  static constexpr int TS = T / QS;               // output tiles per slice
  static constexpr int SC = D / QS;               // output coordinates per slice
  static constexpr int ROW = D * BITS / 8;
  static constexpr int CHUNK = HALF * BITS / 8;
  static constexpr int CHUNK_DW = CHUNK / 4;
  static constexpr int G = (CHUNK % 16 == 0 && ROW % 16 == 0) ? 16 : ((CHUNK % 8 == 0 && ROW % 8 == 0) ? 8 : 4);
  static constexpr int E = OUT == TQ_F32 ? 4 : 2;  // output bytes per element
  static constexpr bool P3 = !decode_one_operand(BITS, OUT);   // c_hi + c_lo: three products
  static constexpr int SET_U4 = TS * KB * 64;       // one tile set of a slice, in u32x4
  static constexpr int FRAG_U4 = 2 * SET_U4;        // A1 and A2
  // Code -> centroid tables, a hi table and a lo table: 2-bit codes go four at a time (one
  // byte -> four fp16, two words per entry), 3- and 4-bit codes two at a time (6 or 8 bits ->
  // two fp16, one word per entry).
  static constexpr int PER_LOOKUP = BITS == 2 ? 4 : 2;
  static constexpr int LOOKUP_BITS = PER_LOOKUP * BITS;
  static constexpr int TAB_N = 1 << LOOKUP_BITS;
  static constexpr int ENTRY_B = PER_LOOKUP * 2;            // bytes per entry (fp16 each)
  static constexpr int TAB_B = TAB_N * ENTRY_B;             // bytes per table
  // the lo table starts LO_OFF bytes after the hi one: further apart than one two-address LDS
  // read reaches and not a multiple of its stride, so each word is read into its own register
  static constexpr int LO_OFF = (TAB_B > 2048 ? TAB_B : 2048) + 8;
  // Launch shape: d = 64 in two 4-wave workgroups per CU; d = 128 in one workgroup per CU (the
  // tile sets take 64 KiB of LDS) of 16 waves with the single-operand centroid table (4 per SIMD
  // within 128 registers: 5% faster than 12) and of 12 with the hi/lo one (3 per SIMD within
  // 170); d = 256 in one 16-wave workgroup per CU: with two tiles per slice it looks its operands
  // up one K block at a time (KB_OUTER), which keeps it within 128 registers.
  static constexpr bool KB_OUTER = D == 256;
  static constexpr int WAVES = D == 64 ? 4 : (D == 128 ? (decode_one_operand(BITS, OUT) ? 16 : 12) : 16);
  static constexpr int WG_PER_CU = D == 64 ? 2 : 1;
  static constexpr int WPE = WAVES * WG_PER_CU / 4;   // waves per SIMD
  static constexpr int SB = SC * E;                    // output bytes of a row in this slice
  // Outputs go out in flushes of FT tiles, 128 bytes of each of the wave's 32 rows (tile t holds
  // slice coordinates 32t .. 32t+31): staged as 32 rows of 128 bytes, each padded by 16 bytes
  // so that rows written by consecutive lanes start in different banks.
  static constexpr int FT = 128 / (32 * E);
  static constexpr int STG_ROW = 128 + 16;
  static constexpr size_t stage_bytes = (size_t)32 * STG_ROW;
  static constexpr size_t lds_bytes = (size_t)FRAG_U4 * 16 + (size_t)WAVES * stage_bytes;
  static_assert(lds_bytes + LO_OFF + TAB_B <= 160 * 1024, "decode LDS budget");
  static_assert(TS % FT == 0, "whole flushes per slice");
};

template <int D, int BITS, int OUT>
constexpr int dec_wpe() { return DecGeo<D, BITS, OUT>::WPE; }

template <int D, int BITS, int OUT, bool SLOT>
__global__ void __launch_bounds__((DecGeo<D, BITS, OUT>::WAVES * 64))
__attribute__((amdgpu_waves_per_eu(dec_wpe<D, BITS, OUT>())))
decode_kernel(DecodeKArgs a) {
  using Geo = DecGeo<D, BITS, OUT>;
  constexpr int TS = Geo::TS, KB = Geo::KB, QS = Geo::QS, WAVES = Geo::WAVES, E = Geo::E, DW = Geo::CHUNK_DW;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  extern __shared__ u32x4 smem[];
  // hi table at 0, lo table at LO_OFF (TAB_B bytes each)
  __shared__ __attribute__((aligned(16))) uint32_t tab[(Geo::LO_OFF + Geo::TAB_B) / 4];

  const int r = blockIdx.y;
  // slice q and vector-group slot of this workgroup (slices of one slot are 8 apart)
  const int wg = blockIdx.x;
  const int q = QS == 1 ? 0 : (wg >> 3) % QS;
  const int slot_id = QS == 1 ? wg : (wg & 7) + 8 * (wg / (8 * QS));
  const int nslots = gridDim.x / QS;
  const u32x4* gfrag = a.frag + (int64_t)r * a.frag_stride + (int64_t)q * Geo::FRAG_U4;

  const int64_t v_begin = a.vpr ? (int64_t)r * a.vpr : 0;
  const int64_t v_end = a.vpr ? min(a.n, v_begin + a.vpr) : a.n;
  const int64_t ntile = (v_end - v_begin + 31) / 32;
  if (ntile <= 0) return;   // uniform per workgroup: no thread is left at the barrier below
  // the wave index through readfirstlane, so that tile indices and the buffer resources built
  // from them stay uniform (scalar registers)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int vl = lane & 31, hh = lane >> 5;
  uint8_t* stg = (uint8_t*)(smem + Geo::FRAG_U4) + wave * Geo::stage_bytes;

  // rows of tile tl that exist (0 past the end), uniform
  auto valid_rows = [&](int64_t tl) -> uint32_t {
    const int64_t left = v_end - (v_begin + tl * 32);
    return left <= 0 ? 0u : (left >= 32 ? 32u : (uint32_t)left);
  };
  // Prefetch one tile ahead (and with a slot gather, the slot index one tile earlier still).
  const int64_t wstride = (int64_t)nslots * WAVES;
  auto slot_row = [&](int64_t tl) -> int64_t {
    if constexpr (SLOT) {
      const int64_t v = v_begin + tl * 32 + vl;
      const bool ok = tl < ntile && v < v_end;
      const int64_t s = a.slot[ok ? v : v_begin];
      return ok ? s : -1;
    } else {
      (void)tl;
      return 0;
    }
  };
  auto fetch = [&](int64_t tl, int64_t srow, uint32_t (&cw)[DW], float& nrm) {
    if constexpr (SLOT) {
      const uint8_t* src = srow >= 0 ? a.packed + srow * Geo::ROW + hh * Geo::CHUNK : a.zero;
      if constexpr (Geo::G == 16) {
#pragma unroll
        for (int w = 0; w < DW; w += 4) {
          const u32x4 v = *(const u32x4*)(src + 4 * w);
          cw[w] = v[0]; cw[w + 1] = v[1]; cw[w + 2] = v[2]; cw[w + 3] = v[3];
        }
      } else if constexpr (Geo::G == 8) {
#pragma unroll
        for (int w = 0; w < DW; w += 2) {
          const u32x2 v = *(const u32x2*)(src + 4 * w);
          cw[w] = v[0]; cw[w + 1] = v[1];
        }
      } else {
#pragma unroll
        for (int w = 0; w < DW; ++w) cw[w] = *(const uint32_t*)(src + 4 * w);
      }
      nrm = *(srow >= 0 ? a.norms + srow : (const float*)a.zero);
    } else {
      (void)srow;
      // the tile's rows through a buffer resource: rows past the end read as zero
      const int64_t vb = v_begin + tl * 32;
      const uint32_t nv = valid_rows(tl);
      const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(a.packed + (nv ? vb : 0) * Geo::ROW, nv * Geo::ROW);
      const __amdgpu_buffer_rsrc_t rn = buffer_rsrc(a.norms + (nv ? vb : 0), nv * 4u);
      const uint32_t off = (uint32_t)(vl * Geo::ROW + hh * Geo::CHUNK);
      if constexpr (Geo::G == 16) {
#pragma unroll
        for (int w = 0; w < DW; w += 4) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rp, off + 4 * w, 0, 0);
          cw[w] = v[0]; cw[w + 1] = v[1]; cw[w + 2] = v[2]; cw[w + 3] = v[3];
        }
      } else if constexpr (Geo::G == 8) {
#pragma unroll
        for (int w = 0; w < DW; w += 2) {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rp, off + 4 * w, 0, 0);
          cw[w] = v[0]; cw[w + 1] = v[1];
        }
      } else {
#pragma unroll
        for (int w = 0; w < DW; ++w) cw[w] = __builtin_amdgcn_raw_buffer_load_b32(rp, off + 4 * w, 0, 0);
      }
      nrm = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, (uint32_t)vl * 4u, 0, 0));
    }
  };

  // tiles go to waves wave-major (as in the encode): an uneven last round is spread over every
  // workgroup instead of falling to a subset of them
  int64_t tile = (int64_t)wave * nslots + slot_id;
  uint32_t cwA[DW], cwB[DW];
  float nA, nB;
  int64_t sA = slot_row(tile), sB = 0;
  // the first tile's loads are issued before the table copies below, so the two latencies overlap
  fetch(tile, sA, cwA, nA);
  sB = slot_row(tile + wstride);

  for (int i = threadIdx.x; i < Geo::FRAG_U4; i += blockDim.x) smem[i] = gfrag[i];
  {
    // centroids straight from the kernel-argument segment (indexing the by-value copy with a
    // lane-dependent index would go through scratch)
    const char* kseg = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    const uint32_t* khi = (const uint32_t*)(kseg + offsetof(DecodeKArgs, chi));
    const uint32_t* klo = (const uint32_t*)(kseg + offsetof(DecodeKArgs, clo));
    auto cent = [&](const uint32_t* t, uint32_t k) -> uint32_t { return (t[k >> 1] >> (16 * (k & 1))) & 0xffffu; };
    constexpr int EW = Geo::ENTRY_B / 4;   // words per entry
    for (int j = threadIdx.x; j < Geo::TAB_N; j += blockDim.x) {
#pragma unroll
      for (int part = 0; part < (Geo::P3 ? 2 : 1); ++part) {
        const uint32_t* kc = part ? klo : khi;
        uint32_t* t = tab + part * (Geo::LO_OFF / 4) + EW * j;
        if constexpr (Geo::PER_LOOKUP == 4) {
          // entry j: codes j, j>>2, j>>4, j>>6 as two words
          const uint32_t k0 = j & MASK, k1 = (j >> BITS) & MASK, k2 = (j >> (2 * BITS)) & MASK, k3 = j >> (3 * BITS);
          t[0] = cent(kc, k0) | (cent(kc, k1) << 16);
          t[1] = cent(kc, k2) | (cent(kc, k3) << 16);
        } else {
          // entry j: codes j & MASK, j >> BITS as one word
          t[0] = cent(kc, j & MASK) | (cent(kc, j >> BITS) << 16);
        }
      }
    }
  }
  __syncthreads();
  wait_vmem_all();

  // per-lane LDS and output offsets (the rest of every address is a constant)
  constexpr uint32_t RB = D * E;                    // bytes per output row
  // lane (v, hh) stages tile t's 16 outputs at byte (t % FT) * 32E + 16hh*E of staged row v; a
  // flush stores 8 rows per instruction, lane l the 16 bytes at 16(l % 8) of row l / 8
  uint8_t* const stg_w = stg + vl * Geo::STG_ROW + 16 * hh * E;
  const uint32_t lrow = (uint32_t)lane >> 3, lchunk = (uint32_t)lane & 7u;
  const uint8_t* const stg_r = stg + lrow * Geo::STG_ROW + 16 * lchunk;
  const uint32_t out_off = lrow * RB + (uint32_t)q * Geo::SB + 16 * lchunk;

  auto decode_tile = [&](const uint32_t (&cw)[DW], float nrm, int64_t tl) {
    const int64_t vbase = v_begin + tl * 32;
    // x_hat = acc * n * 2^-19 (the operand scalings), / alpha with the single-operand table
    const float ns = nrm * a.nscale;

    // ---- codes -> fp16 centroids (hi and lo), 8 per K block (the lane's codes 8kb .. 8kb+7),
    //      every word read from its table straight into its operand register
    const char* tb = (const char*)tab;
    auto lookup = [&](int kb, u32x4& bh, u32x4& bl) {
      if constexpr (BITS == 2) {
        // 8 codes = 16 bits = two table bytes, two fp16 words each
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int p = 16 * kb + 8 * h;               // bit position of the byte in the chunk
          const uint32_t w = cw[p >> 5];
          const int s = p & 31;
          const uint32_t off = (s >= 3 ? (w >> (s - 3)) : (w << (3 - s))) & (255u << 3);
          const u32x2 eh = *(const u32x2*)(tb + off);
          u32x2 el{};
          if constexpr (Geo::P3) el = *(const u32x2*)(tb + Geo::LO_OFF + off);
          bh[2 * h] = eh[0]; bh[2 * h + 1] = eh[1];
          if constexpr (Geo::P3) { bl[2 * h] = el[0]; bl[2 * h + 1] = el[1]; }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          constexpr int PB = 2 * BITS;           // bits per code pair
          const int pos = (4 * kb + c) * PB;     // compile-time after unrolling
          const int s = pos & 31;
          uint32_t off;
          if (s + PB <= 32)
            off = (s >= 2 ? (cw[pos >> 5] >> (s - 2)) : (cw[pos >> 5] << (2 - s))) & (((1u << PB) - 1u) << 2);
          else
            off = funnel(cw[(pos >> 5) + 1], cw[pos >> 5], s - 2) & (((1u << PB) - 1u) << 2);
          bh[c] = *(const uint32_t*)(tb + off);
          if constexpr (Geo::P3) bl[c] = *(const uint32_t*)(tb + Geo::LO_OFF + off);
        }
      }
    };
    u32x4 bhi[Geo::KB_OUTER ? 1 : KB], blo[Geo::KB_OUTER ? 1 : KB]{};
    if constexpr (!Geo::KB_OUTER) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) lookup(kb, bhi[kb], blo[kb]);
    }

    // ---- inverse rotation (an opaque offset keeps the Pi^T tiles in LDS instead of letting
    //      the compiler hoist all of them into registers)
    uint32_t aoff = (uint32_t)lane * 16u;
    asm volatile("" : "+v"(aoff));
    f32x16 accp[2];
    const uint32_t nv = valid_rows(tl);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc((uint8_t*)a.out + (nv ? vbase : 0) * RB, nv * RB);
#pragma unroll
    for (int t = 0; t < TS; ++t) {
      if (t % 2 == 0) {
        // two independent accumulation chains in flight
        accp[0] = f32x16{};
        accp[1] = f32x16{};
        if constexpr (Geo::KB_OUTER) {
          // the operands of one K block at a time, looked up one block ahead (two register sets),
          // so only 16 operand registers are live
          u32x4 bh[2], bl[2]{};
          lookup(0, bh[0], bl[0]);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            if (kb + 1 < KB) lookup(kb + 1, bh[(kb + 1) & 1], bl[(kb + 1) & 1]);
            const u32x4 h = bh[kb & 1], l = bl[kb & 1];
            const char* s0 = (const char*)smem + aoff + (t * KB + kb) * 1024;
            const char* s1 = (const char*)smem + aoff + ((t + 1) * KB + kb) * 1024;
            const u32x4 a1_0 = *(const u32x4*)s0, a2_0 = *(const u32x4*)(s0 + Geo::SET_U4 * 16);
            const u32x4 a1_1 = *(const u32x4*)s1, a2_1 = *(const u32x4*)(s1 + Geo::SET_U4 * 16);
            accp[0] = mfma32_f16(a1_0, h, accp[0]);
            accp[1] = mfma32_f16(a1_1, h, accp[1]);
            accp[0] = mfma32_f16(a2_0, h, accp[0]);
            accp[1] = mfma32_f16(a2_1, h, accp[1]);
            if constexpr (Geo::P3) {
              accp[0] = mfma32_f16(a1_0, l, accp[0]);
              accp[1] = mfma32_f16(a1_1, l, accp[1]);
            }
            // keep the scheduler from pulling every later block's lookups ahead of these MFMAs
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const char* s0 = (const char*)smem + aoff + (t * KB + kb) * 1024;
            const char* s1 = (const char*)smem + aoff + ((t + 1) * KB + kb) * 1024;
            const u32x4 a1_0 = *(const u32x4*)s0, a2_0 = *(const u32x4*)(s0 + Geo::SET_U4 * 16);
            const u32x4 a1_1 = *(const u32x4*)s1, a2_1 = *(const u32x4*)(s1 + Geo::SET_U4 * 16);
            accp[0] = mfma32_f16(a1_0, bhi[kb], accp[0]);
            accp[1] = mfma32_f16(a1_1, bhi[kb], accp[1]);
            accp[0] = mfma32_f16(a2_0, bhi[kb], accp[0]);
            accp[1] = mfma32_f16(a2_1, bhi[kb], accp[1]);
            if constexpr (Geo::P3) {
              accp[0] = mfma32_f16(a1_0, blo[kb], accp[0]);
              accp[1] = mfma32_f16(a1_1, blo[kb], accp[1]);
            }
          }
        }
      }
      const f32x16 acc = accp[t % 2];
      // scaled outputs of slice coordinates 32t + 16hh .. +16 as E 16-byte chunks
      const int tb = (t % Geo::FT) * 32 * E;
      if constexpr (OUT == TQ_F32) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(u32x4*)(stg_w + tb + 16 * q4) =
              u32x4{__float_as_uint(acc[4 * q4] * ns), __float_as_uint(acc[4 * q4 + 1] * ns),
                    __float_as_uint(acc[4 * q4 + 2] * ns), __float_as_uint(acc[4 * q4 + 3] * ns)};
      } else {
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float lo = acc[2 * j] * ns, hi = acc[2 * j + 1] * ns;
          w[j] = OUT == TQ_BF16 ? pack_bf16x2(lo, hi) : pack_f16x2(lo, hi);
        }
        *(u32x4*)(stg_w + tb) = u32x4{w[0], w[1], w[2], w[3]};
        *(u32x4*)(stg_w + tb + 16) = u32x4{w[4], w[5], w[6], w[7]};
      }
      if (t % Geo::FT == Geo::FT - 1) {
        // flush: 128 bytes of each of the 32 rows (a full cache line each), 1 KiB per store
        // instruction, through a buffer resource over the tile's rows (rows past the end are
        // dropped by its range check). Non-temporal: the decoded stream is far larger than the
        // caches, and left in them as dirty lines it is written back during whatever kernel
        // runs next.
        const uint32_t fo = (uint32_t)(t / Geo::FT) * 128u;
#pragma unroll
        for (uint32_t j = 0; j < 4; ++j) {
          const u32x4 qv = *(const u32x4*)(stg_r + j * 8 * Geo::STG_ROW);
          __builtin_amdgcn_raw_buffer_store_b128(qv, ro, out_off + fo + j * 8 * RB, 0, 2 /* nt */);
        }
      }
    }
  };

  // two register sets for the codes, used in turn, so no copy ties a prefetch to its use
  while (true) {
    if (tile >= ntile) break;
    fetch(tile + wstride, sB, cwB, nB);
    sA = slot_row(tile + 2 * wstride);
    decode_tile(cwA, nA, tile);
    tile += wstride;
    if (tile >= ntile) break;
    fetch(tile + wstride, sA, cwA, nA);
    sB = slot_row(tile + 2 * wstride);
    decode_tile(cwB, nB, tile);
    tile += wstride;
  }
}

template <int D, int BITS, int OUT, bool SLOT>
static hipError_t launch_decode_t(const DecodeLaunch& L) {
  using Geo = DecGeo<D, BITS, OUT>;
  DecodeKArgs k;
  k.frag = (const u32x4*)L.rot->dec(0);
  k.frag_stride = (int64_t)(L.rot->dec_stride / sizeof(u32x4));
  k.packed = L.packed;
  k.norms = L.norms;
  k.slot = L.slot_mapping;
  k.out = L.out;
  k.zero = L.rot->zero();
  k.n = L.n;
  k.vpr = L.vectors_per_rot;
  const uint16_t* hi = Geo::P3 ? L.lv.dec_c_hi : L.lv.dec_c_one;
  for (int j = 0; j < 8; ++j) {
    k.chi[j] = (uint32_t)hi[2 * j] | ((uint32_t)hi[2 * j + 1] << 16);
    k.clo[j] = (uint32_t)L.lv.dec_c_lo[2 * j] | ((uint32_t)L.lv.dec_c_lo[2 * j + 1] << 16);
  }
  k.nscale = Geo::P3 ? 0x1p-19f : L.lv.dec_one_nscale;
  const int64_t per_rot = L.vectors_per_rot ? L.vectors_per_rot : L.n;
  const int nrot = L.vectors_per_rot ? (int)((L.n + L.vectors_per_rot - 1) / L.vectors_per_rot) : 1;
  const int64_t tiles = (per_rot + 31) / 32;
  const size_t lds = Geo::lds_bytes;
  hipError_t e = set_kernel_lds((const void*)decode_kernel<D, BITS, OUT, SLOT>, L.rot->device, lds);
  if (e != hipSuccess) return e;
  const int cu = device_cu_count(L.rot->device);
  const int64_t want = (int64_t)cu * Geo::WG_PER_CU;
  int64_t slots = (want / Geo::QS + nrot - 1) / nrot;
  const int64_t need = (tiles + Geo::WAVES - 1) / Geo::WAVES;
  if (slots > need) slots = need;
  if (slots < 1) slots = 1;
  if (Geo::QS > 1) slots = (slots + 7) / 8 * 8;   // whole groups of 8 slots: a slot's slices share an XCD
  const int64_t bx = slots * Geo::QS;
  hipLaunchKernelGGL((decode_kernel<D, BITS, OUT, SLOT>), dim3((unsigned)bx, (unsigned)nrot), dim3(Geo::WAVES * 64),
                     lds, L.stream, k);
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
  if (L.rot->hadamard) return launch_decode_wht(L);
  switch (L.rot->d) {
    case 64: return dec_bits<64>(L);
    case 128: return dec_bits<128>(L);
    default: return dec_bits<256>(L);
  }
}

}  // namespace tq
