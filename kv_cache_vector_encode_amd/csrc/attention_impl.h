// Scores and fused decode attention straight from the compressed cache (kernels and their
// launch templates, shared by attention.hip and attention_qjl.hip).
//
// Method: s_t = scale <q, k_hat_t> (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv,
// TurboQuantKVCache.attention_scores) and o = softmax(s) v_hat (TurboQuantKVCache.attend).
// Because k_hat_t = n_t Pi_K^T c_K[idx_t], <q, k_hat_t> = n_t <Pi_K q, c_K[idx_t]>: the query is
// rotated once and keys are never un-rotated (Turbo Attention PyPI page, "The codec", which
// applies the key rotation to the queries as well). Likewise sum_t p_t v_hat_t =
// Pi_V^T sum_t p_t n^v_t c_V[idx^v_t]: values are accumulated in the rotated domain and
// rotated back once per (sequence, head). Split-K over tokens with an online softmax and a
// log-sum-exp merge plays the role of the pages' split-K paged decode kernel (same page,
// "Kernels").
//
// Work layout. Kernel 1 rotates every query (fp32). Kernel 2: a wave owns one (sequence,
// KV head, token range) and walks it 32 tokens at a time.
//   scores: 16x16x32 bf16 MFMA on hi/lo splits, A = centroids of 16 tokens (lane m+16g holds
//     token m's codes for coordinates g*d/4 + ...), B = the G <= 16 rotated queries of the
//     group (times the score scale), D[token][head]; three passes for 2/3-bit keys, two for
//     4-bit keys (whose K dimension runs over (coordinate, hi / lo) against a duplicated query).
//   QJL keys (TurboQuantCompressorV2.asymmetric_attention_scores on the same page) add
//     ||r_t|| sqrt(pi/2)/d <S q, signs_t>: a second product with A = the token's signs as
//     bf16 +-1 (exact; same lane layout as the codes) and B = S q split into bf16 hi + lo.
//   softmax (base 2): per head running max m, running sum l; the value weights p_t n^v_t are
//     kept relative to the running max V norm N so that they fit fp16; m and N move only past
//     a margin, so most blocks need no cross-lane reduction.
//   P.V: 16x16x32 fp16 MFMA computing acc^T[coord][head]. The 32 tokens of a block are
//     permuted so that lane (head, g) already holds, from the score step, the weights of the
//     8 tokens it must supply (4g..4g+3 and 16+4g..16+4g+3): no shuffles. The A operand is
//     the V centroids of those 8 tokens for coordinate group m (coordinates m*d/16 + t').
// Kernel 3 merges the splits: M = max m_s, L = sum l_s e^(m_s-M), o = Pi_V^T (sum acc_s
// e^(m_s-M)) / L, lse = M + log L.
#pragma once

#include <math.h>

#include <cmath>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "tq_internal.h"

namespace tq {

struct AttnKArgs {
  const float* qrot;
  const uint8_t* kp;
  const float* kn;
  const uint8_t* vp;
  const float* vn;
  const int32_t* seq_lens;
  const int32_t* block_table;
  float* scores;
  float* part;
  float* sink;         // where masked lanes store scores (>= 64 floats)
  int32_t max_seq_len, block_size, bs_shift, mbps;
  int32_t B, Hq, Hkv, G, s_eff;
  int32_t window;     // newest tokens held in the full-precision window (0: none)
  int32_t one_round;  // 1 when every wave of the grid is resident at once (progress priorities)
  float scale;
  uint32_t ctk[16];   // K centroids as bf16 hi | lo << 16
  uint32_t ctv[8];    // V centroids as fp16, two per word
  // QJL keys
  const uint8_t* ksg;  // sign rows, d/8 bytes per token
  const float* krn;    // residual norms
  const float* qsk;    // S q [B, Hq, d]
  float qjl_c;         // sqrt(pi/2) / d
};

constexpr int kAttnWaves = 4;

// Cache addressing: 0 = dense, 1 = paged with a power-of-two block size >= 16 (a 32-token
// block then spans at most two pages, looked up once per block), 2 = any other paging.
enum AttnPaging { kDense = 0, kPagedPow2 = 1, kPagedAny = 2 };

// NB bits of a packed row starting at bit `bitoff`, shifted down to bit 0 of out[0]. Loads are
// unconditional and stay inside the row of ROWB bytes.
template <int NB, int ROWB>
__device__ __forceinline__ void load_chunk(const uint8_t* row, int bitoff, uint32_t (&out)[(NB + 31) / 32]) {
  constexpr int NW = (NB + 31) / 32;
  if constexpr (NB % 32 == 0) {
    // bitoff is a multiple of NB here, so the chunk is NB/8-byte aligned
    const uint8_t* p = row + bitoff / 8;
    if constexpr (NW == 4) {
      const u32x4 v = *(const u32x4*)p;
      out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (NW == 2) {
      const u32x2 v = *(const u32x2*)p;
      out[0] = v[0]; out[1] = v[1];
    } else {
#pragma unroll
      for (int k = 0; k < NW; ++k) out[k] = ((const uint32_t*)p)[k];
    }
  } else if constexpr (NB == 16) {
    out[0] = *(const uint16_t*)(row + bitoff / 8);
  } else if constexpr (NB == 8) {
    out[0] = row[bitoff / 8];
  } else {
    constexpr int ROW_DW = ROWB / 4;
    const uint32_t* rw = (const uint32_t*)row;
    const int idx = bitoff >> 5;
    const uint32_t sh = (uint32_t)bitoff & 31u;
    uint32_t w[NW + 1];
#pragma unroll
    for (int k = 0; k <= NW; ++k) w[k] = rw[min(idx + k, ROW_DW - 1)];   // a clamped word only feeds bits past NB
#pragma unroll
    for (int k = 0; k < NW; ++k) out[k] = funnel(w[k + 1], w[k], sh);
  }
}

// The same through a buffer resource: `row` is the row's byte offset from the resource base.
// Buffer loads take a 32-bit offset next to a uniform base, so a lane's address costs no 64-bit
// arithmetic.
template <int NB, int ROWB>
__device__ __forceinline__ void load_chunk_buf(__amdgpu_buffer_rsrc_t rs, uint32_t row, int bitoff,
                                               uint32_t (&out)[(NB + 31) / 32]) {
  constexpr int NW = (NB + 31) / 32;
  if constexpr (NB % 32 == 0) {
    const uint32_t o = row + (uint32_t)bitoff / 8;
    if constexpr (NW == 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
      out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (NW == 2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
      out[0] = v[0]; out[1] = v[1];
    } else {
#pragma unroll
      for (int k = 0; k < NW; ++k) out[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, o + 4 * k, 0, 0);
    }
  } else if constexpr (NB == 16) {
    out[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, row + (uint32_t)bitoff / 8, 0, 0);
  } else if constexpr (NB == 8) {
    out[0] = __builtin_amdgcn_raw_buffer_load_b8(rs, row + (uint32_t)bitoff / 8, 0, 0);
  } else {
    constexpr int ROW_DW = ROWB / 4;
    const int idx = bitoff >> 5;
    const uint32_t sh = (uint32_t)bitoff & 31u;
    uint32_t w[NW + 1];
#pragma unroll
    for (int k = 0; k <= NW; ++k) w[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, row + 4u * min(idx + k, ROW_DW - 1), 0, 0);
#pragma unroll
    for (int k = 0; k < NW; ++k) out[k] = funnel(w[k + 1], w[k], sh);
  }
}

// 2^x by the hardware instruction (x = -inf gives 0)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// the LDS word at byte offset `off` of table t
__device__ __forceinline__ uint32_t lds_word(const uint32_t* t, uint32_t off) {
  return *(const uint32_t*)((const char*)t + off);
}


// PB bits at bit `pos` of w (pos is a compile-time constant after unrolling)
template <int PB, int NW>
__device__ __forceinline__ uint32_t bits_at(const uint32_t (&w)[NW], int pos) {
  uint32_t v;
  if ((pos & 31) + PB <= 32)
    v = w[pos >> 5] >> (pos & 31);
  else
    v = funnel(w[(pos >> 5) + 1], w[pos >> 5], (uint32_t)(pos & 31));
  return v & ((1u << PB) - 1u);
}

// a, b: up to eight 2-bit codes each (low 16 bits). Returns z with nibble t = a_t | b_t << 2,
// so byte j of z holds codes 2j and 2j+1 of both (bytes of a and b interleaved, then two
// swaps of bit fields inside each 16-bit half).
__device__ __forceinline__ uint32_t interleave2(uint32_t a, uint32_t b) {
  uint32_t y = (a & 0xffu) | ((b & 0xffu) << 8) | ((a & 0xff00u) << 8) | ((b & 0xff00u) << 16);
  uint32_t t = (y ^ (y >> 4)) & 0x00f000f0u;
  y ^= t ^ (t << 4);
  t = (y ^ (y >> 2)) & 0x0c0c0c0cu;
  y ^= t ^ (t << 2);
  return y;
}

// the same with a and b packed as a | b << 16: the byte interleave is one byte permute
__device__ __forceinline__ uint32_t interleave2_packed(uint32_t x) {
  uint32_t y = __builtin_amdgcn_perm(x, x, 0x03010200u);   // bytes a0, b0, a1, b1
  uint32_t t = (y ^ (y >> 4)) & 0x00f000f0u;
  y ^= t ^ (t << 4);
  t = (y ^ (y >> 2)) & 0x0c0c0c0cu;
  y ^= t ^ (t << 2);
  return y;
}

// Waves per SIMD an attention kernel is built for (its register budget with two buffer sets
// of block operands): 3 at d <= 128 (<= 168 registers), 4 for dense caches at d = 128 with
// 4-bit keys and 2-bit values (their operands fit 128 registers), 2 at d = 256 (twice the
// accumulators); one step lower with the QJL operands or 3-bit values (their 24-bit code
// segments take more registers).
constexpr int attn_wpe(int d, int bk, int bv, bool qjl, bool paged) {
  return (bv == 3 && !qjl) ? (d == 256 ? 1 : 2)
         : d == 256        ? (qjl ? 1 : 2)
         : qjl             ? 2
         : (d == 128 && bk == 4 && bv == 2 && !paged) ? 4
                                                      : 3;
}

template <int D, int BK, int BV, bool SCORES, int PAGE, bool QJL, bool MQ>
__global__ void __launch_bounds__(kAttnWaves * 64) __attribute__((amdgpu_waves_per_eu(attn_wpe(D, BK, BV, QJL, PAGE != kDense))))
attn_kernel(AttnKArgs a) {
  constexpr int KB = D / 32;            // K blocks of the score MFMA
  constexpr int TV = D / 16;            // output tiles of the P.V MFMA
  constexpr int NBK = D * BK / 4;       // bits of a lane's K chunk
  constexpr int NBV = D * BV / 16;      // bits of a lane's V segment
  constexpr int NWK = (NBK + 31) / 32, NWV = (NBV + 31) / 32;
  constexpr int NBS = D / 4;            // bits of a lane's sign chunk (QJL keys)
  constexpr int NWS = (NBS + 31) / 32;
  constexpr int ROWK = D * BK / 8, ROWV = D * BV / 8;
  constexpr int PK = 2 * BK;            // bits of a pair of K codes
  // Code -> operand tables in LDS. A table of at most 16 words is read without bank conflicts
  // (lanes that pick the same entry share one read); random picks from a larger table cost
  // more LDS cycles, but a byte index is one instruction (a byte select with the shift), a
  // nibble index two. So:
  //   4-bit keys (K1): a byte of codes (two coordinates) -> two words, each the centroid's
  //     bf16 hi | lo << 16, and the score MFMA's K dimension runs over (coordinate, hi / lo)
  //     with the query duplicated, so one product takes (c_hi + c_lo) q_hi and a second one
  //     (c_hi + c_lo) q_lo;
  //   2/3-bit keys: a pair of codes (at most 64 entries) -> two bf16 hi / lo (both in tkh)
  //     halves, three products per K block (c_hi q_hi + c_lo q_hi + c_hi q_lo);
  //   values: a pair of V codes (one coordinate of two tokens) -> one fp16 pair; 2-bit codes
  //     are first interleaved so that each nibble is such a pair (16 entries).
  constexpr bool K1 = BK == 4;
  constexpr int KB1 = D / 16;           // score MFMAs per pass with one code per operand word
  constexpr int KTAB = K1 ? 512 : 1 << PK;
  constexpr int VTAB = 1 << (2 * BV);
  // 2/3-bit keys: the lo halves start KLO bytes after the hi halves, further apart than one
  // two-address LDS read reaches and not a multiple of its 256-byte stride, so the compiler
  // cannot merge a pair's two reads into one two-register read that would then need moves:
  // each word goes straight into its MFMA operand register
  constexpr int KLO = K1 ? 0 : (4 * KTAB > 1024 ? 4 * KTAB : 1024) + 8;
  __shared__ __attribute__((aligned(16))) uint32_t tkh[K1 ? KTAB : (KLO + 4 * KTAB) / 4];
  __shared__ uint32_t tv[SCORES ? 1 : VTAB];
  constexpr int NQB = K1 ? KB1 : KB;    // query operand words per pass and lane
  __shared__ u32x4 sq[2 * NQB * 64];   // query B operands [hi, lo][kb][lane], shared by the waves
  __shared__ u32x4 ssq[QJL ? 2 * KB * 64 : 1];   // the same for S q (QJL keys)

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int sidx = blockIdx.x * kAttnWaves + wave;
  // compressed tokens: all but the newest min(L, window) of the sequence's L tokens
  const int total = a.seq_lens ? max(0, min(a.seq_lens[b], a.max_seq_len)) : a.max_seq_len;
  const int len = total - min(total, a.window);
  const int nblk = (len + 31) >> 5;
  const int per = (nblk + a.s_eff - 1) / a.s_eff;
  const int start = sidx * per * 32;
  const int end = min(len, start + per * 32);
  const int last = end - 1;
  const int n16 = lane & 15, q4 = lane >> 4;
  const bool head_ok = n16 < a.G;
  const int h = kvh * a.G + (head_ok ? n16 : 0);

  // ---- rotated query as the score MFMA's B operand: lane (head n16, g = q4) holds
  //      f q'[h][q4*d/4 + 8kb + e] for kb < KB, e < 8, split into bf16 hi + lo, where f is the
  //      score scale (bf16 has fp32's exponent range, so the scale can ride on the operand
  //      and the products come out as scores up to the key's norm). 2/3-bit keys take three
  //      bf16 passes (q_hi c_hi + q_hi c_lo + q_lo c_hi), 4-bit keys two ((c_hi + c_lo) q_hi and
  //      (c_hi + c_lo) q_lo), both ~2^-17 relative: with large logits (outlier tokens) softmax
  //      turns score errors into weight errors, so fp16 (2^-11) operands are not enough there. All waves of the workgroup serve the same
  //      (sequence, KV head); wave 0 leaves the operands in LDS and the loop reads them there.
  //      With 4-bit keys (K1) the operand word c of K block kb holds coordinate
  //      q4*d/4 + 4kb + c twice (the code side supplies hi and lo of that coordinate).
  auto query_operands = [&](const float* src, u32x4* dst, float f, auto dup) {
    constexpr bool DUP = decltype(dup)::value;
    float qv[D / 4];
    const float* qp = src + ((int64_t)b * a.Hq + h) * D + q4 * (D / 4);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) qv[i] = head_ok ? qp[i] : 0.f;
    if constexpr (DUP) {
#pragma unroll
      for (int kb = 0; kb < KB1; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float v = qv[4 * kb + c] * f;
          const uint32_t h = f32_to_bf16_bits(v);
          const uint32_t l = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
          if (wave == 0) {
            ((uint32_t*)&dst[kb * 64 + lane])[c] = h | (h << 16);
            ((uint32_t*)&dst[(KB1 + kb) * 64 + lane])[c] = l | (l << 16);
          }
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float v0 = qv[8 * kb + 2 * c] * f, v1 = qv[8 * kb + 2 * c + 1] * f;
          const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
          const uint32_t l0 = f32_to_bf16_bits(v0 - bf16_bits_to_f32(h0));
          const uint32_t l1 = f32_to_bf16_bits(v1 - bf16_bits_to_f32(h1));
          if (wave == 0) {
            ((uint32_t*)&dst[kb * 64 + lane])[c] = h0 | (h1 << 16);
            ((uint32_t*)&dst[(KB + kb) * 64 + lane])[c] = l0 | (l1 << 16);
          }
        }
    }
  };
  // With G <= 8 (MQ) the score MFMA's 16 columns hold (head, part): column n16 is head n16 % 8's
  // query, its bf16 hi part for n16 < 8 and its lo part for n16 >= 8, so ONE product per K
  // block takes both parts (the 2/3-bit keys' c_lo q_lo term comes along) and a row rotation by
  // 8 lanes adds the two halves. Then lane n16 and lane n16 + 8 both hold head n16 % 8's score;
  // only lanes n16 < G are heads. With G > 8 every column is a head and the parts take
  // separate products.
  constexpr bool merged = MQ;
  auto query_operands_m = [&](const float* src, u32x4* dst, float f, auto dup) {
    constexpr bool DUP = decltype(dup)::value;
    const int hm = n16 & 7;
    const bool ok = hm < a.G, lo = n16 >= 8;
    float qv[D / 4];
    const float* qp = src + ((int64_t)b * a.Hq + kvh * a.G + (ok ? hm : 0)) * D + q4 * (D / 4);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) qv[i] = ok ? qp[i] : 0.f;
    auto part = [&](float v) -> uint32_t {
      const uint32_t hb = f32_to_bf16_bits(v);
      return lo ? f32_to_bf16_bits(v - bf16_bits_to_f32(hb)) : hb;
    };
    if constexpr (DUP) {
#pragma unroll
      for (int kb = 0; kb < KB1; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t w = part(qv[4 * kb + c] * f);
          if (wave == 0) ((uint32_t*)&dst[kb * 64 + lane])[c] = w | (w << 16);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t w0 = part(qv[8 * kb + 2 * c] * f), w1 = part(qv[8 * kb + 2 * c + 1] * f);
          if (wave == 0) ((uint32_t*)&dst[kb * 64 + lane])[c] = w0 | (w1 << 16);
        }
    }
  };
  // head n16 % 8's score from the two halves (lanes n16 and n16 + 8 of each row of 16): one
  // v_add_f32 with a row rotation by 8 on its first source per value. Written as asm because
  // this compiler merged separate row-rotation builtins on the elements of one vector into a
  // single rotation of element 0. The inputs come from ordinary VALU instructions (not straight
  // from an MFMA), and DPP needs two wait states after a VALU write of its source: s_nop 1.
  auto add_halves = [](float (&v)[4]) {
    asm volatile(
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0xf"
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
  };
  float m_run = -INFINITY, l_run = 0.f, n_run = 0.f, n_eff = 1.0f, m_eff = -INFINITY;
  f32x4 acc[TV];
#pragma unroll
  for (int t = 0; t < TV; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- operands of one 32-token block, fetched one block ahead of their use. This lane
  //      needs the K codes of token t0 + 16*tile + n16 (score A operand row n16) and, for the
  //      8 tokens tok(e) = t0 + (e < 4 ? 4*q4 + e : 16 + 4*q4 + e - 4) whose scores land in
  //      it and whose weights it supplies to P.V, their K norms, V norms and V codes. Tokens
  //      past the end are clamped to the last one (and masked later): every load is issued
  //      unconditionally, so the in-order memory counter waits only for what is needed.
  struct KBlk {
    uint32_t kc[2][NWK];
    uint32_t sg[QJL ? 2 : 1][NWS];
  };
  // 2-bit value segments of 16 bits (d = 128) are loaded in pairs into one register:
  // pk[c] = segment of tok(2c) | segment of tok(2c+1) << 16
  constexpr bool VPACK = !SCORES && BV == 2 && NBV == 16;
  struct VBlk {
    uint32_t seg[SCORES || VPACK ? 1 : 8][NWV];
    uint32_t pk[VPACK ? 4 : 1];
  };
  constexpr int NR = QJL ? 2 : 1;   // norm values a lane loads per block
  const int64_t dense_base = ((int64_t)b * a.Hkv + kvh) * a.max_seq_len;
  // Dense caches are addressed from this (sequence, KV head)'s first row with 32-bit offsets
  // (a uniform base plus a per-lane offset needs no 64-bit arithmetic per token); paged pools
  // from their first row with 64-bit rows.
  const int64_t base_row = PAGE == kDense ? dense_base : 0;
  const uint8_t* kp0 = a.kp + base_row * ROWK;
  const uint8_t* vp0 = a.vp + base_row * ROWV;
  const float* kn0 = a.kn + base_row;
  const float* vn0 = a.vn + base_row;
  const uint8_t* ks0 = QJL ? a.ksg + base_row * (D / 8) : nullptr;
  const float* kr0 = QJL ? a.krn + base_row : nullptr;
  using Row = typename std::conditional<PAGE == kDense, uint32_t, int64_t>::type;
  const int32_t* btab = a.block_table + (int64_t)b * a.mbps;
  auto pages = [&](int t0, int& p0, int& p1) {
    if constexpr (PAGE == kPagedPow2) {
      p0 = btab[min(t0, last) >> a.bs_shift];
      p1 = btab[min(t0 + 31, last) >> a.bs_shift];
    } else {
      p0 = p1 = 0;
    }
  };
  auto row_of = [&](int tt, int t0, int p0, int p1) -> Row {
    if constexpr (PAGE == kDense) {
      return (uint32_t)tt;
    } else if constexpr (PAGE == kPagedPow2) {
      const int phys = ((tt >> a.bs_shift) == (t0 >> a.bs_shift)) ? p0 : p1;
      return (((int64_t)phys * a.Hkv + kvh) << a.bs_shift) + (tt & (a.block_size - 1));
    } else {
      const int blk = tt / a.block_size;
      return ((int64_t)btab[blk] * a.Hkv + kvh) * a.block_size + (tt - blk * a.block_size);
    }
  };
  auto tok = [&](int t0, int e) { return min(t0 + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + (e - 4)), last); };
  // dense: buffer resources over this (sequence, KV head)'s `len` compressed rows. Reads past
  // them return 0 (the hardware's range check), so dense fetches need no clamping: a lane's
  // offsets are a fixed part plus t0 * row bytes, and the tokens of one block differ by
  // constants that the loads take as immediate offsets.
  const uint32_t nrows = PAGE == kDense ? (uint32_t)len : 0u;
  const __amdgpu_buffer_rsrc_t r_kp = buffer_rsrc(kp0, nrows * ROWK), r_vp = buffer_rsrc(vp0, nrows * ROWV);
  const __amdgpu_buffer_rsrc_t r_ks = buffer_rsrc(ks0, QJL ? nrows * (D / 8) : 0u);
  auto fetch_k = [&](int t0, int p0, int p1, KBlk& B) {
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      if constexpr (PAGE == kDense) {
        const uint32_t row = (uint32_t)t0 + (uint32_t)n16;
        load_chunk_buf<NBK, ROWK>(r_kp, row * ROWK + 16u * tile * ROWK, q4 * NBK, B.kc[tile]);
        if constexpr (QJL)
          load_chunk_buf<NBS, D / 8>(r_ks, row * (D / 8) + 16u * tile * (D / 8), q4 * NBS, B.sg[tile]);
      } else {
        const int tk = min(t0 + 16 * tile + n16, last);
        const Row row = row_of(tk, t0, p0, p1);
        load_chunk<NBK, ROWK>(kp0 + row * (Row)ROWK, q4 * NBK, B.kc[tile]);
        if constexpr (QJL) load_chunk<NBS, D / 8>(ks0 + row * (Row)(D / 8), q4 * NBS, B.sg[tile]);
      }
    }
  };
  auto fetch_v = [&](int t0, int p0, int p1, VBlk& B) {
    if constexpr (!SCORES) {
      if constexpr (VPACK) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u16x2 v;
          if constexpr (PAGE == kDense) {
            const uint32_t o = ((uint32_t)t0 + 4u * q4) * ROWV + (uint32_t)n16 * 2u;
            v[0] = __builtin_amdgcn_raw_buffer_load_b16(r_vp, o + (uint32_t)(2 * c < 4 ? 2 * c : 12 + 2 * c) * ROWV, 0, 0);
            v[1] = __builtin_amdgcn_raw_buffer_load_b16(r_vp, o + (uint32_t)(2 * c + 1 < 4 ? 2 * c + 1 : 13 + 2 * c) * ROWV, 0, 0);
          } else {
            v[0] = *(const uint16_t*)(vp0 + row_of(tok(t0, 2 * c), t0, p0, p1) * (Row)ROWV + n16 * 2);
            v[1] = *(const uint16_t*)(vp0 + row_of(tok(t0, 2 * c + 1), t0, p0, p1) * (Row)ROWV + n16 * 2);
          }
          B.pk[c] = __builtin_bit_cast(uint32_t, v);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (PAGE == kDense) {
            const uint32_t row = (uint32_t)t0 + 4u * q4;
            load_chunk_buf<NBV, ROWV>(r_vp, row * ROWV + (uint32_t)(e < 4 ? e : 12 + e) * ROWV, n16 * NBV, B.seg[e]);
          } else {
            const Row row = row_of(tok(t0, e), t0, p0, p1);
            load_chunk<NBV, ROWV>(vp0 + row * (Row)ROWV, n16 * NBV, B.seg[e]);
          }
        }
      }
    }
  };
  // The block's norms come in one load per value kind: lane l < 32 reads the K norm of token
  // t0 + l, lane l >= 32 the V norm of token t0 + l - 32 (the K norm again for scores), and
  // with QJL keys every lane the residual norm of token t0 + l % 32. They are staged in LDS
  // and read back as the 8 values of the lane's tokens (two runs of 4 consecutive tokens).
  auto fetch_norms = [&](int t0, int p0, int p1, float (&nr)[NR]) {
    const int tt = min(t0 + (lane & 31), last);
    const Row row = row_of(tt, t0, p0, p1);
    const float* np = (SCORES || lane < 32) ? kn0 : vn0;
    nr[0] = np[row];
    if constexpr (QJL) nr[1] = kr0[row];
  };
  __shared__ f32x4 nstage[kAttnWaves][QJL ? 24 : 16];
  float* const nst = (float*)&nstage[wave][0];

  // The first block's loads go out before the query operands are built, so that their latency
  // and that of the query loads overlap.
  KBlk kA, kB;
  VBlk vA, vB;
  float nA[NR], nB[NR];
  int q0 = 0, q1 = 0;   // pages of the next block to fetch
  if (start < end) {
    pages(start, q0, q1);
    fetch_norms(start, q0, q1, nA);
    fetch_k(start, q0, q1, kA);
    fetch_v(start, q0, q1, vA);
    pages(start + 32, q0, q1);
  }
  // code -> operand tables and query operands, shared by the workgroup's waves
  {
    {
      // centroids straight from the kernel-argument segment (`a` is the only argument)
      const char* ka = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
      const uint32_t* kk = (const uint32_t*)(ka + offsetof(AttnKArgs, ctk));
      const uint32_t* kv = (const uint32_t*)(ka + offsetof(AttnKArgs, ctv));
      constexpr uint32_t MK = (1u << BK) - 1u, MV = (1u << BV) - 1u;
      for (int j = threadIdx.x; j < KTAB; j += blockDim.x) {
        if constexpr (K1) {
          tkh[j] = kk[(j & 1) ? ((j >> 5) & 15) : ((j >> 1) & 15)];   // entry j/2: low code, high code
        } else {
          const uint32_t c0 = kk[j & MK], c1 = kk[j >> BK];
          tkh[j] = (c0 & 0xffffu) | (c1 << 16);
          tkh[KLO / 4 + j] = (c0 >> 16) | (c1 & 0xffff0000u);
        }
      }
      if constexpr (!SCORES) {
        auto cv = [&](uint32_t k) -> uint32_t { return (kv[k >> 1] >> (16 * (k & 1))) & 0xffffu; };
        for (int j = threadIdx.x; j < VTAB; j += blockDim.x) tv[j] = cv(j & MV) | (cv((uint32_t)j >> BV) << 16);
      }
    }
    // the softmax runs in base 2 (v_exp_f32 is 2^x): fused-attention scores are kept in units
    // of log2(e) and the running max is converted back when the partial is written
    constexpr float kSU = SCORES ? 1.0f : 1.4426950408889634f;
    if constexpr (merged) {
      query_operands_m(a.qrot, sq, a.scale * kSU, std::integral_constant<bool, K1>{});
      if constexpr (QJL) query_operands_m(a.qsk, ssq, a.scale * a.qjl_c * kSU, std::false_type{});
    } else {
      query_operands(a.qrot, sq, a.scale * kSU, std::integral_constant<bool, K1>{});
      if constexpr (QJL) query_operands(a.qsk, ssq, a.scale * a.qjl_c * kSU, std::false_type{});
    }
    __syncthreads();
  }

  // Double-buffered walk: at the top of a block every load of the next block (norms, key codes,
  // value codes) is issued into the other buffer set, so each load has a whole block of work to
  // arrive before its first use. The two sets alternate by unrolling the walk by two; copying a
  // prefetch buffer instead would make the wave wait for every load in flight.
  if (start < end) {
    // lanes of heads past the group's G read lane 63's operand, which is zero when G < 16 (and,
    // with merged columns, when G < 8): the reads of those lanes then share one address, which
    // costs LDS almost nothing
    const bool col_ok = merged ? (n16 & 7) < a.G : head_ok;
    uint32_t qoff = (uint32_t)(col_ok ? lane : 63) * 16u;
    auto block = [&](int t0, const KBlk& cur, const VBlk& vb, const float (&nr)[NR], KBlk& kN, VBlk& vN,
                     float (&nN)[NR]) {
      // past the wave's range a dense fetch would read the next wave's rows: the last block
      // fetches itself again instead (cache hits); paged fetches clamp their rows already
      const int nx = (PAGE != kDense || t0 + 32 < end) ? t0 + 32 : t0;
      fetch_norms(nx, q0, q1, nN);
      fetch_k(nx, q0, q1, kN);
      fetch_v(nx, q0, q1, vN);
      pages(t0 + 64, q0, q1);
      // this block's norms through LDS into the lane's 8 tokens
      float kn[8], vn[SCORES ? 1 : 8], rn[QJL ? 8 : 1];
      {
        nst[lane] = nr[0];
        if constexpr (QJL) nst[64 + (lane & 31)] = nr[1];
        const f32x4 a0 = *(const f32x4*)&nst[4 * q4], a1 = *(const f32x4*)&nst[16 + 4 * q4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kn[i] = a0[i];
          kn[4 + i] = a1[i];
        }
        if constexpr (!SCORES) {
          const f32x4 b0 = *(const f32x4*)&nst[32 + 4 * q4], b1 = *(const f32x4*)&nst[48 + 4 * q4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vn[i] = b0[i];
            vn[4 + i] = b1[i];
          }
        }
        if constexpr (QJL) {
          const f32x4 c0 = *(const f32x4*)&nst[64 + 4 * q4], c1 = *(const f32x4*)&nst[80 + 4 * q4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rn[i] = c0[i];
            rn[4 + i] = c1[i];
          }
        }
      }
      // query operands are re-read from LDS each block rather than held in 8*KB registers
      asm volatile("" : "+v"(qoff));
      const char* qbase = (const char*)sq + qoff;
      const char* sbase = (const char*)ssq + qoff;

      // ---- scores of the block's two 16-token tiles
      float s[8];
      f32x4 St[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if constexpr (K1) {
        // codes 4kb .. 4kb+3 of the lane's chunk are bytes 2(kb%2), 2(kb%2)+1 of word kb/2
        auto key_operand = [&](int kb, int tile) -> u32x4 {
          const int sh = 16 * (kb & 1);
          const uint32_t w = cur.kc[tile][kb >> 1];
          const u32x2 p0 = *(const u32x2*)((const char*)tkh + 8u * ((w >> sh) & 0xffu));
          const u32x2 p1 = *(const u32x2*)((const char*)tkh + 8u * ((w >> (sh + 8)) & 0xffu));
          return u32x4{p0[0], p0[1], p1[0], p1[1]};
        };
        if constexpr (merged) {
#pragma unroll
          for (int kb = 0; kb < KB1; ++kb) {
            const u32x4 q = *(const u32x4*)(qbase + kb * 1024);
#pragma unroll
            for (int tile = 0; tile < 2; ++tile) St[tile] = mfma16_bf16(key_operand(kb, tile), q, St[tile]);
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < KB1; ++kb) {
            const u32x4 qh = *(const u32x4*)(qbase + kb * 1024);
            const u32x4 ql = *(const u32x4*)(qbase + (KB1 + kb) * 1024);
#pragma unroll
            for (int tile = 0; tile < 2; ++tile) {
              const u32x4 ak = key_operand(kb, tile);
              St[tile] = mfma16_bf16(ak, qh, St[tile]);
              St[tile] = mfma16_bf16(ak, ql, St[tile]);
            }
          }
        }
      }
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        f32x4 S = St[tile];
        if constexpr (!K1) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            u32x4 akh, akl;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              // byte offset of the code pair's entry: its PK bits shifted to bit 2, one mask
              const int pos = (4 * kb + c) * PK, sb = pos & 31;
              const uint32_t* w = cur.kc[tile];
              uint32_t off;
              if (sb + PK <= 32)
                off = (sb >= 2 ? (w[pos >> 5] >> (sb - 2)) : (w[pos >> 5] << (2 - sb))) & (((1u << PK) - 1u) << 2);
              else
                off = funnel(w[(pos >> 5) + 1], w[pos >> 5], sb - 2) & (((1u << PK) - 1u) << 2);
              akh[c] = lds_word(tkh, off);
              akl[c] = lds_word(tkh, off + KLO);
            }
            const u32x4 qh = *(const u32x4*)(qbase + kb * 1024);
            S = mfma16_bf16(akh, qh, S);
            S = mfma16_bf16(akl, qh, S);
            if constexpr (!merged) {
              const u32x4 ql = *(const u32x4*)(qbase + (KB + kb) * 1024);
              S = mfma16_bf16(akh, ql, S);
            }
          }
        }
        // QJL term: <S q, signs> with the signs as exact bf16 +-1 (bit 1 -> +1) against S q hi + lo
        f32x4 S2 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (QJL) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const uint32_t u = bits_at<8>(cur.sg[tile], 8 * kb);
            u32x4 as;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t w = u >> (2 * c);
              as[c] = 0xBF80BF80u ^ ((w & 1u) << 15) ^ ((w & 2u) << 30);
            }
            const u32x4 sh = *(const u32x4*)(sbase + kb * 1024);
            S2 = mfma16_bf16(as, sh, S2);
            if constexpr (!merged) {
              const u32x4 sl = *(const u32x4*)(sbase + (KB + kb) * 1024);
              S2 = mfma16_bf16(as, sl, S2);
            }
          }
        }
        // D layout: lane (head n16, q4) register r = token t0 + 16*tile + 4*q4 + r = tok(4*tile + r)
        float vt[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          vt[r] = S[r] * kn[4 * tile + r];
          if constexpr (QJL) vt[r] = fmaf(S2[r], rn[4 * tile + r], vt[r]);
        }
        // merged columns: the two halves of a head's (token-scaled) score, both rows of one token
        if constexpr (merged) add_halves(vt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = vt[r];
          if constexpr (SCORES) {
            const int tt = t0 + 16 * tile + 4 * q4 + r;
            const bool ok = tt < end;
            v = ok ? v : -INFINITY;
            float* dst = ok && head_ok ? a.scores + ((int64_t)b * a.Hq + h) * a.max_seq_len + tt : a.sink + lane;
            *dst = v;
          }
          s[4 * tile + r] = v;
        }
      }
      if constexpr (!SCORES) {
        // only a wave's last block can run past its range: mask there (a uniform branch)
        if (t0 + 32 > end) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t0 + 16 * (e >> 2) + 4 * q4 + (e & 3) >= end) s[e] = -INFINITY;
        }
      }
      if constexpr (!SCORES) {
        // ---- online softmax: weights p_t n^v_t / N against a running max m and a running max
        //      V norm N (taken as 1 while it is 0 or subnormal), both shared by the 4 lanes of a head. They
        //      move only when some lane's block exceeds them by a margin (2^8 in the weights, 16x
        //      in the norms): until then the weights stay below 2^12 in fp16 and a block needs no
        //      cross-lane reduction and no rescale. 1/N rides in the exponent: p_t / N =
        //      2^(s_t - m_e) with m_e = m + log2 N, and l gains N * sum 2^(s_t - m_e).
        // NaN-propagating maxima (v_maximum3_f32): fmaxf would first quiet every input that the
        // compiler cannot prove canonical (loaded norms, asm results), one instruction each
        float mb = s[0], nb = vn[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) {
          mb = __builtin_elementwise_maximum(mb, s[e]);
          nb = __builtin_elementwise_maximum(nb, vn[e]);
        }
        if (__any(mb > m_run + 8.0f || nb > 16.0f * n_run)) {
          mb = fmaxf(mb, wave_xor(mb, 16));
          mb = fmaxf(mb, wave_xor(mb, 32));
          nb = fmaxf(nb, wave_xor(nb, 16));
          nb = fmaxf(nb, wave_xor(nb, 32));
          const float m_new = fmaxf(m_run, mb);
          const float n_new = fmaxf(n_run, nb);
          const float ne_new = n_new >= 1.17549435e-38f ? n_new : 1.0f;   // 0 (or subnormal): 1
          const float al = exp2_fast(m_run - m_new);
          const float a_acc = al * n_eff / ne_new;
          l_run *= al;
          m_run = m_new;
          n_run = n_new;
          n_eff = ne_new;
          m_eff = m_new + __builtin_amdgcn_logf(ne_new);   // v_log_f32 is log2
          if (__any(a_acc != 1.0f)) {
#pragma unroll
            for (int t = 0; t < TV; ++t) acc[t] = acc[t] * a_acc;
          }
        }
        float lsum = 0.f;
        u32x4 bw;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float e0 = exp2_fast(s[2 * c] - m_eff), e1 = exp2_fast(s[2 * c + 1] - m_eff);
          lsum += e0 + e1;
          bw[c] = pack_f16x2(e0 * vn[2 * c], e1 * vn[2 * c + 1]);
        }
        l_run = fmaf(lsum, n_eff, l_run);

        // ---- P.V: lane (coordinate group m = n16, token group g = q4), same 8 tokens; tile t
        //      is coordinate m*d/16 + t, component c the tokens tok(2c), tok(2c+1)
        if constexpr (BV == 2) {
#pragma unroll
          for (int ch = 0; ch < (NBV + 15) / 16; ++ch) {   // 8 codes = 8 tiles per 16-bit chunk
            // nibble t of z[c] = the codes of tokens tok(2c), tok(2c+1) for coordinate 8ch + t;
            // ze / zo carry the table offsets of the even / odd nibbles in their bytes
            uint32_t ze[4], zo[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              uint32_t z;
              if constexpr (VPACK)
                z = interleave2_packed(vb.pk[c]);
              else
                z = interleave2((vb.seg[2 * c][0] >> (16 * ch)) & 0xffffu, (vb.seg[2 * c + 1][0] >> (16 * ch)) & 0xffffu);
              ze[c] = (z << 2) & 0x3c3c3c3cu;
              zo[c] = (z >> 2) & 0x3c3c3c3cu;
              asm("" : "+v"(ze[c]), "+v"(zo[c]));
            }
#pragma unroll
            for (int j = 0; j < 4 && 8 * ch + 2 * j < TV; ++j) {
              u32x4 av0, av1;
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                av0[c] = lds_word(tv, (ze[c] >> (8 * j)) & 0xffu);
                av1[c] = lds_word(tv, (zo[c] >> (8 * j)) & 0xffu);
              }
              acc[8 * ch + 2 * j] = mfma16_f16(av0, bw, acc[8 * ch + 2 * j]);
              acc[8 * ch + 2 * j + 1] = mfma16_f16(av1, bw, acc[8 * ch + 2 * j + 1]);
            }
          }
        } else {
#pragma unroll
          for (int t = 0; t < TV; ++t) {
            u32x4 av;
#pragma unroll
            for (int c = 0; c < 4; ++c)
              av[c] = tv[bits_at<BV>(vb.seg[2 * c], BV * t) | (bits_at<BV>(vb.seg[2 * c + 1], BV * t) << BV)];
            acc[t] = mfma16_f16(av, bw, acc[t]);
          }
        }
      }
    };
    wait_vmem_all();
    // Waves sharing a SIMD otherwise progress at very different speeds (the oldest wave is
    // issued first), and the SIMD runs its last blocks with fewer and fewer waves. When the
    // whole grid is resident, a wave lowers its issue priority as it passes half and then three
    // quarters of its range, so the others catch up and all finish close together.
    const bool prio = !SCORES && a.one_round;
    const int t_half = start + (end - start) / 2, t_3q = start + 3 * (end - start) / 4;
    int lvl = 0;   // 0: priority 3, 1: past half (priority 1), 2: past three quarters (0)
    if (prio) __builtin_amdgcn_s_setprio(3);
    for (int t0 = start;;) {
      if (prio) {
        if (lvl < 2 && t0 >= t_3q) {
          lvl = 2;
          __builtin_amdgcn_s_setprio(0);
        } else if (lvl < 1 && t0 >= t_half) {
          lvl = 1;
          __builtin_amdgcn_s_setprio(1);
        }
      }
      block(t0, kA, vA, nA, kB, vB, nB);
      if ((t0 += 32) >= end) break;
      block(t0, kB, vB, nB, kA, vA, nA);
      if ((t0 += 32) >= end) break;
    }
    if (prio) __builtin_amdgcn_s_setprio(0);
  }

  if constexpr (!SCORES) {
    // this wave's partial (m in natural-log units, l, acc relative to e^m); lane (head n16, q4)
    // holds the coordinate groups 4*q4 + r (register r of the P.V MFMA's D layout)
    float lt = l_run;
    lt += wave_xor(lt, 16);
    lt += wave_xor(lt, 32);
    float mw = m_run * 0.6931471805599453f;   // back to natural-log units
    float av[4 * TV];
#pragma unroll
    for (int t = 0; t < TV; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r * TV + t] = acc[t][r] * n_eff;
    // The workgroup's four waves cover adjacent token ranges of one (sequence, KV head): their
    // partials are combined here through LDS (waves 2, 3 into 0, 1, then 1 into 0), so one
    // partial per workgroup goes to the merge. Each lane meets the same lane of the other waves,
    // which holds the same heads and coordinates.
    constexpr int CW = 4 * TV + 3;   // floats per lane slot (odd stride: no bank conflicts)
    __shared__ float cmb[2][64][CW];
    auto put = [&](float* sl) {
      sl[0] = mw;
      sl[1] = lt;
#pragma unroll
      for (int i = 0; i < 4 * TV; ++i) sl[2 + i] = av[i];
    };
    auto take = [&](const float* sl) {
      const float m2 = sl[0];
      const float M = fmaxf(mw, m2);
      if (M > -INFINITY) {
        const float w1 = __expf(mw - M), w2 = __expf(m2 - M);   // a -inf side weighs 0
        lt = lt * w1 + sl[1] * w2;
#pragma unroll
        for (int i = 0; i < 4 * TV; ++i) av[i] = av[i] * w1 + sl[2 + i] * w2;
        mw = M;
      }
    };
    if (wave >= 2) put(&cmb[wave - 2][lane][0]);
    __syncthreads();
    if (wave < 2) take(&cmb[wave][lane][0]);
    __syncthreads();
    if (wave == 1) put(&cmb[0][lane][0]);
    __syncthreads();
    if (wave == 0) {
      take(&cmb[0][lane][0]);
      if (head_ok) {
        float* P = a.part + (((int64_t)blockIdx.x * a.B + b) * a.Hq + h) * (D + 2);
        if (q4 == 0) {
          P[0] = mw;
          P[1] = lt;
        }
#pragma unroll
        for (int t = 0; t < TV; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) P[2 + (4 * q4 + r) * (D / 16) + t] = av[r * TV + t];
      }
    }
  }
}

// ---- recent-token window (KV Cache API page, TurboQuantKVCache.attention_scores / attend: the
//      buffered newest tokens are scored exactly and their values added at full precision).
// One workgroup per (sequence, KV head) computes the window's split partial (m, l, acc[d]) for
// the group's query heads, in the original (unrotated) value domain, into the split slot after
// the compressed ones; the merge adds it beside the rotated-back compressed accumulator.
// Token at absolute position t sits at ring slot t mod R. Chunks of kWinChunk tokens: thread i
// scores token i of the chunk against every head (queries in LDS), then an online softmax per
// head, then thread k accumulates coordinate k over the chunk.
struct WinKArgs {
  const void* q;
  const void* kw;
  const void* vw;
  const int32_t* seq_lens;
  float* part;
  int32_t q_dtype, w_dtype, window, max_seq_len;
  int32_t B, Hq, Hkv, G, slot;   // slot: the split index the window partial is written to
  float scale;
};

constexpr int kWinChunk = 256;

__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dt) {
  if (dt == TQ_F32) return ((const float*)p)[i];
  const uint32_t bits = ((const uint16_t*)p)[i];
  return dt == TQ_BF16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
}

// One 16-byte piece of a full-precision row as floats (4 float32 or 8 bfloat16 / float16).
template <int WDT>
struct WinPiece {
  static constexpr int PER = WDT == TQ_F32 ? 4 : 8;
  static constexpr int ESZ = WDT == TQ_F32 ? 4 : 2;
};
template <int WDT>
__device__ __forceinline__ void unpack_piece(const u32x4& p, float (&f)[WinPiece<WDT>::PER]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (WDT == TQ_F32) {
      f[c] = __uint_as_float(p[c]);
    } else if constexpr (WDT == TQ_BF16) {
      f[2 * c] = bf16_lo_to_f32(p[c]);
      f[2 * c + 1] = bf16_hi_to_f32(p[c]);
    } else {
      f[2 * c] = f16_bits_to_f32(p[c]);
      f[2 * c + 1] = f16_bits_to_f32(p[c] >> 16);
    }
  }
}

template <int WDT>
__device__ __forceinline__ float win_elem(const void* p, int64_t i) {
  if constexpr (WDT == TQ_F32) {
    return ((const float*)p)[i];
  } else {
    const uint32_t bits = ((const uint16_t*)p)[i];
    return WDT == TQ_BF16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
  }
}

// GC = the head count G rounded up to 4, 8 or 16: every per-head loop runs GC times without a
// branch (heads >= G get a zero query and are never written), so the loads of a loop can all
// be in flight together.
template <int D, int WDT, int GC>
__global__ void __launch_bounds__(kWinChunk) window_kernel(WinKArgs a) {
  constexpr int NP = kWinChunk / D;   // token parts in the value phase (D <= kWinChunk)
  constexpr int PER = WinPiece<WDT>::PER, ESZ = WinPiece<WDT>::ESZ;
  constexpr int NPIECE = D / PER;     // 16-byte pieces of a row
  __shared__ f32x4 qs[D][GC / 4];     // query coordinate k of head g at qs[k][g / 4][g % 4]
  __shared__ f32x4 ps[kWinChunk][GC / 4];   // softmax weight of chunk token i for head g
  __shared__ float red[GC][kWinChunk / 64];
  __shared__ float mrun[GC], lrun[GC], alpha[GC];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = a.G, R = a.window;
  const int total = a.seq_lens ? max(0, min(a.seq_lens[b], a.max_seq_len)) : a.max_seq_len;
  const int w = min(total, R), c = total - w;
  for (int i = tid; i < GC * D; i += blockDim.x) {
    const int g = i / D, k = i - g * D;
    ((float*)&qs[k][0])[g] = g < G ? load_elem(a.q, ((int64_t)b * a.Hq + kvh * G + g) * D + k, a.q_dtype) : 0.f;
  }
  if (tid < GC) {
    mrun[tid] = -INFINITY;
    lrun[tid] = 0.f;
  }
  float acc[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) acc[g] = 0.f;
  __syncthreads();
  const int64_t ring = ((int64_t)b * a.Hkv + kvh) * R;   // first row of this head's ring
  for (int i0 = 0; i0 < w; i0 += kWinChunk) {
    const int n = min(kWinChunk, w - i0);
    // scores of token i0 + tid against every head, the key row read piece by piece
    float s[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) s[g] = 0.f;
    if (tid < n) {
      const int64_t row = ring + (c + i0 + tid) % R;
      const u32x4* kr = (const u32x4*)((const uint8_t*)a.kw + row * D * ESZ);
#pragma unroll 4
      for (int j = 0; j < NPIECE; ++j) {
        float f[PER];
        unpack_piece<WDT>(kr[j], f);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
#pragma unroll
          for (int g4 = 0; g4 < GC / 4; ++g4) {
            const f32x4 qv = qs[j * PER + e][g4];
#pragma unroll
            for (int r = 0; r < 4; ++r) s[4 * g4 + r] = fmaf(f[e], qv[r], s[4 * g4 + r]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GC; ++g) s[g] = tid < n ? s[g] * a.scale : -INFINITY;
    // chunk max per head
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float m = s[g];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, wave_xor(m, o));
      if (lane == 0) red[g][wv] = m;
    }
    __syncthreads();
    if (tid < GC) {
      float m = red[tid][0];
      for (int j = 1; j < kWinChunk / 64; ++j) m = fmaxf(m, red[tid][j]);
      const float mn = fmaxf(mrun[tid], m);
      alpha[tid] = mn == -INFINITY ? 1.f : __expf(mrun[tid] - mn);   // 0 when mrun is -inf
      mrun[tid] = mn;
    }
    __syncthreads();
    {
      float pw[GC];
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        pw[g] = tid < n ? __expf(s[g] - mrun[g]) : 0.f;
        float l = pw[g];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) l += wave_xor(l, o);
        if (lane == 0) red[g][wv] = l;
      }
#pragma unroll
      for (int g4 = 0; g4 < GC / 4; ++g4) ps[tid][g4] = f32x4{pw[4 * g4], pw[4 * g4 + 1], pw[4 * g4 + 2], pw[4 * g4 + 3]};
    }
    __syncthreads();   // the chunk's weights and per-wave sums are visible from here
    if (tid < GC) {
      float l = 0.f;
      for (int j = 0; j < kWinChunk / 64; ++j) l += red[tid][j];
      lrun[tid] = lrun[tid] * alpha[tid] + l;
    }
    // values: thread (k = tid % D, part = tid / D) accumulates coordinate k over the chunk's
    // tokens i = part, part + NP, ...; the parts are summed once at the end
#pragma unroll
    for (int g = 0; g < GC; ++g) acc[g] *= alpha[g];
    {
      const int k = tid % D, part = tid / D;
      int pos = (c + i0 + part) % R;
#pragma unroll 8
      for (int i = part; i < n; i += NP) {
        const float vv = win_elem<WDT>(a.vw, (ring + pos) * D + k);
        pos += NP;
        if (pos >= R) pos -= R;
#pragma unroll
        for (int g4 = 0; g4 < GC / 4; ++g4) {
          const f32x4 pv = ps[i][g4];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[4 * g4 + r] = fmaf(pv[r], vv, acc[4 * g4 + r]);
        }
      }
    }
    __syncthreads();
  }
  // sum the parts: part 0 threads collect the others through LDS (reusing ps)
  float* red2 = (float*)&ps[0][0];   // needs (NP - 1) * G * D floats <= kWinChunk * GC
  const int k = tid % D, part = tid / D;
  if (part > 0)
    for (int g = 0; g < G; ++g) red2[((part - 1) * G + g) * D + k] = acc[g];
  __syncthreads();
  if (part == 0) {
    for (int g = 0; g < G; ++g) {
      float v = acc[g];
      for (int pp = 1; pp < NP; ++pp) v += red2[((pp - 1) * G + g) * D + k];
      float* P = a.part + (((int64_t)a.slot * a.B + b) * a.Hq + kvh * G + g) * (D + 2);
      if (k == 0) {
        P[0] = mrun[g];
        P[1] = lrun[g];
      }
      P[2 + k] = v;
    }
  }
}

template <int D, int WDT>
static void launch_window(const WinKArgs& w, dim3 grid, hipStream_t st) {
  if (w.G <= 4)
    hipLaunchKernelGGL((window_kernel<D, WDT, 4>), grid, dim3(kWinChunk), 0, st, w);
  else if (w.G <= 8)
    hipLaunchKernelGGL((window_kernel<D, WDT, 8>), grid, dim3(kWinChunk), 0, st, w);
  else
    hipLaunchKernelGGL((window_kernel<D, WDT, 16>), grid, dim3(kWinChunk), 0, st, w);
}

// qrot_kernel / merge_kernel: HB query heads of one sequence per block, thread (k, part) owning
// coordinate k over 1/P of a length-D (or length-s_eff) sum, so that its chain of dependent
// loads is P times shorter; the parts meet in LDS. Every block reads the whole rotation (64 KiB
// at d = 128, from L2), so with many heads (batched decode) a block takes HB = 2 heads with
// P = 4 parts (measured: 1 and 4 heads per block were slower there), and with few (one sequence
// with many splits) one head with P = 1024 / D parts: there each block's load latency is the
// whole cost.
constexpr int kPartsMany = 4, kHeadsMany = 2;
template <int D>
constexpr int parts_few() { return 1024 / D; }
inline bool few_heads(int B, int Hq) { return (int64_t)B * Hq < 512; }

// q' = Pi_K q for HB query heads of one sequence (block (b, head group)). Thread (k, part) owns
// output coordinate k over the rows j of its part, reading Pi_K^T row by row (coalesced across
// k); the queries sit in LDS.
template <int D, int P, int HB>
__global__ void __launch_bounds__(D * P) qrot_kernel(const void* q, int q_dtype, const float* pikt,
                                                     int64_t rot_stride, int Hq, int bpr, float* out) {
  constexpr int JP = D / P;
  __shared__ float qs[HB][D];
  __shared__ float red[P][HB][D];
  const int b = blockIdx.x, h0 = blockIdx.y * HB;
  const int nh = min(HB, Hq - h0);
  const int k = threadIdx.x % D, part = threadIdx.x / D;
  const int r = bpr ? b / bpr : 0;
  // this thread's rows of Pi_K^T first, so that their latency overlaps the queries'
  const float* PT = pikt + r * rot_stride + (int64_t)part * JP * D + k;   // PT[j*D] = Pi[k][part*JP + j]
  float pv[JP];
#pragma unroll
  for (int j = 0; j < JP; ++j) pv[j] = PT[(int64_t)j * D];
  for (int i = threadIdx.x; i < HB * D; i += D * P) {
    const int h = i / D, kk = i - h * D;
    float v = 0.f;
    if (h < nh) {
      const int64_t idx = ((int64_t)b * Hq + h0 + h) * D + kk;
      if (q_dtype == TQ_F32)
        v = ((const float*)q)[idx];
      else if (q_dtype == TQ_BF16)
        v = bf16_bits_to_f32(((const uint16_t*)q)[idx]);
      else
        v = f16_bits_to_f32(((const uint16_t*)q)[idx]);
    }
    qs[h][kk] = v;
  }
  __syncthreads();
  float acc[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) acc[h] = 0.f;
#pragma unroll
  for (int j = 0; j < JP; ++j)
#pragma unroll
    for (int h = 0; h < HB; ++h) acc[h] = fmaf(pv[j], qs[h][part * JP + j], acc[h]);
#pragma unroll
  for (int h = 0; h < HB; ++h) red[part][h][k] = acc[h];
  __syncthreads();
  if (part == 0) {
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      if (h >= nh) continue;
      float v = red[0][h][k];
#pragma unroll
      for (int pp = 1; pp < P; ++pp) v += red[pp][h][k];
      out[((int64_t)b * Hq + h0 + h) * D + k] = v;
    }
  }
}

// Log-sum-exp merge of the token splits for HB query heads of one sequence, then
// o = Pi_V^T (sum_s acc_s e^(m_s - M)) / L (+ the window's partial, already unrotated).
// Thread (k, part) owns coordinate k over splits s = part, part + P, ... and over the rows of
// its part in the final product. The split maxima are read once, for M, and kept in LDS (when
// they fit), so the sum pass issues its loads without waiting for them.
template <int D, int OUT, int P, int HB>
__global__ void __launch_bounds__(D * P) merge_kernel(const float* part, int s_eff, int has_window, int B, int Hq,
                                                      int bpr, const float* piv, int64_t rot_stride, void* out,
                                                      float* lse) {
  constexpr int JP = D / P, NT = D * P, NW = NT / 64;
  constexpr int MS = 2048 / HB;              // split maxima kept in LDS per head
  __shared__ float msplit[HB][MS];
  __shared__ float orot[HB][D];
  __shared__ float red[P][HB][D];
  __shared__ float redm[HB][NW];
  __shared__ float lred[P][HB];
  __shared__ float Msh[HB], Lsh[HB];
  const int b = blockIdx.x, h0 = blockIdx.y * HB;
  const int nh = min(HB, Hq - h0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int k = tid % D, pt = tid / D;
  const int64_t sstride = (int64_t)B * Hq * (D + 2);
  const float* P0 = part + ((int64_t)b * Hq + h0) * (D + 2);   // split s, head h: + s*sstride + h*(D+2)
  const int ns = s_eff + has_window;
  // this thread's rows of Pi_V for the final product, loaded first so that their latency
  // overlaps the reads of the partials: pvr[j] = Pi[pt*JP + j][k]
  const float* Pv = piv + (bpr ? b / bpr : 0) * rot_stride + (int64_t)pt * JP * D + k;
  float pvr[JP];
#pragma unroll
  for (int j = 0; j < JP; ++j) pvr[j] = Pv[(int64_t)j * D];

  // M_h = max over splits (and the window) of m_s
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    float m = -INFINITY;
    if (h < nh)
      for (int s = tid; s < ns; s += NT) {
        const float v = P0[(int64_t)s * sstride + h * (D + 2)];
        if (s < MS) msplit[h][s] = v;
        m = fmaxf(m, v);
      }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, wave_xor(m, o));
    if (lane == 0) redm[h][wv] = m;
  }
  __syncthreads();
  if (tid < HB) {
    float mm = redm[tid][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, redm[tid][w]);
    Msh[tid] = mm;
  }
  __syncthreads();

  // this part's splits
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    float acc = 0.f, lsum = 0.f;
    const float M = Msh[h];
    if (h < nh && M > -INFINITY) {
#pragma unroll 8
      for (int s = pt; s < s_eff; s += P) {
        const float* Ps = P0 + (int64_t)s * sstride + h * (D + 2);
        const float ms = s < MS ? msplit[h][s] : Ps[0];
        const float w = ms > -INFINITY ? __expf(ms - M) : 0.f;
        lsum = fmaf(w, Ps[1], lsum);
        acc = fmaf(w, Ps[2 + k], acc);
      }
    }
    red[pt][h][k] = acc;
    if (k == 0) lred[pt][h] = lsum;
  }
  __syncthreads();
  if (tid < HB) {
    float l = 0.f;
#pragma unroll
    for (int pp = 0; pp < P; ++pp) l += lred[pp][tid];
    // the window's partial joins the normalizer here and the output after the rotation back
    if (has_window && tid < nh && Msh[tid] > -INFINITY) {
      const float* Pw = P0 + (int64_t)s_eff * sstride + tid * (D + 2);
      const float ms = Pw[0];
      if (ms > -INFINITY) l = fmaf(__expf(ms - Msh[tid]), Pw[1], l);
    }
    Lsh[tid] = l;
  }
  __syncthreads();
  if (pt == 0) {
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      float v = red[0][h][k];
#pragma unroll
      for (int pp = 1; pp < P; ++pp) v += red[pp][h][k];
      orot[h][k] = Lsh[h] > 0.f ? v / Lsh[h] : 0.f;
    }
  }
  __syncthreads();

  // o = Pi_V^T orot, this part's rows
  float o[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) o[h] = 0.f;
#pragma unroll
  for (int j = 0; j < JP; ++j)
#pragma unroll
    for (int h = 0; h < HB; ++h) o[h] = fmaf(pvr[j], orot[h][pt * JP + j], o[h]);
#pragma unroll
  for (int h = 0; h < HB; ++h) red[pt][h][k] = o[h];
  __syncthreads();
  if (pt == 0) {
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      if (h >= nh) continue;
      float v = red[0][h][k];
#pragma unroll
      for (int pp = 1; pp < P; ++pp) v += red[pp][h][k];
      const float L = Lsh[h], M = Msh[h];
      if (has_window && L > 0.f && M > -INFINITY) {
        const float* Pw = P0 + (int64_t)s_eff * sstride + h * (D + 2);
        const float ms = Pw[0];
        if (ms > -INFINITY) v += __expf(ms - M) * Pw[2 + k] / L;
      }
      const int64_t idx = ((int64_t)b * Hq + h0 + h) * D + k;
      if constexpr (OUT == TQ_F32)
        ((float*)out)[idx] = v;
      else if constexpr (OUT == TQ_BF16)
        ((uint16_t*)out)[idx] = (uint16_t)f32_to_bf16_bits(v);
      else
        ((uint16_t*)out)[idx] = (uint16_t)f32_to_f16_bits(v);
      if (k == 0 && lse) lse[(int64_t)b * Hq + h0 + h] = L > 0.f ? M + logf(L) : -INFINITY;
    }
  }
}

template <int D, int P, int HB>
static void launch_qrot(const tq_attn_params* p, const float* pikt, int64_t rs, float* dst, hipStream_t st) {
  const unsigned hb = (unsigned)((p->num_q_heads + HB - 1) / HB);
  hipLaunchKernelGGL((qrot_kernel<D, P, HB>), dim3(p->batch, hb), dim3(D * P), 0, st, p->q, p->q_dtype, pikt, rs,
                     p->num_q_heads, p->batch_per_rot, dst);
}
template <int D>
static void launch_qrot_any(const tq_attn_params* p, const float* pikt, int64_t rs, float* dst, hipStream_t st) {
  if (few_heads(p->batch, p->num_q_heads))
    launch_qrot<D, parts_few<D>(), 1>(p, pikt, rs, dst, st);
  else
    launch_qrot<D, kPartsMany, kHeadsMany>(p, pikt, rs, dst, st);
}

template <int D, int OUT, int P, int HB>
static void launch_merge(const tq_attn_params* p, const float* part, int s_eff, int has_win, const float* piv,
                         int64_t rs, hipStream_t st) {
  const unsigned hb = (unsigned)((p->num_q_heads + HB - 1) / HB);
  hipLaunchKernelGGL((merge_kernel<D, OUT, P, HB>), dim3(p->batch, hb), dim3(D * P), 0, st, part, s_eff, has_win,
                     p->batch, p->num_q_heads, p->batch_per_rot, piv, rs, p->out, p->lse);
}
template <int D, int OUT>
static void launch_merge_p(const tq_attn_params* p, const float* part, int s_eff, int has_win, const float* piv,
                           int64_t rs, hipStream_t st) {
  if (few_heads(p->batch, p->num_q_heads))
    launch_merge<D, OUT, parts_few<D>(), 1>(p, part, s_eff, has_win, piv, rs, st);
  else
    launch_merge<D, OUT, kPartsMany, kHeadsMany>(p, part, s_eff, has_win, piv, rs, st);
}

// Resident waves per CU of the fused-attention kernel instance (registers and LDS as compiled),
// from the runtime's occupancy calculator, once per (instance, device). The split count sizes the
// grid to one round of them.
template <int D, int BK, int BV, int PAGE, bool QJL, bool MQ>
static int attn_resident_waves_t(int device) {
  static std::mutex mu;
  static int cached[64] = {0};
  std::lock_guard<std::mutex> lk(mu);
  if (device >= 0 && device < 64 && cached[device]) return cached[device];
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, (const void*)attn_kernel<D, BK, BV, false, PAGE, QJL, MQ>,
                                                   kAttnWaves * 64, 0) != hipSuccess ||
      blocks <= 0)
    blocks = attn_wpe(D, BK, BV, QJL, PAGE != kDense);   // the build's target: wpe waves per SIMD
  const int w = blocks * kAttnWaves;
  if (device >= 0 && device < 64) cached[device] = w;
  return w;
}

template <int D, int BK, int BV, bool QJL>
static int attn_resident_p(const tq_attn_params* p, int device) {
  // query parts in the score MFMA's columns (MQ) when a KV head serves at most 8 query heads
  if (p->num_q_heads <= 8 * p->num_kv_heads) {
    if (!p->block_table) return attn_resident_waves_t<D, BK, BV, kDense, QJL, true>(device);
    const int bs = p->block_size;
    if (bs >= 16 && (bs & (bs - 1)) == 0) return attn_resident_waves_t<D, BK, BV, kPagedPow2, QJL, true>(device);
    return attn_resident_waves_t<D, BK, BV, kPagedAny, QJL, true>(device);
  }
  if (!p->block_table) return attn_resident_waves_t<D, BK, BV, kDense, QJL, false>(device);
  const int bs = p->block_size;
  if (bs >= 16 && (bs & (bs - 1)) == 0) return attn_resident_waves_t<D, BK, BV, kPagedPow2, QJL, false>(device);
  return attn_resident_waves_t<D, BK, BV, kPagedAny, QJL, false>(device);
}

template <int D, bool QJL>
static int attn_resident(const tq_attn_params* p, int bk, int bv, int device) {
  auto by_bv = [&](auto kb) -> int {
    constexpr int BK = decltype(kb)::value;
    switch (bv) {
      case 2: return attn_resident_p<D, BK, 2, QJL>(p, device);
      case 3: return attn_resident_p<D, BK, 3, QJL>(p, device);
      default: return attn_resident_p<D, BK, 4, QJL>(p, device);
    }
  };
  switch (bk) {
    case 1:
      if constexpr (QJL) return by_bv(std::integral_constant<int, 1>{});
      return kAttnWaves;
    case 2: return by_bv(std::integral_constant<int, 2>{});
    case 3: return by_bv(std::integral_constant<int, 3>{});
    default: return by_bv(std::integral_constant<int, 4>{});
  }
}

template <int D, int BK, int BV, int PAGE, bool QJL>
static hipError_t launch_attn_p(const tq_attn_params* p, const Codebook& ck, const Codebook& cv, const Rotation& rk,
                                const Rotation& rv, float* scores, bool scores_only, const AttnLayout& lay,
                                hipStream_t st) {
  uint8_t* ws = (uint8_t*)p->workspace;
  float* qrot = (float*)(ws + lay.qrot_off);
  const int Hq = p->num_q_heads, B = p->batch;
  launch_qrot_any<D>(p, rk.f32t(0), (int64_t)(rk.f32_stride / sizeof(float)), qrot, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* qsk = (float*)(ws + lay.qsk_off);
  if constexpr (QJL) {
    // S q: the same product with S^T in place of Pi^T
    const Qjl& qj = p->qjl_k->q;
    launch_qrot_any<D>(p, qj.st(0), (int64_t)(qj.st_stride / sizeof(float)), qsk, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p->max_seq_len == 0 && scores_only) return hipSuccess;

  AttnKArgs a;
  a.qrot = qrot;
  a.kp = p->k_packed;
  a.kn = p->k_norms;
  a.vp = scores_only ? p->k_packed : p->v_packed;
  a.vn = scores_only ? p->k_norms : p->v_norms;
  a.seq_lens = p->seq_lens;
  a.block_table = p->block_table;
  a.scores = scores;
  a.part = (float*)(ws + lay.part_off);
  a.sink = (float*)rk.sink();
  a.max_seq_len = p->max_seq_len;
  a.block_size = p->block_table ? p->block_size : 1;
  a.bs_shift = -1;
  if (p->block_table && (p->block_size & (p->block_size - 1)) == 0) {
    int s = 0;
    while ((1 << s) < p->block_size) ++s;
    a.bs_shift = s;
  }
  a.mbps = p->max_blocks_per_seq;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = p->num_kv_heads;
  a.G = Hq / p->num_kv_heads;
  a.s_eff = lay.splits * kAttnWaves;
  a.window = p->window;
  {
    const int64_t waves = (int64_t)lay.splits * kAttnWaves * p->num_kv_heads * B;
    const int rw = a.G <= 8 ? attn_resident_waves_t<D, BK, BV, PAGE, QJL, true>(rk.device)
                            : attn_resident_waves_t<D, BK, BV, PAGE, QJL, false>(rk.device);
    const int64_t resident = (int64_t)rw * device_cu_count(rk.device);
    a.one_round = waves <= resident ? 1 : 0;
  }
  a.scale = p->scale;
  LevelArgs lk = make_levels(ck), lv = make_levels(cv);
  for (int j = 0; j < 16; ++j) a.ctk[j] = lk.centroid_bf16x2[j];
  for (int j = 0; j < 8; ++j)
    a.ctv[j] = (uint32_t)lv.centroid_f16[2 * j] | ((uint32_t)lv.centroid_f16[2 * j + 1] << 16);
  a.ksg = p->k_signs;
  a.krn = p->k_rnorms;
  a.qsk = qsk;
  a.qjl_c = (float)(std::sqrt(M_PI / 2.0) / D);
  dim3 grid((unsigned)lay.splits, (unsigned)p->num_kv_heads, (unsigned)B);
  auto launch = [&](auto sc) {
    constexpr bool SC = decltype(sc)::value;
    if (a.G <= 8)
      hipLaunchKernelGGL((attn_kernel<D, BK, BV, SC, PAGE, QJL, true>), grid, dim3(kAttnWaves * 64), 0, st, a);
    else
      hipLaunchKernelGGL((attn_kernel<D, BK, BV, SC, PAGE, QJL, false>), grid, dim3(kAttnWaves * 64), 0, st, a);
  };
  if (scores_only) {
    launch(std::true_type{});
    return hipGetLastError();
  }
  launch(std::false_type{});
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int has_win = p->window > 0 ? 1 : 0;
  if (has_win) {
    WinKArgs w;
    w.q = p->q;
    w.kw = p->k_window;
    w.vw = p->v_window;
    w.seq_lens = p->seq_lens;
    w.part = a.part;
    w.q_dtype = p->q_dtype;
    w.w_dtype = p->window_dtype;
    w.window = p->window;
    w.max_seq_len = p->max_seq_len;
    w.B = B;
    w.Hq = Hq;
    w.Hkv = p->num_kv_heads;
    w.G = a.G;
    w.slot = lay.splits;
    w.scale = p->scale;
    const dim3 wg((unsigned)p->num_kv_heads, (unsigned)B);
    if (p->window_dtype == TQ_F32)
      launch_window<D, TQ_F32>(w, wg, st);
    else if (p->window_dtype == TQ_BF16)
      launch_window<D, TQ_BF16>(w, wg, st);
    else
      launch_window<D, TQ_F16>(w, wg, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t rs = (int64_t)(rv.f32_stride / sizeof(float));
  switch (p->out_dtype) {
    case TQ_F32: launch_merge_p<D, TQ_F32>(p, a.part, lay.splits, has_win, rv.f32(0), rs, st); break;
    case TQ_BF16: launch_merge_p<D, TQ_BF16>(p, a.part, lay.splits, has_win, rv.f32(0), rs, st); break;
    default: launch_merge_p<D, TQ_F16>(p, a.part, lay.splits, has_win, rv.f32(0), rs, st);
  }
  return hipGetLastError();
}

template <int D, int BK, int BV, bool QJL>
static hipError_t launch_attn_t(const tq_attn_params* p, const Codebook& ck, const Codebook& cv, const Rotation& rk,
                                const Rotation& rv, float* scores, bool so, const AttnLayout& lay, hipStream_t st) {
  if (!p->block_table) return launch_attn_p<D, BK, BV, kDense, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
  const int bs = p->block_size;
  if (bs >= 16 && (bs & (bs - 1)) == 0) return launch_attn_p<D, BK, BV, kPagedPow2, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
  return launch_attn_p<D, BK, BV, kPagedAny, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
}

template <int D, int BK, bool QJL>
static hipError_t attn_bv(const tq_attn_params* p, const Codebook& ck, const Codebook& cv, const Rotation& rk,
                          const Rotation& rv, float* scores, bool so, const AttnLayout& lay, hipStream_t st) {
  // scores-only calls use the K width for the (unused) V side to avoid extra instances
  const int bv = so ? BK : cv.bits;
  switch (bv) {
    case 2: return launch_attn_t<D, BK, 2, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
    case 3: return launch_attn_t<D, BK, 3, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
    default: return launch_attn_t<D, BK, 4, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
  }
}

template <int D, bool QJL>
static hipError_t attn_bk(const tq_attn_params* p, const Codebook& ck, const Codebook& cv, const Rotation& rk,
                          const Rotation& rv, float* scores, bool so, const AttnLayout& lay, hipStream_t st) {
  switch (ck.bits) {
    case 1:
      // 1-bit MSE codes only under the QJL sketch (keys of 2 bits); the host refuses the rest
      if constexpr (QJL) return attn_bv<D, 1, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
      return hipErrorInvalidValue;
    case 2: return attn_bv<D, 2, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
    case 3: return attn_bv<D, 3, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
    default: return attn_bv<D, 4, QJL>(p, ck, cv, rk, rv, scores, so, lay, st);
  }
}

}  // namespace tq
