// Internal declarations shared by the host code and the kernel launchers of libtq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "tq.h"

namespace tq {

constexpr int kMaxLevels = 16;   // 4-bit codes on the GPU

// Codebook: host float64 solution plus the float32 / fp16 copies the kernels take by value.
struct Codebook {
  int d = 0, bits = 0;
  std::vector<double> centroids;   // [2^bits] ascending
  std::vector<double> thresholds;  // [2^bits - 1]
  double mse = 0.0;
  // Single-fp16 decode table: every 2^8 alpha c_k rounded to fp16 is within dec_rho (relative)
  // of its exact value; alpha in [1, 2) is chosen to make dec_rho small.
  double dec_alpha = 1.0, dec_rho = 1.0;
};

// The largest dec_rho with which a bfloat16 decode takes one fp16 centroid operand (two MFMA
// products) instead of a hi/lo pair (three).
constexpr double kDecOneOperandRho = 2.5e-5;
// Which decodes take the single-operand table: bfloat16 outputs of codebooks with at most four
// centroid magnitudes (the scan reaches ~2e-5 there; with eight it stops near 1e-4).
constexpr bool decode_one_operand(int bits, int out_dtype) { return out_dtype == TQ_BF16 && bits <= 3; }

// Rotation stack: float64 host copy and device operand tiles.
struct Rotation {
  int d = 0, n_rot = 0, device = -1;
  bool hadamard = false;         // Pi = H_d diag(s) / sqrt(d): encode / decode by the fast transform
  std::vector<double> pi;        // [n_rot, d, d] row-major
  // Device buffers (one allocation, offsets below), per rotation:
  //  enc_frag: bf16 MFMA A tiles of Pi (hi then lo), 4*d*d bytes
  //  dec_frag: fp16 MFMA A tiles of Pi^T for the decode, 4*d*d bytes: per output slice (one at
  //            d <= 128, four at d = 256) the set 2^11 P_hi, then the set 2^11 P_lo, with
  //            Pi^T = P_hi + P_lo and P_hi = fp16(Pi^T)
  //  pi_f32:   Pi in float32 row-major, 4*d*d bytes
  //  pit_f32:  Pi^T in float32 row-major, 4*d*d bytes
  //  pad:      kZeroBytes of zeros that masked lanes load from, then kSinkBytes that masked
  //            lanes store to (contents undefined), so kernels issue every access unconditionally
  void* dev = nullptr;
  size_t enc_stride = 0, dec_stride = 0, f32_stride = 0;   // bytes per rotation
  size_t enc_off = 0, dec_off = 0, f32_off = 0, f32t_off = 0, pad_off = 0;  // bytes from dev
  const uint8_t* enc(int r) const { return (const uint8_t*)dev + enc_off + (size_t)r * enc_stride; }
  const uint8_t* dec(int r) const { return (const uint8_t*)dev + dec_off + (size_t)r * dec_stride; }
  const float* f32(int r) const { return (const float*)((const uint8_t*)dev + f32_off + (size_t)r * f32_stride); }
  const float* f32t(int r) const {
    return (const float*)((const uint8_t*)dev + f32t_off + (size_t)r * f32_stride);
  }
  const uint8_t* zero() const { return (const uint8_t*)dev + pad_off; }
  uint8_t* sink() const { return (uint8_t*)dev + pad_off + kZeroBytes; }
  static constexpr size_t kZeroBytes = 256, kSinkBytes = 8192;
};

// QJL sketch of a rotation stack: per rotation r, M_r = S_r Pi_r^T as bf16 hi / lo MFMA tiles
// (same tile order as Pi's encode tiles, 4*d*d bytes) and S_r^T in float32 (4*d*d bytes).
struct Qjl {
  const Rotation* rot = nullptr;
  int d = 0, n_rot = 0, device = -1;
  void* dev = nullptr;
  size_t frag_stride = 0, st_stride = 0, frag_off = 0, st_off = 0;
  const uint8_t* frag(int r) const { return (const uint8_t*)dev + frag_off + (size_t)r * frag_stride; }
  const float* st(int r) const { return (const float*)((const uint8_t*)dev + st_off + (size_t)r * st_stride); }
};

// Quantization table for the encode. f = y * scale + offset (y the rotated, normalized
// coordinate) maps |y| < 1.0009 into [1, 2), one float binade, cut into 128 bins of width 1/128;
// bin j is byte 2 of bits(f) minus 128 (the exponent's low bit, then the top 7 fraction bits),
// so a kernel's table index is one byte select. Each bin holds at most one decision boundary,
// and the code base + (f > thr) = #{k : t_k < y} is (bits(f) - e) >> 24 for the bin's entry e:
//   bin with boundary thr:  e = bits(thr) + 1 - 2^24 - (base << 24)   (f > thr <=> bits(f) > bits(thr))
//   bin without boundary:   e = bits(lowest f of the bin) - (base << 24)
// (all f of the binade share one exponent, so their bit patterns differ by less than 2^23). The
// boundary is kept exactly as a float. Kernels hold the entries at LDS word 128 + j (byte 2 of
// bits(f) times 4), with a second copy below for inputs that are not finite.
// entry_top is the same table with the carry moved from bit 24 to bit 32 - b (2^24 and base << 24
// become 2^(32-b) and base << (32-b)): the code is then the top b bits of bits(f) - e, which a
// funnel shift appends to a packed word in one instruction. The f's of one binade differ by less
// than 2^23 < 2^(32-b), so the carry analysis is unchanged.
constexpr int kLutBins = 128;
struct QuantLut {
  float scale, offset;
  bool ok;                  // every bin holds at most one boundary
  uint32_t entry[kLutBins];
  uint32_t entry_top[kLutBins];
};

// Levels passed to kernels by value.
struct LevelArgs {
  float pos_thresholds[kMaxLevels / 2];   // t_{L/2+1} .. t_{L-1}: positive decision boundaries
  uint16_t centroid_f16[kMaxLevels];      // c_k as fp16 bits
  uint16_t dec_c_hi[kMaxLevels];          // decode operands: 2^8 fp16(c_k) and 2^8 (c_k - fp16(c_k)),
  uint16_t dec_c_lo[kMaxLevels];          //   each as fp16 bits
  uint16_t dec_c_one[kMaxLevels];         // 2^8 alpha c_k as fp16 bits (Codebook::dec_alpha)
  float dec_one_nscale;                   // 2^-19 / alpha: the norm multiplier that goes with it
  float dec_one_rho;                      // Codebook::dec_rho
  uint32_t centroid_bf16x2[kMaxLevels];   // c_k = hi + lo as bf16 bits: hi | lo << 16
  float centroid_f32[kMaxLevels];
  float centroid_sq[kMaxLevels];          // c_k^2 (float64 square, rounded once)
  QuantLut lut;
};

LevelArgs make_levels(const Codebook& cb);
inline bool lut_covers_unit_range(const LevelArgs& lv) { return lv.lut.ok; }

void set_error(const std::string& msg);

// ---- launchers (return hipError_t) ----
struct EncodeLaunch {
  const Rotation* rot;
  LevelArgs lv;
  int bits, x_dtype;
  int64_t vectors_per_rot, n, x_row_stride;
  const void* x;
  uint8_t* packed;
  float* norms;
  const int64_t* slot_mapping;
  bool norm_correct;   // store n / ||c[idx]|| instead of n
  hipStream_t stream;
};
hipError_t launch_encode(const EncodeLaunch& a);
hipError_t launch_encode_wht(const EncodeLaunch& a);   // Hadamard rotations (fast transform)

// QJL key encode: the MSE encode of `enc` (codebook at the MSE width, no norm correction) plus
// the residual's sign sketch and norm.
struct QjlEncodeLaunch {
  EncodeLaunch enc;
  const Qjl* qjl;
  uint8_t* signs;
  float* rnorms;
};
hipError_t launch_qjl_encode(const QjlEncodeLaunch& a);

// Recent-token window append: stage the flushed rows, encode them (K and V), fill the rings.
struct WindowAppendLaunch {
  EncodeLaunch enc_k, enc_v;   // codebook, rotation, output cache and vectors_per_rot of each side
  const void* k_new;
  const void* v_new;
  void* k_ring;
  void* v_ring;
  void* k_stage;
  void* v_stage;
  int64_t* slot;
  int32_t* seq_lens;
  const int32_t* block_table;
  int B, Hkv, n_new, R, d, elem, max_seq_len, block_size, mbps;
  hipStream_t stream;
};
hipError_t launch_window_append(const WindowAppendLaunch& a);

// Affine group quantization of values (groups of 32): encode (x -> packed, scales, zeros) or
// decode (packed, scales, zeros -> out).
struct GqLaunch {
  bool encode;
  int bits, d, dtype;   // dtype: x_dtype (encode) or out_dtype (decode)
  int64_t n, x_row_stride;
  const void* x;
  uint8_t* packed;
  uint16_t* scales;
  uint16_t* zeros;
  void* out;
  hipStream_t stream;
};
hipError_t launch_gq(const GqLaunch& a);

struct DecodeLaunch {
  const Rotation* rot;
  LevelArgs lv;
  int bits, out_dtype;
  int64_t vectors_per_rot, n;
  const uint8_t* packed;
  const float* norms;
  const int64_t* slot_mapping;
  void* out;
  hipStream_t stream;
};
hipError_t launch_decode(const DecodeLaunch& a);
hipError_t launch_decode_wht(const DecodeLaunch& a);   // Hadamard rotations (fast transform)

// Attention / scores: workspace layout is computed by attn_workspace_layout.
struct AttnLayout {
  int splits;            // token splits per (b, kv head)
  size_t qrot_off;       // float [B, Hq, d]: Pi_K q
  size_t qsk_off;        // float [B, Hq, d]: S q (QJL keys only; else == part_off, unused)
  size_t part_off;       // float [splits, B, Hq, d + 2]: (m, l, acc[d])
  size_t total;
};
AttnLayout attn_workspace_layout(const tq_attn_params* p, int d, int num_cu);
// Resident waves per CU of the fused-attention kernel for these parameters (plain / QJL keys).
int attn_resident_waves(const tq_attn_params* p, int d, int bk, int bv, int device);
int attn_resident_waves_qjl(const tq_attn_params* p, int d, int bk, int bv, int device);
hipError_t launch_attention(const tq_attn_params* p, const Codebook& ck, const Codebook& cv,
                            const Rotation& rk, const Rotation& rv, float* scores_out,
                            bool scores_only, const AttnLayout& lay, hipStream_t stream);
// Static scratch of tq_attn_decode_noalloc: kAttnScratchBytes per device; attn_scratch returns
// the device address of `device`'s copy (resolved once per device, which must be current).
constexpr size_t kAttnScratchBytes = (size_t)32 << 20;
hipError_t attn_scratch(int device, void** ptr);
// The same with QJL keys (p->qjl_k set), in its own translation unit.
hipError_t launch_attention_qjl(const tq_attn_params* p, const Codebook& ck, const Codebook& cv,
                                const Rotation& rk, const Rotation& rv, float* scores_out,
                                bool scores_only, const AttnLayout& lay, hipStream_t stream);

int device_cu_count(int device);

// Raise a kernel's dynamic LDS limit to `lds` bytes on `device`, once per (kernel, device);
// thread-safe (handles may be shared by threads, and two first calls may race).
hipError_t set_kernel_lds(const void* kernel, int device, size_t lds);

}  // namespace tq

struct tq_codebook {
  tq::Codebook cb;
};
struct tq_rotation {
  tq::Rotation rot;
};
struct tq_qjl {
  tq::Qjl q;
};
