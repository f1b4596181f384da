/*
 * tq.h - C ABI of libtq, the MI355X (gfx950) TurboQuant KV-cache codec hot path.
 *
 * The codec (TurboQuant, as the pages describe it):
 *   encode: n = ||x||_2; y = Pi x / (n + 1e-8); idx_i = nearest Lloyd-Max centroid of y_i;
 *           store the b-bit codes densely and n separately.
 *   decode: x_hat = n * Pi^T c[idx].
 *   scores: s_t = scale * <q, k_hat_t> = scale * n_t * <Pi q, c[idx_t]> (query rotated once).
 *   attention (decode step): o = sum_t softmax(s)_t v_hat_t.
 * Sources: KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), compressor classes
 * (__init__, compress, decompress) and TurboQuantKVCache.attention_scores / attend;
 * aitherkvcache landing page (encode -> uint8 codes + float32 norms); Turbo Attention
 * (turbo-attn) PyPI page, "The codec" (queries rotated like keys, no un-rotation) and
 * "Kernels" (split-K paged decode; fused compress-store).
 *
 * Conventions for every call:
 *   - Sizes are element counts unless named *_bytes. Pointers named "device" must be HIP
 *     device memory on the device the handles were created on; "host" pointers are CPU memory.
 *   - The caller owns every buffer. The library owns only the handles (freed by *_free).
 *     Hot-path calls (tq_encode*, tq_qjl_encode, tq_decode, tq_scores_compressed,
 *     tq_attn_decode, tq_gq_*, tq_window_append) never
 *     allocate device memory and never synchronize: they enqueue kernels on `stream`
 *     (a hipStream_t; NULL is the null stream) and return.
 *   - Return value: TQ_OK (0) or a negative tq_status. On error nothing is launched and
 *     tq_last_error() (per thread) names the argument and the accepted values.
 *     NaN/Inf inputs are not checked; they propagate.
 *   - Handles are immutable after creation and may be shared by threads and streams.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_VERSION 1

typedef struct tq_codebook tq_codebook_t;
typedef struct tq_rotation tq_rotation_t;
typedef struct tq_qjl tq_qjl_t;
typedef void* tq_stream_t; /* hipStream_t */

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,   /* a size, dtype, bit width or head dim out of range */
  TQ_ERR_NULL = -2,          /* a required pointer is NULL */
  TQ_ERR_ALIGN = -3,         /* a pointer or row stride is not aligned as required */
  TQ_ERR_NOT_ORTHOGONAL = -4,/* a rotation matrix fails max|Pi^T Pi - I| <= 1e-9 */
  TQ_ERR_WORKSPACE = -5,     /* workspace NULL or smaller than tq_attn_workspace_size */
  TQ_ERR_HIP = -6,           /* a HIP runtime call failed (message has hipGetErrorString) */
  TQ_ERR_NO_DEVICE = -7      /* no HIP device, or the handles belong to another device */
} tq_status;

int tq_version(void);

/* Message of the last failed call on this thread ("" if none). Valid until the next call. */
const char* tq_last_error(void);

/* ---- codebook (host, float64) --------------------------------------------------------
 * Lloyd-Max scalar quantizer with 2^bits levels for one coordinate of a uniformly random
 * unit vector in R^d, density f_d(x) = C_d (1 - x^2)^((d-3)/2) on [-1, 1]. Data
 * independent: depends on (d, bits) only (TurboQuant forum article, zingnex.cn, "two core
 * steps": codebooks precomputed from mathematics, no calibration; KV Cache API page,
 * compressor __init__ builds it from (head_dim, bits) alone). Solved by Lloyd's iteration
 * to its fixed point (unique: f_d is log-concave), cell integrals by Gauss-Legendre
 * quadrature.
 *   d:    3 <= d <= 4096 (the GPU kernels accept 64, 128, 256)
 *   bits: 1..4 (the GPU kernels accept 2, 3, 4)
 * Returns NULL on bad arguments (tq_last_error says which). No device memory is used:
 * the kernels receive the levels by value. */
tq_codebook_t* tq_codebook_init(int d, int bits);

/* Copy out the codebook (host buffers, may each be NULL):
 *   centroids[2^bits] ascending, thresholds[2^bits - 1] (midpoints; the middle one is 0),
 *   mse = expected squared error of one coordinate E[(X - Q(X))^2]. */
int tq_codebook_get(const tq_codebook_t* cb, double* centroids, double* thresholds, double* mse);
int tq_codebook_dims(const tq_codebook_t* cb, int* d, int* bits);
void tq_codebook_free(tq_codebook_t* cb);

/* ---- rotation (host QR, uploaded once) -------------------------------------------------
 * A stack of n_rot Haar rotations for head dim d (64, 128 or 256), e.g. one per layer.
 * From Gaussian draws (KV Cache API page, TurboQuantCompressorV2.__init__): each
 * gaussian[r] (host, float32, [n_rot, d, d] row-major, the caller's seeded N(0,1) draw)
 * is QR-factored in float64 (Householder) and Pi = Q diag(sign(diag R)), a zero sign
 * counting as +1. tq_rotation_from_matrix takes the float64 matrices Pi themselves (host,
 * [n_rot, d, d] row-major) and checks max|Pi^T Pi - I| <= 1e-9.
 * Both upload the kernels' device copies (MFMA operand tiles of Pi in bf16 hi/lo and fp16,
 * and Pi in fp32) to the current HIP device, which the handle is then bound to.
 * Returns NULL on error (bad d/n_rot, non-orthogonal input, no device, HIP failure). */
tq_rotation_t* tq_rotation_from_gaussian(int d, int n_rot, const float* gaussian);
tq_rotation_t* tq_rotation_from_matrix(int d, int n_rot, const double* pi);

/* Hadamard rotation (Turbo Attention PyPI page, "The codec", Hadamard rotation row: a
 * Walsh-Hadamard transform that smears large channels over all coordinates, applied to the
 * query side as well):
 * Pi_r = H_d diag(s_r) / sqrt(d), H_d Sylvester's +-1 Walsh-Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)), s_r = signs[r] (host int8 [n_rot, d], each +1 or -1;
 * NULL = all +1). Uploaded like the other constructors; every kernel takes it unchanged.
 * Returns NULL on error (bad d/n_rot, a sign other than +-1, no device, HIP failure). */
tq_rotation_t* tq_rotation_hadamard(int d, int n_rot, const int8_t* signs);

/* Host only, no device: the float64 rotation (host, [d, d]) that tq_rotation_from_gaussian
 * makes from one Gaussian draw (host, float32 [d, d]). 3 <= d <= 4096. */
int tq_rotation_compute(int d, const float* gaussian, double* pi);

/* Copy the float64 rotations out (host, [n_rot, d, d]). */
int tq_rotation_get(const tq_rotation_t* rot, double* pi);
int tq_rotation_dims(const tq_rotation_t* rot, int* d, int* n_rot);
void tq_rotation_free(tq_rotation_t* rot);

/* ---- encode -------------------------------------------------------------------------------
 * x: device, n vectors of d elements, dtype x_dtype (TQ_F32, TQ_BF16 or TQ_F16); vector i
 *    starts at element i * x_row_stride (x_row_stride >= d). x must be 16-byte aligned and
 *    x_row_stride * sizeof(dtype) a multiple of 16.
 * Rotation of vector i: r = i / vectors_per_rot (vectors_per_rot = 0: every vector uses
 *    rotation 0); requires r < n_rot for every i.
 * Outputs (device): packed row j = (d*bits)/8 bytes, codes as an LSB-first bitstream (code k
 *    in stream bits [k*bits, (k+1)*bits), stream bit s = bit s%8 of byte s/8; 3-bit codes
 *    cross bytes); norms[j] = ||x_i||_2 as float32. Vector i is written to row
 *    j = slot_mapping[i] (device int64 [n]; NULL = identity; a negative slot skips the
 *    vector). packed must be 8-byte aligned, norms 4-byte aligned.
 * n = 0 is a no-op. Codebook and rotation must have the same d. */
int tq_encode(const tq_codebook_t* cb, const tq_rotation_t* rot, int64_t vectors_per_rot,
              const void* x, int x_dtype, int64_t n, int64_t x_row_stride,
              uint8_t* packed, float* norms, const int64_t* slot_mapping, tq_stream_t stream);

/* tq_encode with key-side norm correction (Turbo Attention PyPI page, "The codec", Norms
 * row: the decoded key keeps its length): same codes, same arguments, same errors, but
 * norms[j] = ||x_i|| / ||c[codes of row j]||_2, so tq_decode returns a vector of length
 * ||x_i|| and scores / attention use the corrected length with no other change. */
int tq_encode_norm_corrected(const tq_codebook_t* cb, const tq_rotation_t* rot, int64_t vectors_per_rot,
                             const void* x, int x_dtype, int64_t n, int64_t x_row_stride,
                             uint8_t* packed, float* norms, const int64_t* slot_mapping, tq_stream_t stream);

/* ---- QJL residual stage of keys -------------------------------------------------------------
 * KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), TurboQuantCompressorV2: a key of b
 * bits keeps the MSE codes of its direction at max(b - 1, 1) bits, its norm n, the residual
 * norm ||r|| with r = x - n Pi^T c[idx], and the signs of S r for a d x d sketch S (a zero
 * projection counts as +1); scores use <q, k> ~ n <Pi q, c[idx]> + ||r|| sqrt(pi/2)/d <S q, signs>.
 *
 * tq_qjl_create: sketch is host float32 [n_rot, d, d] row-major, one S_r per rotation of rot
 * (the page draws S from a CPU generator seeded seed + 10000). The library forms
 * M_r = S_r Pi_r^T in float64 and uploads M_r's MFMA tiles and S_r^T (float32) to rot's device.
 * The handle refers to rot, which must outlive it; d in {64, 128, 256}. NULL on error. */
tq_qjl_t* tq_qjl_create(const tq_rotation_t* rot, const float* sketch);
void tq_qjl_free(tq_qjl_t* qjl);

/* QJL encode of keys with qjl's rotation: packed / norms exactly as tq_encode with cb (the
 * MSE codebook, 1..4 bits for keys of 2..5 bits, same d), plus (device, row j as in tq_encode)
 *   signs[j]:  d/8 bytes, bit i (LSB-first stream as the codes) = 1 iff (S_r r)_i >= 0;
 *   rnorms[j]: ||r||_2 as float32.
 * signs must be 16-byte aligned, rnorms 4-byte aligned; other arguments and errors as in
 * tq_encode (norm correction does not apply). n = 0 is a no-op. */
int tq_qjl_encode(const tq_codebook_t* cb, const tq_qjl_t* qjl, int64_t vectors_per_rot,
                  const void* x, int x_dtype, int64_t n, int64_t x_row_stride,
                  uint8_t* packed, float* norms, uint8_t* signs, float* rnorms,
                  const int64_t* slot_mapping, tq_stream_t stream);

/* ---- decode -------------------------------------------------------------------------------
 * Inverse of tq_encode: out[i] (device, dtype out_dtype, contiguous [n, d], 16-byte aligned)
 * = norms[j] * Pi_r^T c[codes of row j] with j = slot_mapping[i] (NULL = identity; a negative
 * slot writes zeros) and r = i / vectors_per_rot as in tq_encode. */
int tq_decode(const tq_codebook_t* cb, const tq_rotation_t* rot, int64_t vectors_per_rot,
              const uint8_t* packed, const float* norms, const int64_t* slot_mapping,
              int64_t n, void* out, int out_dtype, tq_stream_t stream);

/* ---- scores and fused decode attention over the compressed cache ---------------------
 * One decode step: query q[b, h] (h < num_q_heads) attends to the cached tokens
 * t < seq_lens[b] of KV head g = h / (num_q_heads / num_kv_heads) (contiguous groups;
 * 1 <= num_q_heads / num_kv_heads <= 16).
 * Cache layouts (device; K codes at cb_k's width, V codes at cb_v's width, rows as in
 * tq_encode, norms float32):
 *   dense (block_table == NULL): packed [batch, num_kv_heads, max_seq_len, row],
 *         norms [batch, num_kv_heads, max_seq_len]; max_seq_len * row must be < 2^32
 *         bytes (else TQ_ERR_INVALID_ARG: use the paged layout);
 *   paged: pools packed [num_blocks, num_kv_heads, block_size, row], norms
 *         [num_blocks, num_kv_heads, block_size]; token t of sequence b is in block
 *         block_table[b * max_blocks_per_seq + t / block_size] at offset t % block_size.
 * seq_lens: device int32 [batch] (0 <= len <= max_seq_len), or NULL: every sequence has
 *   max_seq_len tokens. Rotation of sequence b: b / batch_per_rot (0 = rotation 0 for all).
 * scale: multiplies <q, k>; pass 1/sqrt(d) for the pages' default. */
typedef struct {
  const tq_codebook_t* cb_k;
  const tq_codebook_t* cb_v;
  const tq_rotation_t* rot_k;
  const tq_rotation_t* rot_v;
  int32_t batch, num_q_heads, num_kv_heads;
  const void* q;            /* device [batch, num_q_heads, d], dtype q_dtype, contiguous */
  int32_t q_dtype;
  const uint8_t* k_packed;
  const float* k_norms;
  const uint8_t* v_packed;
  const float* v_norms;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  const int32_t* block_table;
  int32_t block_size, max_blocks_per_seq;
  int32_t batch_per_rot;
  float scale;
  void* out;                /* device [batch, num_q_heads, d], dtype out_dtype */
  int32_t out_dtype;
  float* lse;               /* optional device [batch, num_q_heads]: log sum_t exp(s_t) */
  void* workspace;          /* device, >= tq_attn_workspace_size bytes, 256-byte aligned */
  size_t workspace_bytes;
  int32_t num_splits;       /* token splits per (sequence, KV head); 0 = chosen by the library */
  /* Recent-token window (optional; KV Cache API page, TurboQuantKVCache.prefill / append /
   * attention_scores / attend: the newest tokens stay at full precision beside the compressed
   * ones). With window = R > 0, sequence b has L_b = seq_lens[b] tokens (<= max_seq_len) in
   * total: the newest w_b = min(L_b, R) are read from the rings k_window / v_window (device
   * [batch, num_kv_heads, R, d], dtype window_dtype, the token at position t in slot t mod R)
   * and only positions [0, L_b - w_b) from the compressed cache (rows indexed by position as
   * above). tq_attn_decode takes one softmax over all L_b tokens; tq_scores_compressed scores
   * the compressed positions only. window = 0 (and NULL rings): every token is compressed. */
  const void* k_window;
  const void* v_window;
  int32_t window;
  int32_t window_dtype;
  /* QJL keys (optional; KV Cache API page, TurboQuantCompressorV2.asymmetric_attention_scores):
   * with qjl_k != NULL the compressed keys were written by tq_qjl_encode with cb_k and qjl_k
   * (built on rot_k; cb_k may then have 1 bit, keys of 2 bits), and every compressed score becomes
   *   scale * (n_t <Pi_K q, c_K[idx_t]> + ||r_t|| sqrt(pi/2)/d <S q, signs_t>).
   * k_signs (d/8 bytes per token, 16-byte aligned base) and k_rnorms (float32) follow the
   * layout of k_packed / k_norms (dense or paged). qjl_k = NULL: plain MSE keys. */
  const tq_qjl_t* qjl_k;
  const uint8_t* k_signs;
  const float* k_rnorms;
} tq_attn_params;

/* Bytes of workspace tq_attn_decode and tq_scores_compressed need for these parameters. */
size_t tq_attn_workspace_size(const tq_attn_params* p);

/* s[b, h, t] = scale * n_t * <Pi_K q[b, h], c_K[idx_t]> (plus the QJL term with qjl_k) for
 * t < seq_lens[b] (entries beyond are left untouched). scores: device float32 [batch, num_q_heads, max_seq_len]. Uses the K
 * fields of p (cb_v, rot_v, v_*, out, lse are ignored) and p->workspace. */
int tq_scores_compressed(const tq_attn_params* p, float* scores, tq_stream_t stream);

/* Fused decode attention: o[b, h] = Pi_V^T sum_t p_t n^v_t c_V[idx^v_t] with
 * p = softmax_t(s[b, h, :len_b]), computed without materialising K or V: split-K over
 * tokens with an online softmax, then a log-sum-exp merge of the splits. len_b = 0 gives
 * o = 0 and lse = -inf. */
int tq_attn_decode(const tq_attn_params* p, tq_stream_t stream);

/* tq_attn_decode without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * parameters, results and errors as tq_attn_decode, except that p->workspace and
 * p->workspace_bytes are ignored: the rotated queries and split partials go to a static device
 * array of 32 MiB (one per GPU the library runs on, held until the process ends) that the
 * library resolves once per device; no device memory is allocated or freed by this call.
 * A call whose tq_attn_workspace_size exceeds 32 MiB fails with TQ_ERR_WORKSPACE before any
 * launch (use fewer num_splits or tq_attn_decode). All calls on one GPU share that array and
 * nothing in it must start at zero: calls that overlap on one GPU (other streams, other host
 * threads) race, so serialize them (one stream, or events between streams). */
int tq_attn_decode_noalloc(const tq_attn_params* p, tq_stream_t stream);

/* ---- affine group quantization of values ---------------------------------------------------
 * KV Cache API page, quantize_values / dequantize_values: per group of 32 consecutive
 * elements of a vector, zero = min, scale = max((max - min) / (2^bits - 1), 1e-12) in float32,
 * q = clamp(round_half_even((x - zero) / scale), 0, 2^bits - 1); the decode is
 * x_hat = q * scale16 + zero16 (float32 product, then sum) with scale16 / zero16 the float16
 * copies the encode stores. All float32 steps are IEEE, so codes, metadata and outputs are
 * exact functions of the input. bits in {2, 3, 4, 8}; d a multiple of 32 (32..8192).
 * Layouts (device): x [n, d] (row stride x_row_stride elements, 16-byte aligned rows);
 * packed [n, d*bits/8] bytes, the 32 codes of a group as an LSB-first bitstream of 4*bits
 * bytes (16-byte aligned base); scales / zeros float16 [n, d/32]; out [n, d] contiguous,
 * 16-byte aligned. Launch on the current device; n = 0 is a no-op. */
int tq_gq_encode(int d, int bits, const void* x, int x_dtype, int64_t n, int64_t x_row_stride,
                 uint8_t* packed, uint16_t* scales, uint16_t* zeros, tq_stream_t stream);
int tq_gq_decode(int d, int bits, const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                 int64_t n, void* out, int out_dtype, tq_stream_t stream);

/* ---- recent-token window: append and flush ------------------------------------------------
 * KV Cache API page, TurboQuantKVCache.prefill / append: the newest R = window tokens of each
 * sequence stay at full precision; tokens leaving the window are compressed. One call appends
 * n_new tokens to every sequence of the batch: with L = seq_lens[b] tokens before, positions
 * [L - min(L, R), L + n_new - min(L + n_new, R)) are encoded (codebook/rotation of each side,
 * as tq_encode) into the compressed cache rows of their positions, the new tokens that stay
 * in the window are written to ring slot (position mod R), and seq_lens[b] += n_new. A first
 * call on empty sequences with n_new = prompt length is the page's prefill split; repeated
 * calls with n_new = 1 are its decode-time append (same final state either way).
 * Layouts (device): k_new / v_new [batch, num_kv_heads, n_new, d] and the rings
 * [batch, num_kv_heads, window, d], all of dtype window_dtype, 16-byte aligned; compressed
 * cache dense [batch, num_kv_heads, max_seq_len, row] or paged as in tq_attn_params.
 * The caller keeps seq_lens[b] + n_new <= max_seq_len (rows past it are not written). The
 * workspace (device, 256-byte aligned) holds the staged rows and their slot mapping. */
typedef struct {
  const tq_codebook_t* cb_k;
  const tq_codebook_t* cb_v;
  const tq_rotation_t* rot_k;
  const tq_rotation_t* rot_v;
  int32_t batch, num_kv_heads, n_new;
  const void* k_new;
  const void* v_new;
  void* k_window;
  void* v_window;
  int32_t window, window_dtype;
  int32_t* seq_lens;        /* device int32 [batch]: tokens before the call; advanced by n_new */
  uint8_t* k_packed;
  float* k_norms;
  uint8_t* v_packed;
  float* v_norms;
  int32_t max_seq_len;
  const int32_t* block_table;
  int32_t block_size, max_blocks_per_seq;
  int32_t batch_per_rot;    /* rotation of sequence b: b / batch_per_rot (0 = rotation 0) */
  void* workspace;
  size_t workspace_bytes;
} tq_window_append_params;

size_t tq_window_append_workspace_size(const tq_window_append_params* p);
int tq_window_append(const tq_window_append_params* p, tq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
