// Recent-token window maintenance: append tokens to the per-(sequence, KV head) rings and
// flush the tokens that leave the window into the compressed cache.
//
// Method (KV Cache API page, TurboQuantKVCache.prefill / append): the newest R tokens of a
// sequence stay at full precision; an append that grows the buffer beyond R moves its oldest
// tokens into the compressed store, and a prefill of L tokens compresses all but the newest R.
// With L tokens before and n appended, positions [c0, c1) are flushed, c0 = L - min(L, R),
// c1 = L + n - min(L + n, R): each comes from the ring when it was already there (position
// < L) and straight from the new tokens otherwise. The flush reuses the encode kernel: a
// gather kernel stages the flushed rows and their destination rows (slot mapping), the encode
// runs on the staging rows for K and for V, then the new tokens that remain in the window are
// written into their ring slots (position mod R) and the lengths are advanced.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {

struct WinAppendKArgs {
  const void* k_new;
  const void* v_new;
  void* k_ring;
  void* v_ring;
  void* k_stage;
  void* v_stage;
  int64_t* slot;
  int32_t* seq_lens;
  const int32_t* block_table;
  int32_t B, Hkv, n_new, R, elem, max_seq_len, block_size, mbps;
};

// destination row of position e of (b, h) in the compressed cache, -1 when out of range
__device__ __forceinline__ int64_t win_row(const WinAppendKArgs& a, int b, int h, int e) {
  if (e >= a.max_seq_len) return -1;
  if (!a.block_table) return ((int64_t)b * a.Hkv + h) * a.max_seq_len + e;
  const int blk = e / a.block_size;
  return ((int64_t)a.block_table[(int64_t)b * a.mbps + blk] * a.Hkv + h) * a.block_size + (e - blk * a.block_size);
}

// one block per staging row (b, h, j); threads copy the row in 16-byte pieces
__global__ void win_gather_kernel(WinAppendKArgs a, int row_bytes) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = a.seq_lens[b];
  const int c0 = L - min(L, a.R), c1 = L + a.n_new - min(L + a.n_new, a.R);
  const int e = c0 + j;
  const bool flush = e < c1;
  const int64_t srow = ((int64_t)b * a.Hkv + h) * a.n_new + j;
  const uint8_t *ks = nullptr, *vs = nullptr;
  if (flush) {
    if (e < L) {
      const int64_t r = ((int64_t)b * a.Hkv + h) * a.R + e % a.R;
      ks = (const uint8_t*)a.k_ring + r * row_bytes;
      vs = (const uint8_t*)a.v_ring + r * row_bytes;
    } else {
      const int64_t r = ((int64_t)b * a.Hkv + h) * a.n_new + (e - L);
      ks = (const uint8_t*)a.k_new + r * row_bytes;
      vs = (const uint8_t*)a.v_new + r * row_bytes;
    }
  }
  uint8_t* kd = (uint8_t*)a.k_stage + srow * row_bytes;
  uint8_t* vd = (uint8_t*)a.v_stage + srow * row_bytes;
  for (int o = threadIdx.x * 16; o < row_bytes; o += blockDim.x * 16) {
    u32x4 kq = {0u, 0u, 0u, 0u}, vq = {0u, 0u, 0u, 0u};   // rows not flushed are staged as zeros
    if (flush) {
      kq = *(const u32x4*)(ks + o);
      vq = *(const u32x4*)(vs + o);
    }
    *(u32x4*)(kd + o) = kq;
    *(u32x4*)(vd + o) = vq;
  }
  if (threadIdx.x == 0) a.slot[srow] = flush ? win_row(a, b, h, e) : -1;
}

// new tokens that stay in the window go to ring slot position mod R
__global__ void win_insert_kernel(WinAppendKArgs a, int row_bytes) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = a.seq_lens[b];
  const int p = L + j;
  const int c1 = L + a.n_new - min(L + a.n_new, a.R);
  if (p < c1 || a.R == 0) return;
  const int64_t src = ((int64_t)b * a.Hkv + h) * a.n_new + j;
  const int64_t dst = ((int64_t)b * a.Hkv + h) * a.R + p % a.R;
  for (int o = threadIdx.x * 16; o < row_bytes; o += blockDim.x * 16) {
    *(u32x4*)((uint8_t*)a.k_ring + dst * row_bytes + o) = *(const u32x4*)((const uint8_t*)a.k_new + src * row_bytes + o);
    *(u32x4*)((uint8_t*)a.v_ring + dst * row_bytes + o) = *(const u32x4*)((const uint8_t*)a.v_new + src * row_bytes + o);
  }
}

__global__ void win_bump_kernel(int32_t* seq_lens, int B, int n) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) seq_lens[b] += n;
}

hipError_t launch_window_append(const WindowAppendLaunch& L) {
  WinAppendKArgs a;
  a.k_new = L.k_new;
  a.v_new = L.v_new;
  a.k_ring = L.k_ring;
  a.v_ring = L.v_ring;
  a.k_stage = L.k_stage;
  a.v_stage = L.v_stage;
  a.slot = L.slot;
  a.seq_lens = L.seq_lens;
  a.block_table = L.block_table;
  a.B = L.B;
  a.Hkv = L.Hkv;
  a.n_new = L.n_new;
  a.R = L.R;
  a.elem = L.elem;
  a.max_seq_len = L.max_seq_len;
  a.block_size = L.block_size;
  a.mbps = L.mbps;
  const int row_bytes = L.d * L.elem;   // a multiple of 16 for d in {64, 128, 256}
  const dim3 grid((unsigned)L.n_new, (unsigned)L.Hkv, (unsigned)L.B);
  const int threads = 64;
  hipLaunchKernelGGL(win_gather_kernel, grid, dim3(threads), 0, L.stream, a, row_bytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_rows = (int64_t)L.B * L.Hkv * L.n_new;
  for (int side = 0; side < 2; ++side) {
    EncodeLaunch en = side == 0 ? L.enc_k : L.enc_v;
    en.x = side == 0 ? L.k_stage : L.v_stage;
    en.n = n_rows;
    en.x_row_stride = L.d;
    en.slot_mapping = L.slot;
    en.stream = L.stream;
    if ((e = launch_encode(en)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(win_insert_kernel, grid, dim3(threads), 0, L.stream, a, row_bytes);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(win_bump_kernel, dim3((unsigned)((L.B + 255) / 256)), dim3(256), 0, L.stream, L.seq_lens, L.B,
                     L.n_new);
  return hipGetLastError();
}

}  // namespace tq
