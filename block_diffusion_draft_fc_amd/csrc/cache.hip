// Draft KV cache writes: the raw row append and the page-table update.
//
// The append is the cache update of "DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析"
// section 4 for rows that are already normed and rotated: row j of sequence s
// lands at position len_s + j.  It moves storage words as integers, so any
// bit pattern (including NaN payloads) arrives unchanged.  The page table maps
// logical pages to physical pages ("KV Cache + Speculative Decoding 面试 Cheat
// Sheet" 5.3); its new entries travel in the kernel arguments.
#include "kernels.hpp"

namespace dflash {

// One thread per (row, K/V head, 8-element group).
template <typename W>
__global__ __launch_bounds__(256) void cache_append_kernel(AppendArgs a, int64_t n_rows) {
  const int g8n = a.cache.d_h >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = n_rows * a.cache.n_kv * g8n;
  if (idx >= total) return;
  const int c8 = (int)(idx % g8n);
  const int64_t rg = idx / g8n;
  const int g = (int)(rg % a.cache.n_kv);
  const int64_t j = rg / a.cache.n_kv;
  int s = 0;
  while (s + 1 < a.n_seqs && j >= a.cu[s + 1]) ++s;
  const int pos = a.L[s] + (int)(j - a.cu[s]);
  const int64_t page = cache_page(a.cache, s, pos);
  const int slot = pos % a.cache.page_rows;
  const int64_t src = (j * a.cache.n_kv + g) * a.cache.d_h + c8 * 8;
  const W* ks = static_cast<const W*>(a.k_rows) + src;
  const W* vs = static_cast<const W*>(a.v_rows) + src;
  W* kd = static_cast<W*>(a.cache.k_pool) + k_offset(a.cache, page, g, slot) + c8 * 8;
  W* vd = static_cast<W*>(a.cache.v_pool) + v_offset(a.cache, page, g, slot) + c8 * 8 * kVTile;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kd[e] = ks[e];
    vd[e * kVTile] = vs[e];
  }
}

hipError_t launch_cache_append(int dtype, const AppendArgs& a, int64_t n_rows, hipStream_t s) {
  const int64_t total = n_rows * a.cache.n_kv * (a.cache.d_h >> 3);
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dtype == 2)
    launch(cache_append_kernel<uint8_t>, dim3(blocks), dim3(256), 0, s, a, n_rows);
  else if (dtype == 1)
    launch(cache_append_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, a, n_rows);
  else
    launch(cache_append_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s, a, n_rows);
  return hipGetLastError();
}

__global__ void bt_update_kernel(BtUpdateArgs a) {
  const int i = threadIdx.x;
  if (i < a.count) a.table[a.index[i]] = a.value[i];
}

hipError_t launch_bt_update(const BtUpdateArgs& a, hipStream_t s) {
  if (a.count == 0) return hipSuccess;
  launch(bt_update_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- device-side lengths
__global__ __launch_bounds__(64) void len_update_kernel(LenArgs a) {
  const int r = threadIdx.x;
  if (r >= a.R) return;
  a.d_len[r] = a.set ? a.value[r] : max(0, a.d_len[r] + a.delta);
}

hipError_t launch_len_update(const LenArgs& a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  launch(len_update_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
