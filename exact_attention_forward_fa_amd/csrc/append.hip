// Append new keys and values to a KV cache before a decode step
// ("FlashAttention 常用接口简单介绍", §3.3: the optional k and v that update the
// cache).  The cache lengths count the tokens already cached, so token t of
// sequence b's new block lands at position cache_seqlens[b] + t.  With a block
// table, position pos lives in page block_table[b, pos / page_size] at row
// pos % page_size (update notes, v2.5); a dense cache holds it at row
// b * Smax + pos.
//
// Pure data movement: one lane copies one 16-byte piece of a (token, kv head)
// row of K and the same piece of V.  A position outside the cache (past Smax,
// past the block-table row, or a page number outside the pool) is skipped, so
// no write leaves the cache whatever the lengths and page numbers hold.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int ch = p.D / 8;   // 16-byte pieces per head row (2-byte elements)
  const int64_t n = (int64_t)p.B * p.S * p.Hkv * ch;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n) return;
  const int c = (int)(g % ch);
  int64_t r = g / ch;
  const int hk = (int)(r % p.Hkv);
  r /= p.Hkv;
  const int t = (int)(r % p.S);
  const int b = (int)(r / p.S);
  const int pos = p.cache_seqlens[b] + t;
  if (pos < 0) return;
  int64_t row;   // token row of the cache
  if (p.block_table) {
    const int pi = pos / p.page_size;
    if (pi >= p.bt_stride) return;
    const int page = p.block_table[(int64_t)b * p.bt_stride + pi];
    if (page < 0 || page >= p.num_blocks) return;
    row = (int64_t)page * p.page_size + (pos - pi * p.page_size);
  } else {
    if (pos >= p.smax) return;
    row = (int64_t)b * p.smax + pos;
  }
  const int64_t dst = (row * p.Hkv + hk) * p.D + c * 8;   // elements
  const u32x4 kv = *(const u32x4*)((const uint16_t*)p.k_new + b * p.kn_sb + t * p.kn_ss + hk * p.kn_sh + c * 8);
  const u32x4 vv = *(const u32x4*)((const uint16_t*)p.v_new + b * p.vn_sb + t * p.vn_ss + hk * p.vn_sh + c * 8);
  *(u32x4*)((uint16_t*)p.k_cache + dst) = kv;
  *(u32x4*)((uint16_t*)p.v_cache + dst) = vv;
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.S * p.Hkv * (p.D / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
