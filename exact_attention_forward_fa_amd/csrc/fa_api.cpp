// Host side of the C ABI declared in include/fa.h: argument validation,
// defaults, workspace layout and kernel launches on the caller's stream.
// Validation never touches the HIP runtime, so every error path can be
// exercised on a machine without a GPU.  The one exception is opt-in: with
// the environment variable FA_DEBUG=1, the device-side index data the caller
// promises to keep consistent (cu_seqlens, cache_seqlens, block_table) is
// copied back and checked before anything is launched.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "fa_kernels.hpp"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa_status ok() {
  g_last_error.clear();
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fa_status check_opts(const fa_attn_opts* o, int D, float* scale_out) {
  float scale = 0.f;
  if (o) {
    if (!std::isfinite(o->softmax_scale)) return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
    if (o->window_left < -1 || o->window_right < -1)
      return fail(FA_ERR_INVALID_ARGUMENT, "window (%d, %d): each side must be >= -1", o->window_left, o->window_right);
    if (!std::isfinite(o->softcap) || o->softcap < 0.f)
      return fail(FA_ERR_INVALID_ARGUMENT, "softcap must be finite and >= 0");
    if (o->softmax_scale < 0.f)
      return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale %g is negative (0 selects 1/sqrt(D))", o->softmax_scale);
    scale = o->softmax_scale;
  }
  *scale_out = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  return FA_OK;
}

// D in {32, 64, 96, 128, 256} for every call
fa_status check_common(int dtype, int Hq, int Hkv, int D) {
  if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARGUMENT, "Hkv=%d must divide Hq=%d", Hkv, Hq);
  if (D <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "head_dim must be positive (D=%d)", D);
  if (D != 32 && D != 64 && D != 96 && D != 128 && D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not built (32, 64, 96, 128 or 256)", D);
  return FA_OK;
}

fa_status check_strides(const char* name, const int64_t* s, int n) {
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s stride %d is negative", name, i);
    if (s[i] % 8 != 0) return fail(FA_ERR_UNSUPPORTED, "%s stride %d (%lld elements) is not a multiple of 8", name, i, (long long)s[i]);
  }
  return FA_OK;
}

// Window sides as the kernels take them: -1 (unbounded) or a distance.  Any
// side of 2^30 or more reaches every key of a sequence shorter than 2^30, so
// it is capped there, which keeps position + side inside int32 in the kernels.
int window_side(const fa_attn_opts* o, bool left) {
  const int w = o ? (left ? o->window_left : o->window_right) : -1;
  return w > (1 << 30) ? (1 << 30) : w;
}

void fill_opts(fa::PrefillParams& p, const fa_attn_opts* o, float scale) {
  p.scale = scale;
  p.out_scale = 1.f;
  p.softcap = o ? o->softcap : 0.f;
  p.alibi = o ? o->alibi_slopes : nullptr;
  p.causal = o ? (o->causal != 0) : 0;
  p.wl = window_side(o, true);
  p.wr = window_side(o, false);
}

// Keys a query row can see besides its own position: the left window side plus
// the right one (0 under causal), or -1 when either side is unbounded.
int key_span(const fa_attn_opts* o) {
  const int wl = window_side(o, true), wr = window_side(o, false);
  const bool causal = o && o->causal;
  if (wl < 0 || (!causal && wr < 0)) return -1;
  return (int)std::min<int64_t>((int64_t)wl + (causal ? 0 : wr), 1 << 30);
}

fa_status launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// An HSA dispatch counts work-items in 32 bits: workgroups times threads per
// workgroup must stay below 2^32.
bool dispatch_fits(int64_t groups, int threads) { return groups >= 0 && groups * threads <= 0xffffffffLL; }
fa_status grid_too_large(int64_t groups, int threads) {
  return fail(FA_ERR_UNSUPPORTED, "%lld workgroups of %d threads exceed the 2^32 work-items of one dispatch",
              (long long)groups, threads);
}

// compute units of the current device (256 if the query fails)
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    return 256;
  return cus;
}

// ---- FA_DEBUG=1: checks of device-side index data (synchronous, debugging only)
bool debug_checks() {
  const char* e = std::getenv("FA_DEBUG");
  return e && e[0] == '1' && e[1] == 0;
}

fa_status read_ints(const int* d, size_t n, std::vector<int>& h, hipStream_t s) {
  h.assign(n, 0);
  if (n == 0) return FA_OK;
  hipError_t e = hipMemcpyAsync(h.data(), d, n * sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "FA_DEBUG read of index data: %s", hipGetErrorString(e));
  return FA_OK;
}

// cu_seqlens_q/k: non-negative, non-decreasing, every length within max_seqlen,
// the last entry within total
fa_status debug_check_cu(const int* cu_q, const int* cu_k, int B, int max_q, int max_k, int total_q, int total_k,
                         hipStream_t s) {
  std::vector<int> q, k;
  fa_status st;
  if ((st = read_ints(cu_q, (size_t)B + 1, q, s)) || (st = read_ints(cu_k, (size_t)B + 1, k, s))) return st;
  for (int b = 0; b <= B; ++b) {
    if (q[b] < 0 || k[b] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "FA_DEBUG: cu_seqlens[%d] is negative", b);
    if (b == 0) continue;
    const int lq = q[b] - q[b - 1], lk = k[b] - k[b - 1];
    if (lq < 0 || lk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "FA_DEBUG: cu_seqlens decrease at entry %d", b);
    if (lq > max_q || lk > max_k)
      return fail(FA_ERR_INVALID_ARGUMENT, "FA_DEBUG: sequence %d has %d queries / %d keys, above max_seqlen %d / %d",
                  b - 1, lq, lk, max_q, max_k);
  }
  if (q[B] > total_q || k[B] > total_k)
    return fail(FA_ERR_INVALID_ARGUMENT, "FA_DEBUG: cu_seqlens end at %d / %d, beyond total %d / %d", q[B], k[B],
                total_q, total_k);
  return FA_OK;
}

// cache_seqlens non-negative; when the decode runs (reads = true) every
// sequence's cached plus new tokens fit the cache and the block-table entries
// of the pages it reads name pages of the pool
fa_status debug_check_cache(const int* lens, const int* bt, int bt_stride, int page_size, int num_blocks_or_smax,
                            int B, int S_new, bool reads, hipStream_t s) {
  std::vector<int> l, t;
  fa_status st;
  if ((st = read_ints(lens, (size_t)B, l, s))) return st;
  if (bt && reads && (st = read_ints(bt, (size_t)B * bt_stride, t, s))) return st;
  for (int b = 0; b < B; ++b) {
    if (l[b] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "FA_DEBUG: cache_seqlens[%d] = %d is negative", b, l[b]);
    if (!reads) continue;
    const int64_t n = (int64_t)l[b] + S_new;
    const int64_t cap = bt ? (int64_t)bt_stride * page_size : num_blocks_or_smax;
    if (n > cap)
      return fail(FA_ERR_INVALID_ARGUMENT, "FA_DEBUG: sequence %d attends %lld tokens, the cache holds %lld", b,
                  (long long)n, (long long)cap);
    if (!bt) continue;
    for (int64_t pg = 0; pg * page_size < n; ++pg) {
      const int e = t[(size_t)b * bt_stride + pg];
      if (e < 0 || e >= num_blocks_or_smax)
        return fail(FA_ERR_INVALID_ARGUMENT, "FA_DEBUG: block_table[%d, %lld] = %d is outside the pool of %d pages", b,
                    (long long)pg, e, num_blocks_or_smax);
    }
  }
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "FA_ERR_WORKSPACE_TOO_SMALL";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "unknown fa_status";
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

fa_status fa_fwd(fa_dtype dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Sq, int Sk, int Hq, int Hkv, int D,
                 const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                 const int64_t* o_stride, const fa_attn_opts* opts, void* stream) {
  fa_status st = check_common(dtype, Hq, Hkv, D);
  if (st) return st;
  if (B < 0 || Sq < 0 || Sk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative size (B=%d Sq=%d Sk=%d)", B, Sq, Sk);
  float scale;
  if ((st = check_opts(opts, D, &scale))) return st;
  if (B == 0 || Sq == 0) return ok();
  if (!q || !out || !lse || (Sk > 0 && (!k || !v))) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(FA_ERR_UNSUPPORTED, "q/k/v/out must be 16-byte aligned");
  const int64_t qd[3] = {(int64_t)Sq * Hq * D, (int64_t)Hq * D, D};
  const int64_t kd[3] = {(int64_t)Sk * Hkv * D, (int64_t)Hkv * D, D};
  const int64_t* qs = q_stride ? q_stride : qd;
  const int64_t* ks = k_stride ? k_stride : kd;
  const int64_t* vs = v_stride ? v_stride : kd;
  const int64_t* os = o_stride ? o_stride : qd;
  if ((st = check_strides("q", qs, 3)) || (st = check_strides("k", ks, 3)) || (st = check_strides("v", vs, 3)) ||
      (st = check_strides("out", os, 3)))
    return st;
  const int bm = fa::prefill_block_m(D, (int64_t)B * Hq, Sq, device_cus(), key_span(opts));
  const int64_t nqt = (Sq + bm - 1) / bm;
  if (!dispatch_fits(nqt * Hq * (int64_t)B, 512)) return grid_too_large(nqt * Hq * (int64_t)B, 512);

  fa::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.q_sb = qs[0]; p.q_ss = qs[1]; p.q_sh = qs[2];
  p.k_sb = ks[0]; p.k_ss = ks[1]; p.k_sh = ks[2];
  p.v_sb = vs[0]; p.v_ss = vs[1]; p.v_sh = vs[2];
  p.o_sb = os[0]; p.o_ss = os[1]; p.o_sh = os[2];
  p.lse_sb = (int64_t)Hq * Sq; p.lse_sh = Sq;
  p.cu_seqlens_q = nullptr; p.cu_seqlens_k = nullptr;
  p.B = B; p.Sq = Sq; p.Sk = Sk; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  fill_opts(p, opts, scale);
  p.n_qtiles = (int)nqt;
  p.n_heads = B * Hq;
  p.block_m = bm;
  p.remap_xcd = (((int64_t)Hq * B) % 8) == 0;
  p.order_group = fa::order_group(p.causal != 0, (int64_t)Hq * B, nqt, p.remap_xcd != 0);
  return launch_status(fa::launch_prefill((fa::Dtype)dtype, D, p, (hipStream_t)stream), "prefill launch");
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D,
                     const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                     const int64_t* o_stride, float q_descale, float k_descale, float v_descale,
                     const fa_attn_opts* opts, void* stream) {
  fa_status st = check_common(FA_BF16, Hq, Hkv, D);
  if (st) return st;
  if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "fp8 head_dim %d not built (64 or 128)", D);
  if (B < 0 || Sq < 0 || Sk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative size (B=%d Sq=%d Sk=%d)", B, Sq, Sk);
  if (!(q_descale > 0.f) || !(k_descale > 0.f) || !(v_descale > 0.f) || !std::isfinite(q_descale) ||
      !std::isfinite(k_descale) || !std::isfinite(v_descale))
    return fail(FA_ERR_INVALID_ARGUMENT, "descale factors must be positive and finite");
  float scale;
  if ((st = check_opts(opts, D, &scale))) return st;
  if (B == 0 || Sq == 0) return ok();
  if (!q || !out || !lse || (Sk > 0 && (!k || !v))) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(FA_ERR_UNSUPPORTED, "q/k/v/out must be 16-byte aligned");
  const int64_t qd[3] = {(int64_t)Sq * Hq * D, (int64_t)Hq * D, D};
  const int64_t kd[3] = {(int64_t)Sk * Hkv * D, (int64_t)Hkv * D, D};
  const int64_t* qs = q_stride ? q_stride : qd;
  const int64_t* ks = k_stride ? k_stride : kd;
  const int64_t* vs = v_stride ? v_stride : kd;
  const int64_t* os = o_stride ? o_stride : qd;
  if ((st = check_strides("q", qs, 3)) || (st = check_strides("k", ks, 3)) || (st = check_strides("v", vs, 3)) ||
      (st = check_strides("out", os, 3)))
    return st;
  const int bm = fa::prefill_block_m_fp8(D);
  const int64_t nqt = (Sq + bm - 1) / bm;
  if (!dispatch_fits(nqt * Hq * (int64_t)B, 512)) return grid_too_large(nqt * Hq * (int64_t)B, 512);

  fa::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.q_sb = qs[0]; p.q_ss = qs[1]; p.q_sh = qs[2];
  p.k_sb = ks[0]; p.k_ss = ks[1]; p.k_sh = ks[2];
  p.v_sb = vs[0]; p.v_ss = vs[1]; p.v_sh = vs[2];
  p.o_sb = os[0]; p.o_ss = os[1]; p.o_sh = os[2];
  p.lse_sb = (int64_t)Hq * Sq; p.lse_sh = Sq;
  p.cu_seqlens_q = nullptr; p.cu_seqlens_k = nullptr;
  p.B = B; p.Sq = Sq; p.Sk = Sk; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  fill_opts(p, opts, scale * q_descale * k_descale);   // scores of the dequantised q and k
  p.out_scale = v_descale;
  p.n_qtiles = (int)nqt;
  p.n_heads = B * Hq;
  p.block_m = bm;
  p.remap_xcd = (((int64_t)Hq * B) % 8) == 0;
  p.order_group = fa::order_group(p.causal != 0, (int64_t)Hq * B, nqt, p.remap_xcd != 0);
  return launch_status(fa::launch_prefill_fp8(D, p, (hipStream_t)stream), "fp8 prefill launch");
}

fa_status fa_fwd_varlen(fa_dtype dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                        int Hq, int Hkv, int D,
                        const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                        const int64_t* o_stride, const fa_attn_opts* opts, void* stream) {
  fa_status st = check_common(dtype, Hq, Hkv, D);
  if (st) return st;
  if (B < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "negative size");
  float scale;
  if ((st = check_opts(opts, D, &scale))) return st;
  if (B == 0 || max_seqlen_q == 0 || total_q == 0) return ok();
  if (!q || !out || !lse || !cu_seqlens_q || !cu_seqlens_k || (total_k > 0 && (!k || !v)))
    return fail(FA_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(FA_ERR_UNSUPPORTED, "q/k/v/out must be 16-byte aligned");
  const int64_t qd[2] = {(int64_t)Hq * D, D};
  const int64_t kd[2] = {(int64_t)Hkv * D, D};
  const int64_t* qs = q_stride ? q_stride : qd;
  const int64_t* ks = k_stride ? k_stride : kd;
  const int64_t* vs = v_stride ? v_stride : kd;
  const int64_t* os = o_stride ? o_stride : qd;
  if ((st = check_strides("q", qs, 2)) || (st = check_strides("k", ks, 2)) || (st = check_strides("v", vs, 2)) ||
      (st = check_strides("out", os, 2)))
    return st;
  const int bm = fa::prefill_block_m(D, (int64_t)B * Hq, max_seqlen_q, device_cus(), key_span(opts));
  const int64_t nqt = (max_seqlen_q + bm - 1) / bm;
  if (!dispatch_fits(nqt * Hq * (int64_t)B, 512)) return grid_too_large(nqt * Hq * (int64_t)B, 512);
  if (debug_checks() && (st = debug_check_cu(cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, max_seqlen_k, total_q,
                                             total_k, (hipStream_t)stream)))
    return st;

  fa::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.q_sb = 0; p.q_ss = qs[0]; p.q_sh = qs[1];
  p.k_sb = 0; p.k_ss = ks[0]; p.k_sh = ks[1];
  p.v_sb = 0; p.v_ss = vs[0]; p.v_sh = vs[1];
  p.o_sb = 0; p.o_ss = os[0]; p.o_sh = os[1];
  p.lse_sb = 0; p.lse_sh = total_q;
  p.cu_seqlens_q = cu_seqlens_q; p.cu_seqlens_k = cu_seqlens_k;
  p.B = B; p.Sq = max_seqlen_q; p.Sk = max_seqlen_k; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  fill_opts(p, opts, scale);
  p.n_qtiles = (int)nqt;
  p.n_heads = B * Hq;
  p.block_m = bm;
  p.remap_xcd = (((int64_t)Hq * B) % 8) == 0;
  p.order_group = fa::order_group(p.causal != 0, (int64_t)Hq * B, nqt, p.remap_xcd != 0);
  return launch_status(fa::launch_prefill((fa::Dtype)dtype, D, p, (hipStream_t)stream), "varlen prefill launch");
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t fa_kvcache_workspace_size(int B, int Sq, int Hq, int D, int num_splits) {
  if (B <= 0 || Sq <= 0 || Hq <= 0 || D <= 0 || num_splits <= 0) return 0;
  const size_t rows = (size_t)B * Sq * Hq * num_splits;
  return align256(rows * D * sizeof(float)) + align256(rows * sizeof(float)) + align256((size_t)B * 2 * sizeof(int));
}

int fa_kvcache_num_splits(int B, int Hkv, int max_seqlen_k, int num_splits) {
  if (num_splits > 0) return num_splits;
  const int64_t groups = (int64_t)(B > 0 ? B : 1) * (Hkv > 0 ? Hkv : 1);
  int64_t n = (1024 + groups - 1) / groups;              // ~4 workgroups per CU
  const int64_t by_len = (int64_t)(max_seqlen_k > 0 ? max_seqlen_k : 1) / 64;
  if (n > by_len) n = by_len;
  if (n < 1) n = 1;
  if (n > 64) n = 64;
  return (int)n;
}

}  // extern "C"

// The decode path of fa_fwd_kvcache and fa_fwd_kvcache_append: optionally
// append S_new new tokens (k_new/v_new non-null), then split-KV decode over
// cache_seqlens[b] + S_new tokens and the LSE combine.
static fa_status kvcache_impl(fa_dtype dtype, const void* q, void* k_cache, void* v_cache,
                              const int* cache_seqlens, const int* block_table, int block_table_stride,
                              int page_size, int num_blocks_or_smax, int num_splits,
                              void* workspace, size_t workspace_bytes, void* out, float* lse,
                              int B, int Sq, int Hq, int Hkv, int D, const fa_attn_opts* opts, void* stream,
                              const void* k_new, const void* v_new, int S_new,
                              const int64_t* kn_stride, const int64_t* vn_stride) {
  fa_status st = check_common(dtype, Hq, Hkv, D);
  if (st) return st;
  if (B < 0 || Sq < 0 || num_blocks_or_smax < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative size");
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARGUMENT, "num_splits must be >= 0");
  if (num_splits > 64) return fail(FA_ERR_UNSUPPORTED, "num_splits %d > 64", num_splits);
  if (block_table && (page_size <= 0 || block_table_stride <= 0))
    return fail(FA_ERR_INVALID_ARGUMENT, "paged cache needs page_size > 0 and block_table_stride > 0");
  float scale;
  if ((st = check_opts(opts, D, &scale))) return st;
  // the decode works on at most 16 query rows per work item: the query heads of
  // a kv head are split into kv_split groups (each reading the same K/V) when
  // (Hq/Hkv)*Sq is larger
  const int G = Hq / Hkv;
  int kv_split = 1;
  while (kv_split <= G && (G % kv_split != 0 || (int64_t)(G / kv_split) * Sq > 16)) ++kv_split;
  if (kv_split > G)
    return fail(FA_ERR_UNSUPPORTED, "Sq = %d query positions per kv head; at most 16 are built", Sq);
  // the other way round, for head rows of at most 128 bytes (D <= 64) when a kv
  // head has few query rows and the caller vouches that the cache is finite
  // (opts->finite_cache): 2, 4 or 8 adjacent kv heads form one work head, which
  // reads their rows of a token as one run of hpi*D elements (longer contiguous
  // reads stream faster), as long as the run stays within 256 elements and the
  // rows within 16.  A query then meets the other heads' elements with zeros, so
  // a non-finite value there would reach its sum; without the promise every
  // work head reads its own kv head only.  The choice depends on the shapes and
  // that flag, never on the cache layout, so a paged cache and its dense
  // equivalent give the same bits.
  int hpi = 1;
  if (opts && opts->finite_cache && kv_split == 1 && (D == 32 || D == 64))
    while (D * hpi * 2 <= 256 && Hkv % (hpi * 2) == 0 && (int64_t)G * Sq * hpi * 2 <= 16) hpi *= 2;
  if ((int64_t)B * Sq * Hq * D * 2 > ((int64_t)1 << 31))
    return fail(FA_ERR_UNSUPPORTED, "q of %lld bytes; the decode takes at most 2^31",
                (long long)B * Sq * Hq * D * 2);
  if (S_new < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative number of new tokens");
  if (S_new > 0 && (!k_new || !v_new)) return fail(FA_ERR_INVALID_ARGUMENT, "null k_new / v_new");
  const int64_t knd[3] = {(int64_t)S_new * Hkv * D, (int64_t)Hkv * D, D};
  const int64_t* kns = kn_stride ? kn_stride : knd;
  const int64_t* vns = vn_stride ? vn_stride : knd;
  if (S_new > 0) {
    for (int i = 0; i < 3; ++i) {
      if (kns[i] < 0 || vns[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative k_new / v_new stride");
      if (kns[i] % 8 || vns[i] % 8)
        return fail(FA_ERR_UNSUPPORTED, "k_new / v_new strides must be multiples of 8 elements");
    }
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(FA_ERR_UNSUPPORTED, "k_new / v_new must be 16-byte aligned");
  }
  if (B == 0 || (Sq == 0 && S_new == 0)) return ok();
  if (!k_cache || !v_cache || !cache_seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(FA_ERR_UNSUPPORTED, "k_cache/v_cache must be 16-byte aligned");
  if (S_new > 0 && num_blocks_or_smax == 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "new tokens for an empty cache");
  if (S_new > 0 && !dispatch_fits(((int64_t)B * S_new * Hkv * (D / 8) + 255) / 256, 256))
    return grid_too_large(((int64_t)B * S_new * Hkv * (D / 8) + 255) / 256, 256);
  // everything the decode needs is checked before anything is launched
  int ns = 0;
  if (Sq > 0) {
    if (!q || !out || !lse) return fail(FA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(q)) return fail(FA_ERR_UNSUPPORTED, "q must be 16-byte aligned");
    const int smax_bound = block_table ? block_table_stride * page_size : num_blocks_or_smax;
    ns = fa_kvcache_num_splits(B, Hkv, smax_bound, num_splits);
    const size_t need = fa_kvcache_workspace_size(B, Sq, Hq, D, ns);
    if (!workspace) return fail(FA_ERR_INVALID_ARGUMENT, "null workspace");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(FA_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    // the decode schedule numbers work items (b, split, kv head) and rounds in int
    if ((int64_t)B * ns * Hkv * kv_split > (int64_t)1 << 30)
      return fail(FA_ERR_UNSUPPORTED, "B*num_splits*Hkv = %lld work items; at most 2^30 are built",
                  (long long)B * ns * Hkv * kv_split);
  }

  hipStream_t s = (hipStream_t)stream;
  if (debug_checks() && (st = debug_check_cache(cache_seqlens, block_table, block_table_stride, page_size,
                                                num_blocks_or_smax, B, S_new, Sq > 0, s)))
    return st;
  if (S_new > 0) {
    fa::AppendParams a{};
    a.k_new = k_new; a.v_new = v_new;
    a.kn_sb = kns[0]; a.kn_ss = kns[1]; a.kn_sh = kns[2];
    a.vn_sb = vns[0]; a.vn_ss = vns[1]; a.vn_sh = vns[2];
    a.k_cache = k_cache; a.v_cache = v_cache;
    a.cache_seqlens = cache_seqlens;
    a.block_table = block_table; a.bt_stride = block_table_stride; a.page_size = page_size;
    a.num_blocks = block_table ? num_blocks_or_smax : 0;
    a.smax = block_table ? 0 : num_blocks_or_smax;
    a.B = B; a.S = S_new; a.Hkv = Hkv; a.D = D;
    hipError_t e = fa::launch_append(a, s);
    if (e != hipSuccess) return launch_status(e, "append launch");
  }
  if (Sq == 0) return ok();

  const size_t rows = (size_t)B * Sq * Hq * ns;
  char* ws = static_cast<char*>(workspace);
  float* op = reinterpret_cast<float*>(ws);
  float* lp = reinterpret_cast<float*>(ws + align256(rows * D * sizeof(float)));
  int2* order = reinterpret_cast<int2*>(ws + align256(rows * D * sizeof(float)) + align256(rows * sizeof(float)));

  fa::DecodeParams d{};
  d.q = q; d.k = k_cache; d.v = v_cache;
  // the decode kernel may read row 0 of the cache past the end of its work; an
  // empty cache (every sequence of length 0) gets q as a stand-in
  if (num_blocks_or_smax == 0) { d.k = q; d.v = q; }
  d.cache_seqlens = cache_seqlens;
  d.seqlen_add = S_new;
  d.block_table = block_table;
  d.bt_stride = block_table_stride;
  d.page_size = block_table ? page_size : num_blocks_or_smax;
  d.cache_rows = (int64_t)num_blocks_or_smax * (block_table ? page_size : B);
  d.log2_page = -1;
  if (block_table && (page_size & (page_size - 1)) == 0) {
    int lg = 0;
    while ((1 << lg) < page_size) ++lg;
    d.log2_page = lg;
  }
  d.out_partial = op; d.lse_partial = lp;
  d.order = B > 64 ? order : nullptr;   // up to 64 sequences are ranked inside the decode kernel
  d.B = B; d.Sq = Sq; d.Hq = Hq; d.Hkv = Hkv * kv_split / hpi; d.group = G / kv_split * hpi;
  d.kv_heads = Hkv / hpi; d.kv_split = kv_split;
  d.head_dim = D;
  d.head_shift = 30;
  if (hpi > 1) {
    d.head_shift = 0;
    while ((1 << d.head_shift) < D) ++d.head_shift;
  }
  d.num_splits = ns;
  d.scale = scale;
  d.softcap = opts ? opts->softcap : 0.f;
  d.alibi = opts ? opts->alibi_slopes : nullptr;
  d.causal = opts ? (opts->causal != 0) : 0;
  d.wl = window_side(opts, true);
  d.wr = window_side(opts, false);
  hipError_t e = fa::launch_decode((fa::Dtype)dtype, D * hpi, d, s);
  if (e != hipSuccess) return launch_status(e, "decode launch");

  fa::CombineParams c{};
  c.out_partial = op; c.lse_partial = lp;
  c.op_sn = D; c.op_sd = 1; c.op_sh = (int64_t)ns * D; c.op_ss = c.op_sh * Hq; c.op_sb = c.op_ss * Sq;
  c.lp_sn = 1; c.lp_sh = ns; c.lp_ss = (int64_t)ns * Hq; c.lp_sb = c.lp_ss * Sq;
  c.out = out;
  c.o_sh = D; c.o_ss = (int64_t)Hq * D; c.o_sb = c.o_ss * Sq;
  c.lse = lse;
  c.l_sh = Sq; c.l_ss = 1; c.l_sb = (int64_t)Hq * Sq;
  c.B = B; c.S = Sq; c.H = Hq; c.D = D; c.num_splits = ns;
  return launch_status(fa::launch_combine((fa::Dtype)dtype, c, s), "combine launch");
}

extern "C" {

fa_status fa_fwd_kvcache(fa_dtype dtype, const void* q, const void* k_cache, const void* v_cache,
                         const int* cache_seqlens, const int* block_table, int block_table_stride,
                         int page_size, int num_blocks_or_smax, int num_splits,
                         void* workspace, size_t workspace_bytes, void* out, float* lse,
                         int B, int Sq, int Hq, int Hkv, int D, const fa_attn_opts* opts, void* stream) {
  return kvcache_impl(dtype, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), cache_seqlens, block_table,
                      block_table_stride, page_size, num_blocks_or_smax, num_splits, workspace, workspace_bytes,
                      out, lse, B, Sq, Hq, Hkv, D, opts, stream, nullptr, nullptr, 0, nullptr, nullptr);
}

// ---- fa_fwd_kvcache_noalloc: the decode workspace in a static device array.
// In host code `scratch` is a host-side stand-in for the array, not a device
// address: kernels are handed the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in g_scratch_dev.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static std::atomic<void*> g_scratch_dev[kScratchDevices];
static std::mutex g_scratch_mu;

static fa_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(FA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev, kScratchDevices - 1);
  void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      g_scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return FA_OK;
}

size_t fa_kvcache_noalloc_max_bytes(void) { return kScratchBytes; }

fa_status fa_fwd_kvcache_noalloc(fa_dtype dtype, const void* q, const void* k_cache, const void* v_cache,
                                 const int* cache_seqlens, const int* block_table, int block_table_stride,
                                 int page_size, int num_blocks_or_smax, int num_splits, void* out, float* lse,
                                 int B, int Sq, int Hq, int Hkv, int D, const fa_attn_opts* opts, void* stream) {
  fa_status st = check_common(dtype, Hq, Hkv, D);
  if (st) return st;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // sizes that describe work (the rest is validated, or is a no-op, in the shared path)
  if (B > 0 && Sq > 0 && num_splits >= 0 && num_splits <= 64 && num_blocks_or_smax >= 0 &&
      (!block_table || (page_size > 0 && block_table_stride > 0))) {
    const int cap = block_table ? block_table_stride * page_size : num_blocks_or_smax;
    const int ns = fa_kvcache_num_splits(B, Hkv, cap, num_splits);
    const size_t need = fa_kvcache_workspace_size(B, Sq, Hq, D, ns);
    if (need > kScratchBytes)
      return fail(FA_ERR_UNSUPPORTED, "the decode needs %zu bytes of workspace; the static scratch holds %zu", need,
                  kScratchBytes);
    if ((st = scratch_of_current_device(&ws))) return st;
    ws_bytes = kScratchBytes;
  }
  return kvcache_impl(dtype, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), cache_seqlens, block_table,
                      block_table_stride, page_size, num_blocks_or_smax, num_splits, ws, ws_bytes, out, lse, B, Sq,
                      Hq, Hkv, D, opts, stream, nullptr, nullptr, 0, nullptr, nullptr);
}

fa_status fa_fwd_kvcache_append(fa_dtype dtype, const void* q, void* k_cache, void* v_cache,
                                const int* cache_seqlens, const int* block_table, int block_table_stride,
                                int page_size, int num_blocks_or_smax, int num_splits,
                                const void* k_new, const void* v_new, int S_new,
                                const int64_t* kn_stride, const int64_t* vn_stride,
                                void* workspace, size_t workspace_bytes, void* out, float* lse,
                                int B, int Sq, int Hq, int Hkv, int D, const fa_attn_opts* opts, void* stream) {
  return kvcache_impl(dtype, q, k_cache, v_cache, cache_seqlens, block_table, block_table_stride, page_size,
                      num_blocks_or_smax, num_splits, workspace, workspace_bytes, out, lse, B, Sq, Hq, Hkv, D,
                      opts, stream, k_new, v_new, S_new, kn_stride, vn_stride);
}

size_t fa_bwd_workspace_size(int B, int Sq, int Hq) {
  if (B <= 0 || Sq <= 0 || Hq <= 0) return 0;
  return ((size_t)B * Hq * Sq * sizeof(float) + 255) & ~(size_t)255;
}

fa_status fa_bwd(fa_dtype dtype, const void* dout, const void* q, const void* k, const void* v, const void* out,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                 const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                 const int64_t* o_stride, const int64_t* do_stride, const fa_attn_opts* opts,
                 void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(dtype, Hq, Hkv, D);
  if (st) return st;
  if (B < 0 || Sq < 0 || Sk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative size (B=%d Sq=%d Sk=%d)", B, Sq, Sk);
  float scale;
  if ((st = check_opts(opts, D, &scale))) return st;
  if (B == 0 || (Sq == 0 && Sk == 0)) return ok();
  if (Sq > 0 && (!q || !dout || !out || !lse || !dq))
    return fail(FA_ERR_INVALID_ARGUMENT, "null q/dout/out/lse/dq pointer");
  if (Sk > 0 && (!k || !v || !dk || !dv)) return fail(FA_ERR_INVALID_ARGUMENT, "null k/v/dk/dv pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(FA_ERR_UNSUPPORTED, "q/k/v/out/dout/dq/dk/dv must be 16-byte aligned");
  const int64_t qd[3] = {(int64_t)Sq * Hq * D, (int64_t)Hq * D, D};
  const int64_t kd[3] = {(int64_t)Sk * Hkv * D, (int64_t)Hkv * D, D};
  const int64_t* qs = q_stride ? q_stride : qd;
  const int64_t* ks = k_stride ? k_stride : kd;
  const int64_t* vs = v_stride ? v_stride : kd;
  const int64_t* os = o_stride ? o_stride : qd;
  const int64_t* gs = do_stride ? do_stride : qd;
  if ((st = check_strides("q", qs, 3)) || (st = check_strides("k", ks, 3)) || (st = check_strides("v", vs, 3)) ||
      (st = check_strides("out", os, 3)) || (st = check_strides("dout", gs, 3)))
    return st;
  const size_t need = fa_bwd_workspace_size(B, Sq, Hq);
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_INVALID_ARGUMENT, "null workspace");
    if (!aligned16(workspace)) return fail(FA_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  }
  const int bn = fa::backward_block_n(D), bm = fa::backward_block_m(D);
  const int64_t nkt = (Sk + bn - 1) / bn, nqt = (Sq + bm - 1) / bm;
  if (!dispatch_fits(nkt * B * (int64_t)Hkv, 512) || !dispatch_fits(nqt * B * (int64_t)Hq, 512) ||
      !dispatch_fits(((int64_t)B * Sq * Hq * (D / 8) + 255) / 256, 256))
    return grid_too_large(std::max(nkt * B * (int64_t)Hkv, nqt * B * (int64_t)Hq), 512);

  fa::BackwardParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.delta = (float*)workspace;
  p.q_sb = qs[0]; p.q_ss = qs[1]; p.q_sh = qs[2];
  p.k_sb = ks[0]; p.k_ss = ks[1]; p.k_sh = ks[2];
  p.v_sb = vs[0]; p.v_ss = vs[1]; p.v_sh = vs[2];
  p.o_sb = os[0]; p.o_ss = os[1]; p.o_sh = os[2];
  p.do_sb = gs[0]; p.do_ss = gs[1]; p.do_sh = gs[2];
  p.dq_sb = qd[0]; p.dq_ss = qd[1]; p.dq_sh = qd[2];
  p.dk_sb = kd[0]; p.dk_ss = kd[1]; p.dk_sh = kd[2];
  p.dv_sb = kd[0]; p.dv_ss = kd[1]; p.dv_sh = kd[2];
  p.lse_sb = (int64_t)Hq * Sq; p.lse_sh = Sq;
  p.dl_sb = (int64_t)Hq * Sq; p.dl_sh = Sq;
  p.cu_seqlens_q = nullptr; p.cu_seqlens_k = nullptr;
  p.B = B; p.Sq = Sq; p.Sk = Sk; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.scale = scale;
  p.softcap = opts ? opts->softcap : 0.f;
  p.alibi = opts ? opts->alibi_slopes : nullptr;
  p.causal = opts ? (opts->causal != 0) : 0;
  p.wl = window_side(opts, true);
  p.wr = window_side(opts, false);
  p.n_ktiles = (int)nkt;
  p.n_qtiles = (int)nqt;
  return launch_status(fa::launch_backward((fa::Dtype)dtype, D, p, (hipStream_t)stream), "backward launch");
}

fa_status fa_bwd_varlen(fa_dtype dtype, const void* dout, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, void* dq, void* dk, void* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                        int max_seqlen_k, int total_q, int total_k, int Hq, int Hkv, int D,
                        const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                        const int64_t* o_stride, const int64_t* do_stride, const fa_attn_opts* opts,
                        void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(dtype, Hq, Hkv, D);
  if (st) return st;
  if (B < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "negative size");
  float scale;
  if ((st = check_opts(opts, D, &scale))) return st;
  if (B == 0 || (total_q == 0 && total_k == 0)) return ok();
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(FA_ERR_INVALID_ARGUMENT, "null cu_seqlens pointer");
  if (total_q > 0 && (!q || !dout || !out || !lse || !dq))
    return fail(FA_ERR_INVALID_ARGUMENT, "null q/dout/out/lse/dq pointer");
  if (total_k > 0 && (!k || !v || !dk || !dv)) return fail(FA_ERR_INVALID_ARGUMENT, "null k/v/dk/dv pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(FA_ERR_UNSUPPORTED, "q/k/v/out/dout/dq/dk/dv must be 16-byte aligned");
  const int64_t qd[2] = {(int64_t)Hq * D, D};
  const int64_t kd[2] = {(int64_t)Hkv * D, D};
  const int64_t* qs = q_stride ? q_stride : qd;
  const int64_t* ks = k_stride ? k_stride : kd;
  const int64_t* vs = v_stride ? v_stride : kd;
  const int64_t* os = o_stride ? o_stride : qd;
  const int64_t* gs = do_stride ? do_stride : qd;
  if ((st = check_strides("q", qs, 2)) || (st = check_strides("k", ks, 2)) || (st = check_strides("v", vs, 2)) ||
      (st = check_strides("out", os, 2)) || (st = check_strides("dout", gs, 2)))
    return st;
  const size_t need = fa_bwd_workspace_size(1, total_q, Hq);
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_INVALID_ARGUMENT, "null workspace");
    if (!aligned16(workspace)) return fail(FA_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  }
  const int bn = fa::backward_block_n(D), bm = fa::backward_block_m(D);
  const int64_t nkt = (max_seqlen_k + bn - 1) / bn, nqt = (max_seqlen_q + bm - 1) / bm;
  if (!dispatch_fits(nkt * B * (int64_t)Hkv, 512) || !dispatch_fits(nqt * B * (int64_t)Hq, 512) ||
      !dispatch_fits(((int64_t)total_q * Hq * (D / 8) + 255) / 256, 256))
    return grid_too_large(std::max(nkt * B * (int64_t)Hkv, nqt * B * (int64_t)Hq), 512);
  if (debug_checks() && (st = debug_check_cu(cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, max_seqlen_k, total_q,
                                             total_k, (hipStream_t)stream)))
    return st;

  fa::BackwardParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.delta = (float*)workspace;
  p.q_sb = 0; p.q_ss = qs[0]; p.q_sh = qs[1];
  p.k_sb = 0; p.k_ss = ks[0]; p.k_sh = ks[1];
  p.v_sb = 0; p.v_ss = vs[0]; p.v_sh = vs[1];
  p.o_sb = 0; p.o_ss = os[0]; p.o_sh = os[1];
  p.do_sb = 0; p.do_ss = gs[0]; p.do_sh = gs[1];
  p.dq_sb = 0; p.dq_ss = qd[0]; p.dq_sh = qd[1];
  p.dk_sb = 0; p.dk_ss = kd[0]; p.dk_sh = kd[1];
  p.dv_sb = 0; p.dv_ss = kd[0]; p.dv_sh = kd[1];
  p.lse_sb = 0; p.lse_sh = total_q;
  p.dl_sb = 0; p.dl_sh = total_q;
  p.cu_seqlens_q = cu_seqlens_q; p.cu_seqlens_k = cu_seqlens_k;
  p.B = B; p.Sq = max_seqlen_q; p.Sk = max_seqlen_k; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.scale = scale;
  p.softcap = opts ? opts->softcap : 0.f;
  p.alibi = opts ? opts->alibi_slopes : nullptr;
  p.causal = opts ? (opts->causal != 0) : 0;
  p.wl = window_side(opts, true);
  p.wr = window_side(opts, false);
  p.n_ktiles = (int)nkt;
  p.n_qtiles = (int)nqt;
  return launch_status(fa::launch_backward((fa::Dtype)dtype, D, p, (hipStream_t)stream), "varlen backward launch");
}

fa_status fa_combine(const float* out_partial, const float* lse_partial, int B, int S, int H, int D,
                     int num_splits, const int64_t* op_stride, const int64_t* lp_stride,
                     fa_dtype out_dtype, void* out, const int64_t* o_stride, float* lse, void* stream) {
  if (out_dtype != FA_F16 && out_dtype != FA_BF16) return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype %d", out_dtype);
  if (B < 0 || S < 0 || H < 0 || D <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "bad size");
  if (num_splits < 1) return fail(FA_ERR_INVALID_ARGUMENT, "num_splits must be >= 1");
  if (num_splits > 64) return fail(FA_ERR_UNSUPPORTED, "num_splits %d > 64", num_splits);
  if ((int64_t)B * S * H == 0) return ok();
  if (!out_partial || !lse_partial || !out) return fail(FA_ERR_INVALID_ARGUMENT, "null pointer");
  const int64_t opd[5] = {(int64_t)S * H * D * num_splits, (int64_t)H * D * num_splits, (int64_t)D * num_splits,
                          num_splits, 1};
  const int64_t lpd[4] = {(int64_t)S * H * num_splits, (int64_t)H * num_splits, num_splits, 1};
  const int64_t od[3] = {(int64_t)S * H * D, (int64_t)H * D, D};
  const int64_t* os = op_stride ? op_stride : opd;
  const int64_t* ls = lp_stride ? lp_stride : lpd;
  const int64_t* oo = o_stride ? o_stride : od;
  for (int i = 0; i < 5; ++i)
    if (os[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative out_partial stride");
  for (int i = 0; i < 4; ++i)
    if (ls[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative lse_partial stride");
  for (int i = 0; i < 3; ++i)
    if (oo[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative out stride");
  if (!dispatch_fits(((int64_t)B * S * H + 3) / 4, 256)) return grid_too_large(((int64_t)B * S * H + 3) / 4, 256);
  fa::CombineParams c{};
  c.out_partial = out_partial; c.lse_partial = lse_partial;
  c.op_sb = os[0]; c.op_ss = os[1]; c.op_sh = os[2]; c.op_sd = os[3]; c.op_sn = os[4];
  c.lp_sb = ls[0]; c.lp_ss = ls[1]; c.lp_sh = ls[2]; c.lp_sn = ls[3];
  c.out = out; c.o_sb = oo[0]; c.o_ss = oo[1]; c.o_sh = oo[2];
  c.lse = lse; c.l_sb = (int64_t)S * H; c.l_ss = H; c.l_sh = 1;
  c.B = B; c.S = S; c.H = H; c.D = D; c.num_splits = num_splits;
  return launch_status(fa::launch_combine((fa::Dtype)out_dtype, c, (hipStream_t)stream), "combine launch");
}

}  // extern "C"
