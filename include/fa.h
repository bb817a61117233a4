/*
 * fa.h -- C ABI of the MI355X (gfx950) exact attention forward library, libfa.so.
 *
 * The library computes exact attention, out = softmax(scale * Q Kᵀ) V, tile by
 * tile with an online softmax so that the Sq x Sk score matrix never reaches
 * HBM, and returns the per-row log-sum-exp next to the output.  The calls and
 * their options follow the Python interface described on
 * "FlashAttention 常用接口简单介绍" (xllm-io.github.io): §3.1 flash_attn_func,
 * §3.2 flash_attn_varlen_func, §3.3 flash_attn_with_kvcache, §3.4
 * flash_attn_combine; the option semantics come from the Flash-Attention
 * v2.0-v2.7 update notes (framerc.cn): bottom-right causal alignment, v2.2
 * split-KV, v2.3 sliding window, v2.4 ALiBi, v2.5 paged KV cache, v2.6 softcap.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains device memory, and inputs are read-only.
 *  - Element type: fa_dtype (fp16 or bf16) for q/k/v/out; float32 for lse,
 *    ALiBi slopes and the decode workspace; int32 for cu_seqlens,
 *    cache_seqlens and block_table.
 *  - Head dimension D: 32, 64, 96, 128 or 256 for fa_fwd, fa_fwd_varlen, the
 *    KV-cache calls, fa_bwd and fa_bwd_varlen; any D for fa_combine.  Other values return
 *    FA_ERR_UNSUPPORTED.  The head-dim stride is 1 and row starts must be
 *    16-byte aligned (strides multiples of 8 elements, base pointers 16-byte
 *    aligned).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns without synchronising; results
 *    are valid once the stream has reached that point.
 *  - Every element of out and lse is written, including rows that have no
 *    allowed key: out = 0 and lse = -inf there.
 *  - Errors: host-side checks run before anything is enqueued; on any error
 *    nothing is launched and a status other than FA_OK is returned, with a
 *    thread-local message available from fa_last_error().  B == 0 or an empty
 *    query side is a valid no-op.  Device-side contents (monotonic cu_seqlens,
 *    in-range block_table entries, cache_seqlens within the cache) are the
 *    caller's contract and are not checked, except with the environment
 *    variable FA_DEBUG=1: then the varlen and KV-cache calls copy them back
 *    (synchronising the stream) and return FA_ERR_INVALID_ARGUMENT, with
 *    nothing launched, if they are inconsistent.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, Hq % Hkv != 0, window < -1, ... */
  FA_ERR_UNSUPPORTED = 2,        /* valid but not built: D not in {32,64,96,128,256}, misalignment, ... */
  FA_ERR_WORKSPACE_TOO_SMALL = 3,/* decode workspace below fa_kvcache_workspace_size() */
  FA_ERR_HIP = 4                 /* a HIP launch error; fa_last_error() carries its text */
} fa_status;

typedef enum {
  FA_F16 = 0,
  FA_BF16 = 1,
  /* range markers (not types): they make every int32 value a valid fa_dtype, so
   * an unknown code is reported as FA_ERR_INVALID_ARGUMENT, never undefined */
  FA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  FA_DTYPE_RANGE_MAX_ = 0x7fffffff
} fa_dtype;

/* Attention options ("FlashAttention 常用接口简单介绍", §3.1 keyword arguments). */
typedef struct {
  float softmax_scale;          /* 0 selects the default 1/sqrt(D); negative is invalid          */
  int causal;                   /* nonzero: key j allowed for query i iff j <= i + Sk - Sq       */
  int window_left;              /* local window: keys in [i' - left, i' + right], i' = i + Sk - Sq; */
  int window_right;             /*   -1 = unbounded on that side; both -1 = global attention    */
  float softcap;                /* > 0: score s becomes softcap * tanh(s / softcap); 0 = off    */
  const float* alibi_slopes;    /* device float32 [Hq]: score -= slope[h] * |i' - j|; NULL = off */
  int finite_cache;             /* KV-cache calls only: nonzero promises that the K and V values   */
                                /*   of every attended token are finite, which lets the decode at */
                                /*   D = 32 or 64 read 2-8 adjacent kv heads as one work item;    */
                                /*   0 = each kv head is read alone                               */
} fa_attn_opts;

/*
 * Dense forward ("FlashAttention 常用接口简单介绍", §3.1 flash_attn_func).
 *   q   [B, Sq, Hq, D], k/v [B, Sk, Hkv, D], out [B, Sq, Hq, D] (dtype),
 *   lse [B, Hq, Sq] float32, contiguous.
 *   *_stride: element strides of the (batch, sequence, head) dimensions; NULL
 *   means the contiguous [B, S, H, D] layout.
 *   Hkv must divide Hq (GQA/MQA: query head h reads kv head h / (Hq/Hkv)).
 *   opts may be NULL (defaults: scale 1/sqrt(D), no mask, no softcap, no ALiBi).
 */
fa_status fa_fwd(fa_dtype dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Sq, int Sk, int Hq, int Hkv, int D,
                 const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                 const int64_t* o_stride, const fa_attn_opts* opts, void* stream);

/*
 * Dense forward on fp8 inputs ("optimizing-attention-flash" skill page, workflow
 * three: q, k and v converted to float8_e4m3fn and passed to the forward).
 *   q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D] in OCP fp8 e4m3 (float8_e4m3fn, one
 *   byte per element); out [B, Sq, Hq, D] bf16; lse [B, Hq, Sq] float32.
 *   The pages give no scaling recipe.  Reading: each tensor carries one
 *   positive descale factor (the real value is code value * descale; 1 when the
 *   tensor was converted directly, as on the pages), and the result is the
 *   exact attention of the dequantised tensors: scores are
 *   softmax_scale * q_descale * k_descale * (q . k), out is v_descale times
 *   the softmax average of the v codes, lse is of the dequantised scores.
 *   Q Kᵀ runs on the fp8 MFMA with fp32 accumulation (exact products); V is
 *   widened exactly to bf16 and P rounded to bf16 for P V, as in the bf16 path.
 *   D is 64 or 128.  Strides, alignment, options and errors are those of
 *   fa_fwd; strides count elements (bytes here) and must be multiples of 8.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D,
                     const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                     const int64_t* o_stride, float q_descale, float k_descale, float v_descale,
                     const fa_attn_opts* opts, void* stream);

/*
 * Packed variable-length forward ("FlashAttention 常用接口简单介绍", §3.2).
 *   q [total_q, Hq, D], k/v [total_k, Hkv, D], out [total_q, Hq, D],
 *   lse [Hq, total_q] float32.  cu_seqlens_q/k: device int32 [B+1] prefix sums;
 *   sequence b owns rows [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]) and
 *   is masked/aligned on its own lengths.  max_seqlen_q/k bound every
 *   sequence's length (the grid is sized from max_seqlen_q).
 *   *_stride: element strides of the (token, head) dimensions; NULL = contiguous.
 */
fa_status fa_fwd_varlen(fa_dtype dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                        int Hq, int Hkv, int D,
                        const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                        const int64_t* o_stride, const fa_attn_opts* opts, void* stream);

/* Bytes of workspace fa_fwd_kvcache needs: the float32 out partials
 * [B, Sq, Hq, num_splits, D], the float32 lse partials [B, Sq, Hq, num_splits]
 * and the int32 schedule order [B, 2], each padded to 256 bytes; about
 * B*Sq*Hq*num_splits*(D+1)*4.  num_splits as passed to fa_fwd_kvcache after
 * resolving 0 (see fa_kvcache_num_splits). */
size_t fa_kvcache_workspace_size(int B, int Sq, int Hq, int D, int num_splits);

/* The split count fa_fwd_kvcache uses when passed num_splits = 0, for a cache
 * whose sequences hold at most max_seqlen_k tokens: enough workgroups to fill
 * the GPU, at least 64 tokens per split, at most 64 splits. */
int fa_kvcache_num_splits(int B, int Hkv, int max_seqlen_k, int num_splits);

/*
 * Decode against a KV cache ("FlashAttention 常用接口简单介绍", §3.3), split along
 * the cache sequence into num_splits chunks (update notes, v2.2) and merged by
 * a separate LSE-weighted combine kernel (§3.4).
 *   q [B, Sq, Hq, D] contiguous, out [B, Sq, Hq, D] contiguous, lse [B, Hq, Sq].
 *   block_table == NULL: k_cache/v_cache are dense [B, num_blocks_or_smax, Hkv, D].
 *   block_table != NULL: k_cache/v_cache are page pools [num_blocks_or_smax,
 *     page_size, Hkv, D] and block_table is int32 [B, block_table_stride]; token
 *     t of sequence b lives in page block_table[b, t / page_size], row
 *     t % page_size (update notes, v2.5).
 *   cache_seqlens: device int32 [B], tokens attended per sequence; the Sq
 *     queries are bottom-right aligned against them.
 *   num_splits: 1..64, or 0 for fa_kvcache_num_splits().  Sq <= 16 when each
 *   kv head has one query head; otherwise any Sq with (Hq/Hkv)*Sq rows that
 *   can be split over work items of at most 16 rows (the query heads of a kv
 *   head are split into groups, each group reading the same cache rows);
 *   FA_ERR_UNSUPPORTED if none.
 *   workspace: device memory of at least fa_kvcache_workspace_size() bytes,
 *     256-byte aligned, any contents; it holds the per-split partials between
 *     the kernels.  Calls sharing a workspace must not overlap in time.
 *   B*num_splits*Hkv*(query-head groups per kv head) <= 2^30, and q holds at
 *   most 2^31 bytes (B*Sq*Hq*D*2); FA_ERR_UNSUPPORTED otherwise.
 *   Arithmetic: each query head's scores take its own kv head's keys only.
 *   With opts->finite_cache set, at D = 32 and 64 and few query rows per kv
 *   head, 2, 4 or 8 adjacent kv heads (at most 256 elements together, at most
 *   16 rows) are read as one work item and each query meets the other heads'
 *   elements with zeros: exact for finite caches, while one Inf or NaN in a
 *   neighbouring head would then reach every head of the item.
 *   num_splits = 0 resolves with max_seqlen_k = the cache capacity
 *   (block_table_stride * page_size, or Smax); a paged cache and a dense cache
 *   of equal capacity take the same split count and give the same bits.
 */
fa_status fa_fwd_kvcache(fa_dtype dtype, const void* q, const void* k_cache, const void* v_cache,
                         const int* cache_seqlens, const int* block_table, int block_table_stride,
                         int page_size, int num_blocks_or_smax, int num_splits,
                         void* workspace, size_t workspace_bytes, void* out, float* lse,
                         int B, int Sq, int Hq, int Hkv, int D, const fa_attn_opts* opts, void* stream);

/*
 * fa_fwd_kvcache with new keys and values appended first ("FlashAttention
 * 常用接口简单介绍", §3.3: the optional k and v that update the cache).
 *   k_new, v_new: [B, S_new, Hkv, D] of dtype; kn_stride / vn_stride give the
 *     element strides of (batch, token, head), NULL = contiguous; strides must
 *     be multiples of 8 elements and both pointers 16-byte aligned.
 *   cache_seqlens counts the tokens already cached: token t of sequence b is
 *     written at cache position cache_seqlens[b] + t (through block_table when
 *     given), in place in k_cache / v_cache, and the Sq queries then attend to
 *     cache_seqlens[b] + S_new tokens, bottom-right aligned.  cache_seqlens
 *     itself is not modified; advancing it is the caller's step.
 *   The caller guarantees cache_seqlens[b] + S_new fits the cache (Smax, or the
 *     pages of block_table row b); a new token whose position falls outside the
 *     cache is not written.
 *   Sq = 0 only appends.  All other arguments, limits and errors are those of
 *   fa_fwd_kvcache, which is this call with S_new = 0.  Arguments are checked
 *   before anything is launched.
 */
fa_status fa_fwd_kvcache_append(fa_dtype dtype, const void* q, void* k_cache, void* v_cache,
                                const int* cache_seqlens, const int* block_table, int block_table_stride,
                                int page_size, int num_blocks_or_smax, int num_splits,
                                const void* k_new, const void* v_new, int S_new,
                                const int64_t* kn_stride, const int64_t* vn_stride,
                                void* workspace, size_t workspace_bytes, void* out, float* lse,
                                int B, int Sq, int Hq, int Hkv, int D, const fa_attn_opts* opts, void* stream);

/*
 * fa_fwd_kvcache without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The decode partials live in a static device array of
 * fa_kvcache_noalloc_max_bytes() bytes (32 MiB) that the library holds on every
 * GPU it runs on until the process ends; the call allocates nothing and calls
 * no allocating routine.  A call whose workspace (fa_kvcache_workspace_size for
 * the resolved split count) exceeds that size returns FA_ERR_UNSUPPORTED with
 * nothing launched.  All calls on one GPU share its array: calls that overlap
 * in time on one GPU (other streams, other threads) race and give undefined
 * results.  Nothing in the array needs clearing between calls: every partial
 * the combine reads is written first by the same call.  Arguments, results and
 * errors are otherwise those of fa_fwd_kvcache; the outputs equal its outputs
 * bit for bit.
 */
size_t fa_kvcache_noalloc_max_bytes(void);
fa_status fa_fwd_kvcache_noalloc(fa_dtype dtype, const void* q, const void* k_cache, const void* v_cache,
                                 const int* cache_seqlens, const int* block_table, int block_table_stride,
                                 int page_size, int num_blocks_or_smax, int num_splits, void* out, float* lse,
                                 int B, int Sq, int Hq, int Hkv, int D, const fa_attn_opts* opts, void* stream);

/*
 * Merge split partial results by their log-sum-exp ("FlashAttention 常用接口简单介绍",
 * §3.4 flash_attn_combine).  out_partial [B, S, H, D, num_splits] and
 * lse_partial [B, S, H, num_splits] float32; op_stride (5 entries: b, s, h, d,
 * split) and lp_stride (4 entries: b, s, h, split) give element strides, NULL =
 * contiguous in that order.  out [B, S, H, D] of out_dtype (o_stride: b, s, h;
 * NULL = contiguous); lse [B, S, H] float32 contiguous, may be NULL.
 * 1 <= num_splits <= 64.  out = Σ_s exp(lse_s - lse) out_s, lse = log Σ_s exp(lse_s).
 */
fa_status fa_combine(const float* out_partial, const float* lse_partial, int B, int S, int H, int D,
                     int num_splits, const int64_t* op_stride, const int64_t* lp_stride,
                     fa_dtype out_dtype, void* out, const int64_t* o_stride, float* lse, void* stream);

/* Bytes of workspace fa_bwd needs: the float32 row sums delta [B, Hq, Sq]
 * (delta_i = dout_i · out_i), padded to 256 bytes; 0 when B, Sq or Hq is 0. */
size_t fa_bwd_workspace_size(int B, int Sq, int Hq);

/*
 * Backward of fa_fwd: gradients of a loss with respect to q, k and v given its
 * gradient dout with respect to out.  The attention weights are recomputed from
 * q, k and the forward's lse rather than stored (xhh.club "flash attention" tag
 * page, the summaries on recomputation in the backward pass); every output
 * element is written by one workgroup in a fixed order, so repeated calls give
 * identical bits (the deterministic backward of the update notes, v2.4, and
 * "FlashAttention 常用接口简单介绍", §5.3).
 *   dout, q, out [B, Sq, Hq, D] and k, v [B, Sk, Hkv, D] (dtype) with element
 *   strides as in fa_fwd (do_stride for dout; NULL = contiguous); lse
 *   [B, Hq, Sq] float32 as written by fa_fwd for the same inputs and options.
 *   dq [B, Sq, Hq, D], dk and dv [B, Sk, Hkv, D] (dtype), contiguous, are
 *   overwritten; GQA kv heads receive the sum over their query heads.  Keys no
 *   query may attend get dk = dv = 0, rows with no allowed key get dq = 0.
 *   opts must be those of the forward call.  D is 32, 64, 96, 128 or 256.
 *   workspace: device memory of at least fa_bwd_workspace_size(B, Sq, Hq)
 *   bytes, 16-byte aligned, owned by the caller (NULL allowed when that is 0);
 *   FA_ERR_WORKSPACE_TOO_SMALL otherwise.  Arithmetic: products in fp32 from
 *   the fp16/bf16 inputs; P and dS are rounded to the input dtype before the
 *   products that accumulate dv, dk and dq in fp32.
 */
fa_status fa_bwd(fa_dtype dtype, const void* dout, const void* q, const void* k, const void* v, const void* out,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                 const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                 const int64_t* o_stride, const int64_t* do_stride, const fa_attn_opts* opts,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of fa_fwd_varlen (packed sequences, "FlashAttention 常用接口简单介绍",
 * §3.2), with the conventions of fa_bwd.
 *   dout, q, out [total_q, Hq, D]; k, v [total_k, Hkv, D]; lse [Hq, total_q]
 *   float32 as written by fa_fwd_varlen; dq [total_q, Hq, D], dk and dv
 *   [total_k, Hkv, D] contiguous.  cu_seqlens_q/k, B and max_seqlen_q/k as for
 *   fa_fwd_varlen; *_stride: (token, head) element strides, NULL = contiguous.
 *   workspace: at least fa_bwd_workspace_size(1, total_q, Hq) bytes.
 *   Each sequence's gradients equal those of fa_bwd on that sequence alone,
 *   bit for bit.
 */
fa_status fa_bwd_varlen(fa_dtype dtype, const void* dout, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, void* dq, void* dk, void* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                        int max_seqlen_k, int total_q, int total_k, int Hq, int Hkv, int D,
                        const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                        const int64_t* o_stride, const int64_t* do_stride, const fa_attn_opts* opts,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* fa_status_string(fa_status status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
