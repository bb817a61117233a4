// Parameter blocks and launcher entry points shared by the C-ABI host layer
// (fa_api.cpp) and the kernel translation units.  Everything here is plain
// data: device pointers, sizes and element strides.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum Dtype { kF16 = 0, kBF16 = 1 };

// Prefill (dense or packed variable-length) forward.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  // element strides: batch, sequence, head (head_dim stride is 1)
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh;      // lse element (b, h, i) at b*lse_sb + h*lse_sh + row_base + i
  const int* cu_seqlens_q;     // varlen: [B+1] prefix sums (nullptr for dense)
  const int* cu_seqlens_k;
  int B, Sq, Sk;               // dense sizes; for varlen Sq/Sk hold max_seqlen_q/k
  int Hq, Hkv, group;          // group = Hq / Hkv
  float scale;                 // softmax scale (for fp8 inputs times the q and k descales)
  float out_scale;             // out = out_scale * sum_j p_j v_j / sum_j p_j (fp8: the v descale; else 1)
  float softcap;               // 0 = off
  const float* alibi;          // [Hq] slopes or nullptr
  int causal;
  int wl, wr;                  // window (left, right), -1 = unbounded
  int n_qtiles;                // ceil(Sq / block_m)
  int n_heads;                 // B * Hq: the grid is n_heads x n_qtiles (head, query tile) units
  int block_m;                 // query rows per workgroup (prefill_block_m)
  int remap_xcd;               // 1 when B*Hq is a multiple of 8: each XCD takes a contiguous eighth of the heads
  int order_group;             // heads per longest-first group (causal), 0 = head by head (see tile_order)
};

// Split-KV decode over a dense or paged cache: partial results per split.
struct DecodeParams {
  const void* q;               // [B, Sq, Hq, D]
  const void* k;               // dense [B, Smax, Hkv, D] or pool [P, page, Hkv, D]
  const void* v;
  const int* cache_seqlens;    // [B]
  int seqlen_add;              // tokens appended by this call: sequence b attends to cache_seqlens[b] + seqlen_add
  const int* block_table;      // [B, bt_stride] or nullptr (dense)
  int bt_stride;
  int page_size;               // paged: tokens per page; dense: Smax
  int64_t cache_rows;          // token rows in k (and v): pages * page_size, or B * Smax
  int log2_page;               // log2(page_size) when page_size is a power of two, else -1
  float* out_partial;          // [B, Sq, Hq, num_splits, D] fp32
  float* lse_partial;          // [B, Sq, Hq, num_splits] fp32
  int2* order;                 // [B] schedule order: (b, cache_seqlens[b]) by decreasing split length;
                               // nullptr: B <= 64, ranked inside the decode kernel
  int B, Sq, Hq, Hkv, group;  // Hkv: work heads, kv_heads * kv_split; group = Hq / Hkv query heads each
  int kv_heads;                // kv heads of the cache
  int kv_split;                // work heads per cache head: a cache head's query heads split into
                               // kv_split groups of at most 16 rows, each reading the same K/V
  int head_dim;                // head dim of q, the cache and the partials; the kernel's D is
                               // head_dim * (cache heads per work head): a work head may take
                               // 2, 4 or 8 adjacent cache heads as one row of D elements
  int head_shift;              // log2(head_dim) when a work head takes several cache heads, else 30
  int num_splits;
  float scale;
  float softcap;
  const float* alibi;
  int causal;
  int wl, wr;
};

// New keys/values [B, S, Hkv, D] written into a KV cache at positions
// cache_seqlens[b] + t (dense [B, smax, Hkv, D] or pool [num_blocks, page_size, Hkv, D]).
struct AppendParams {
  const void* k_new;
  const void* v_new;
  int64_t kn_sb, kn_ss, kn_sh;   // element strides of k_new (b, t, head)
  int64_t vn_sb, vn_ss, vn_sh;
  void* k_cache;
  void* v_cache;
  const int* cache_seqlens;
  const int* block_table;        // [B, bt_stride] or nullptr (dense)
  int bt_stride, page_size, num_blocks;
  int smax;                      // dense: rows per sequence
  int B, S, Hkv, D;
};

// LSE-weighted merge of split partials.
struct CombineParams {
  const float* out_partial;
  const float* lse_partial;
  int64_t op_sb, op_ss, op_sh, op_sd, op_sn;   // element strides of out_partial (b, s, h, d, split)
  int64_t lp_sb, lp_ss, lp_sh, lp_sn;          // element strides of lse_partial (b, s, h, split)
  void* out;
  int64_t o_sb, o_ss, o_sh;                    // out element strides (d stride 1)
  float* lse;                                  // optional
  int64_t l_sb, l_ss, l_sh;                    // lse element strides
  int B, S, H, D, num_splits;
};

// Backward (gradients of q, k, v) of the dense forward, weights recomputed from lse.
struct BackwardParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;            // [B, Hq, Sq] as written by the forward
  void* dq;
  void* dk;
  void* dv;
  float* delta;                // workspace: rowsum(dout * out), element (b, h, i) at b*dl_sb + h*dl_sh + row_base + i
  const int* cu_seqlens_q;     // varlen: [B+1] prefix sums (nullptr for dense)
  const int* cu_seqlens_k;
  // element strides: batch, sequence, head (head_dim stride is 1)
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  int64_t lse_sb, lse_sh;      // as for the forward: element (b, h, i) at b*lse_sb + h*lse_sh + row_base + i
  int64_t dl_sb, dl_sh;
  int B, Sq, Sk, Hq, Hkv, group;   // varlen: Sq/Sk hold max_seqlen_q/k
  float scale;
  float softcap;
  const float* alibi;
  int causal;
  int wl, wr;
  int n_ktiles;                // ceil(Sk / backward_block_n(D))
  int n_qtiles;                // ceil(Sq / backward_block_m(D))
  int remap_xcd;               // set per kernel by the launcher: its head count is a multiple of 8
  int order_group;             // set per kernel by the launcher (see tile_order)
};

hipError_t launch_prefill(Dtype dt, int D, const PrefillParams& p, hipStream_t s);
// fp8 e4m3 q/k/v, bf16 out; D in {64, 128}
hipError_t launch_prefill_fp8(int D, const PrefillParams& p, hipStream_t s);
int prefill_block_m_fp8(int D);
hipError_t launch_decode(Dtype dt, int D, const DecodeParams& p, hipStream_t s);
hipError_t launch_combine(Dtype dt, const CombineParams& p, hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
// D in {32, 64, 96, 128, 256}; launches nothing for an empty grid
hipError_t launch_backward(Dtype dt, int D, const BackwardParams& p, hipStream_t s);
int backward_block_n(int D);   // keys per dK/dV workgroup
int backward_block_m(int D);   // queries per dQ workgroup

// Prefill workgroup shape per head dim: NW waves, each owning RB blocks of 32 query rows.
#ifndef FA_PREFILL_NW64
#define FA_PREFILL_NW64 8
#endif
#ifndef FA_PREFILL_RB64
#define FA_PREFILL_RB64 1
#endif
#ifndef FA_PREFILL_NW128
#define FA_PREFILL_NW128 8
#endif
#ifndef FA_PREFILL_RB128
#define FA_PREFILL_RB128 1
#endif
// query rows per prefill workgroup for head dim D (the host sizes the grid with it)
// query rows per prefill workgroup for B*Hq = heads and the longest query
// sequence, on a device with cus compute units
// span: keys a row can see besides its own position (window sides, right side 0
// when causal), or -1 when unbounded
int prefill_block_m(int D, int64_t heads, int max_sq, int cus, int span);

// Heads per longest-first group for a grid of n_units heads x n_tiles tiles of
// unequal length: enough tiles per group to fill the about 64 workgroups an
// XCD holds at once; 0 (head by head) when the tiles are of equal length.
inline int order_group(bool unequal, int64_t n_units, int64_t n_tiles, bool xcd) {
#ifdef FA_ORDER_GROUP
  return unequal ? FA_ORDER_GROUP : 0;
#else
  if (!unequal || n_tiles <= 0) return 0;
  const int64_t nu = xcd ? n_units / 8 : n_units;
  int64_t g = (64 + n_tiles - 1) / n_tiles;
  if (g > nu) g = nu;
  return g < 1 ? 1 : (int)g;
#endif
}

}  // namespace fa
