// Split-KV decode for gfx950: new queries against a (paged) KV cache.
//
// Flash-decoding, as the Flash-Attention v2.0-v2.7 update notes describe it
// (v2.2): the cache of each sequence is cut along its length into num_splits
// contiguous chunks of ceil(len / num_splits) tokens; each (sequence, kv head,
// split) item yields a partial softmax average with its log-sum-exp, and a
// separate kernel merges the items of a row by their log-sum-exp (combine.hip).
// The cache may be paged (v2.5): token t of sequence b lives in page
// block_table[b, t / page_size], row t % page_size.
//
// Decode reads every K/V byte once at about 4 FLOP per byte, so it is bound by
// HBM bandwidth.  Design:
//  * persistent workgroups of one wave, as many as fit on the GPU, walk a static
//    schedule: sequences sorted by decreasing split length (ranked in each
//    workgroup for batches of up to 64, else by decode_order_kernel),
//    item k = (sequence rank, split, kv head) with the kv head fastest, and round
//    r of the schedule hands items r*P .. r*P+P-1 to the P workgroups forward for
//    even r and backward for odd r.  Longest items first in this snake order
//    balances ragged lengths to about 1%;
//  * the items of a workgroup form one stream of 64-token chunks.  A chunk's K
//    and V rows are read as whole rows (16 lanes per 256-byte row, full cache
//    lines) into registers and then stored to LDS; the next chunk's loads are
//    issued as one batch before the current chunk is computed, across item
//    boundaries, so starting an item (its page numbers, its queries) costs no
//    exposed memory latency;
//  * the page numbers of a chunk are requested one step earlier again, before
//    the K/V loads of the chunk in between: vector-memory results return in
//    order, so waiting for the page numbers never waits for K/V data in flight;
//  * an item's token range is clamped to the union of its rows' sliding windows,
//    so keys no row can see are never read;
//  * at D = 128 on a paged cache under 4 GiB (the KD form), K goes from HBM
//    straight into MFMA operand registers and only V is staged in LDS, in two
//    tiles, so K of two chunks can be in flight while one is computed.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

#ifndef FA_DECODE_CHUNK
#define FA_DECODE_CHUNK 64
#endif
#ifndef FA_DECODE_WPE
#define FA_DECODE_WPE 1
#endif
constexpr int kDecodeChunk = FA_DECODE_CHUNK;    // tokens per pipeline step
// D = 256 halves the chunk: a 64-token chunk of K and V would need 256 registers per lane
template <int D> constexpr int decode_chunk() { return D >= 256 ? kDecodeChunk / 2 : kDecodeChunk; }
constexpr float kTauD = 8.f;        // lazy-rescale threshold (log2 units)
constexpr int kOrderMaxB = 2048;    // larger batches are scheduled in their given order

// order[i] = (b, len_b) of the sequence with the i-th largest split length
// ceil(len_b / num_splits), ties by b.  One workgroup; rank by counting.
// Lengths are lens[b] + add.
__global__ __launch_bounds__(1024) void decode_order_kernel(const int* __restrict__ lens, int add, int B, int ns,
                                                           int2* __restrict__ order) {
  __shared__ int s_key[kOrderMaxB];
  const int tid = threadIdx.x;
  if (B > kOrderMaxB) {
    for (int b = tid; b < B; b += blockDim.x) order[b] = make_int2(b, lens[b] + add);
    return;
  }
  for (int b = tid; b < B; b += blockDim.x) {
    const int l = lens[b] + add;
    s_key[b] = l > 0 ? (l - 1) / ns + 1 : 0;
  }
  __syncthreads();
  for (int b = tid; b < B; b += blockDim.x) {
    const int key = s_key[b];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int kj = s_key[j];
      rank += (kj > key) | ((kj == key) & (j < b));
    }
    order[rank] = make_int2(b, lens[b] + add);
  }
}

// One pipeline slot: a chunk of one work item.  Every field is wave-uniform.
struct DecodeChunk {
  int ok;                   // 0: past the end of the workgroup's schedule
  int b, len, hk, split;    // the item
  int te;                   // end of the item's token range (exclusive)
  int base;                 // first token of the chunk
  int first, last;          // first / last chunk of the item
};

// ---------------------------------------------------------------------------
// One wave per workgroup.  The query rows of the GQA group (G heads x Sq
// positions, at most 16) sit on the N side of v_mfma_f32_16x16x32, so both
// contractions run on the matrix cores:
//   S^T = K Q^T : the A operand (lane = token % 16, 8 consecutive d) is read
//                 from the K tile in LDS, Q^T is a register-resident B operand;
//   O^T += V^T P^T : P stays in registers as the B operand (its contraction
//                 index is a fixed permutation of the chunk's tokens, applied
//                 identically to V), V^T comes from LDS through the
//                 transposing read ds_read_b64_tr_b16.
// Lane l holds query row l % 16; the four lanes sharing a row exchange their
// chunk maxima with two shuffles, so P of a chunk shares one reference max.
// MODE: 0 = dense cache, 1 = paged with pages of >= 64 tokens (a chunk spans at
// most two pages), 2 = paged with smaller pages.  OFF32: the cache holds fewer
// than 2^32 bytes, so byte offsets into it fit in 32 bits.
// ---------------------------------------------------------------------------
template <class E, int D, int MODE, bool OFF32, bool KD>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(FA_DECODE_WPE))) void decode_kernel(DecodeParams p) {
  using T = typename E::T;
  using V8 = typename E::V8;
  using V2 = typename E::V2;
  constexpr int C = decode_chunk<D>();
  constexpr int KSTEP = D / 32;           // MFMA K-steps of Q K^T
  constexpr int DBK = D / 16;             // 16-wide d blocks of O^T
  constexpr int VROW = D + 16;            // V LDS row stride (elements): conflict-free transposing reads
  constexpr int KROW = D + 8;             // K LDS row stride: conflict-free 16-byte reads
  constexpr int CH = D / 8;               // 16-byte pieces per K/V row
  // lanes per row: CH rounded up to a power of two (D = 96: 16 lanes for 12
  // pieces; the other 4 reread piece 0 and store nothing)
  constexpr int CHP = CH <= 4 ? 4 : CH <= 8 ? 8 : CH <= 16 ? 16 : 32;
  constexpr int NL = C * CHP / 64;        // K (and V) pieces a lane loads per chunk, one per row
  constexpr int RPI = 64 / CHP;           // rows covered by one 16-byte load of all 64 lanes
  constexpr int NE = MODE == 2 ? NL : 1;  // page numbers a lane holds per chunk
  static_assert(NL * 64 == C * CHP, "");
  constexpr int NG = C / 16;              // 16-token groups per chunk (MFMA M blocks of S^T)
  // KD: K goes from HBM straight into MFMA operand registers and only V is
  // staged in LDS, in two tiles (see the KD pipeline at the end)
  __shared__ __attribute__((aligned(16))) T vbuf[(KD ? 2 : 1) * C * VROW];
  __shared__ __attribute__((aligned(16))) T kbuf[KD ? 8 : C * KROW];

  const int lane = threadIdx.x, n = lane & 15, q4 = lane >> 4;
  lds_poison(vbuf, sizeof(vbuf), lane, 64);
  lds_poison(kbuf, sizeof(kbuf), lane, 64);
  const int lpc = lane % CHP;             // this lane's piece of its row
  const bool piece_ok = CH == CHP || lpc < CH;
  const int lcol = piece_ok ? lpc : 0;    // the piece it loads
  const int P = gridDim.x, w = blockIdx.x;
  const int per_seq = p.num_splits * p.Hkv;
  const int n_items = p.B * per_seq;
  const int rows = p.group * p.Sq;
  const int sqi = n / p.group, gq = n - sqi * p.group;   // row n: position sqi, head hk*G + gq
  const bool live = n < rows;
  // several cache heads per work head: row n's query head belongs to cache head
  // hrow of the work head, whose elements are D-row elements hrow*head_dim ..
  const int heads_per_item = p.head_shift < 30 ? D >> p.head_shift : 1;
  const int hrow = gq / (p.group / heads_per_item);
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_in = p.softcap > 0.f ? 2.f * p.scale * kLog2e / p.softcap : 0.f;
  const int64_t row_elems = (int64_t)p.kv_heads * D;
  const int page = p.page_size;
  auto div_page = [&](int t) __attribute__((always_inline)) { return p.log2_page >= 0 ? t >> p.log2_page : t / page; };
  auto prow_of = [&](const DecodeChunk& d) __attribute__((always_inline)) {
    return (((int64_t)d.b * p.Sq + sqi) * p.Hq + d.hk * p.group + gq) * p.num_splits + d.split;
  };

  // ---- static schedule: round r gives item item_of(r); s_wnd[j] holds the
  // (sequence, length) pair of round rb + j.  (Kept in LDS: a register that a
  // rarely taken reload may still be loading would make every use wait for all
  // loads in flight.)
  __shared__ int2 s_wnd[64];
  __shared__ int2 s_ord[64];
  if (!p.order) {
    // B <= 64: rank the sequences here, lane b holding sequence b (lanes past B
    // get key -1 and so ranks B .. 63)
    const int lb = lane < p.B ? p.cache_seqlens[lane] + p.seqlen_add : 0;
    const int key = lane < p.B ? (lb > 0 ? (lb - 1) / p.num_splits + 1 : 0) : -1;
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const int kj = __builtin_amdgcn_readlane(key, j);
      rank += (kj > key) | ((kj == key) & (j < lane));
    }
    s_ord[rank] = make_int2(lane, lb);
  }
  // A kv head's row that does not fill whole 128-byte lines (D = 32: 64 bytes,
  // D = 96: 192) shares lines with the neighbouring heads of the same token.
  // Workgroup w runs on XCD w mod 8, so there the slots of a round are dealt so
  // that each XCD's workgroups take 8 consecutive slots (the heads of one
  // sequence and split) and the shared lines are fetched into one L2.  The
  // snake pairing is kept: a workgroup takes slot ws in even rounds and
  // P - 1 - ws in odd ones.
  constexpr bool kGroupHeads = (D * sizeof(T)) % 128 != 0;
  const int ws = !kGroupHeads || w >= (P & ~63) ? w : (w & ~63) + 8 * (w & 7) + ((w >> 3) & 7);
  auto item_of = [&](int r) __attribute__((always_inline)) { return r * P + ((r & 1) ? P - 1 - ws : ws); };
  int rb = 0, lr = -1;
  auto load_window = [&]() __attribute__((always_inline)) {
    const int k = item_of(rb + lane);
    const int i = k < n_items ? k / per_seq : 0;
    const int2 bl = p.order ? p.order[i] : s_ord[i];
    s_wnd[lane] = k < n_items ? bl : make_int2(0, 0);
  };
  load_window();

  // d := the first chunk of the next non-empty item; empty items get lse = -inf
  auto next_item = [&](DecodeChunk& d) __attribute__((always_inline)) {
    for (;;) {
      ++lr;
      const int k = item_of(lr);
      if (k >= n_items) {
        d.ok = 0;
        return;
      }
      if (lr - rb >= 64) {
        rb = lr;
        load_window();
      }
      const int2 bl = s_wnd[lr - rb];
      const int b = __builtin_amdgcn_readfirstlane(bl.x);
      const int len = __builtin_amdgcn_readfirstlane(bl.y);
      const int rem = k % per_seq;
      const int split = rem / p.Hkv, hk = rem - split * p.Hkv;
      const int chunk = len > 0 ? (len - 1) / p.num_splits + 1 : 0;
      int t0 = min(len, split * chunk);
      const int t1 = min(len, t0 + chunk);
      if (p.wl >= 0) t0 = max(t0, len - p.Sq - p.wl);   // below every row's window
      d.ok = 1;
      d.b = b; d.len = len; d.hk = hk; d.split = split;
      d.te = t1; d.base = t0;
      d.first = 1; d.last = t0 + C >= t1;
      if (t0 < t1) return;
      if (live && q4 == 0) p.lse_partial[prow_of(d)] = kNegInf;   // weight 0 in the combine
    }
  };
  auto advance = [&](DecodeChunk& d) __attribute__((always_inline)) {
    if (!d.ok) return;
    if (d.base + C < d.te) {
      d.base += C;
      d.first = 0;
      d.last = d.base + C >= d.te;
    } else {
      next_item(d);
    }
  };

  // Every load of the chunk stream is issued on every path (a chunk past the end
  // of the schedule reads row 0 and page-table entry 0, and the values are never
  // used), and loaded values are left untouched until they are consumed: the
  // compiler can then wait for exactly the loads a use needs, instead of for all
  // loads in flight.

  // page numbers of chunk d.  MODE 1: even lanes fetch the page of the chunk's
  // first token, odd lanes the next page when the chunk reaches it.  MODE 2: the
  // page of each row the lane loads.
  auto request = [&](const DecodeChunk& d, int (&e)[NE]) __attribute__((always_inline)) {
    if constexpr (MODE != 0) {
      const int* bt = p.block_table + (d.ok ? (int64_t)d.b * p.bt_stride : 0);
      if constexpr (MODE == 1) {
        const int pg0 = div_page(d.base);
        const bool second = (lane & 1) && (pg0 + 1) * page < d.te;
        e[0] = bt[d.ok ? pg0 + (second ? 1 : 0) : 0];
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int r = RPI * i + lane / CHP;
          e[i] = bt[d.ok ? div_page(min(d.base + r, d.te - 1)) : 0];
        }
      }
    }
  };
  // LDS tile: row RPI*i + lane/CHP, 16-byte piece lane%CHP, from one base
  // address per lane and constant offsets
  T* const kst = kbuf + (lane / CHP) * KROW + lcol * 8;
  T* const vst = vbuf + (lane / CHP) * VROW + lcol * 8;
  auto put = [&](int i, const u32x4 (&kr)[NL], const u32x4 (&vr)[NL]) __attribute__((always_inline)) {
    if (piece_ok) {
      *(u32x4*)(kst + i * RPI * KROW) = kr[i];
      *(u32x4*)(vst + i * RPI * VROW) = vr[i];
    }
  };

  // Load chunk d: its K and V rows (rows past the item's end repeat its last
  // row), the item's query rows (rows past the group read row 0) and ALiBi
  // slopes (a stand-in address without slopes); qs and sls are raw loaded
  // values.  With Swap, the chunk the registers hold is stored to the LDS tile
  // piece by piece, each register reloaded right after its store, so the new
  // chunk's loads leave as soon as the old one starts to arrive.
  // Rows of chunk d's tokens in the cache (MODE 0 and 1): token t lives in row
  // t + d0 below bnd and t + d0 + dd from bnd on (MODE 1: the chunk's first page
  // and, past it, the next one, from the page numbers in lanes 0 and 1 of e).
  auto page_rows = [&](const DecodeChunk& d, const int (&e)[NE], int& d0, int& dd, int& bnd)
      __attribute__((always_inline)) {
    if constexpr (MODE == 0) {
      d0 = (d.ok ? d.b : 0) * page; dd = 0; bnd = 0x7fffffff;
    } else if constexpr (MODE == 1) {
      const int pg0 = div_page(d.base);
      const int e0 = __builtin_amdgcn_readlane(e[0], 0), e1 = __builtin_amdgcn_readlane(e[0], 1);
      bnd = (pg0 + 1) * page; d0 = (e0 - pg0) * page; dd = (e1 - e0 - 1) * page;
    } else {
      d0 = 0; dd = 0; bnd = 0x7fffffff;
    }
  };
  // The item's query rows (rows past the group read row 0) and ALiBi slopes (a
  // stand-in address without slopes), as raw loaded values.
  auto issue_q = [&](const DecodeChunk& d, u32x4 (&qs)[KSTEP], float& sls) __attribute__((always_inline)) {
    const int b = d.ok ? d.b : 0, hk = d.ok ? d.hk : 0;
    const int hq = hk * p.group + (live ? gq : 0);
    // q holds at most 2^31 bytes (checked on the host): a 32-bit byte offset per
    // lane from a wave-uniform base, the piece's place within its head uniform per ks
    const uint32_t qoff = (uint32_t)(((b * p.Sq + (live ? sqi : 0)) * p.Hq + hq) * p.head_dim + q4 * 8) *
                          (uint32_t)sizeof(T);
    const int qmask = (1 << p.head_shift) - 1;   // element within its head (all ones: one head)
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks)
      qs[ks] = *(const u32x4*)((const char*)p.q + ((ks * 32) & qmask) * (int)sizeof(T) + qoff);
    sls = *(p.alibi ? p.alibi + hq : p.lse_partial);
  };
  auto issue = [&](const DecodeChunk& d, const int (&e)[NE], u32x4 (&kr)[NL], u32x4 (&vr)[NL],
                   u32x4 (&qs)[KSTEP], float& sls, auto Swap) __attribute__((always_inline)) {
    constexpr bool swap = decltype(Swap)::value;
    const int b = d.ok ? d.b : 0, hk = d.ok ? d.hk : 0;
    const int hc = hk / p.kv_split;                      // the cache head this work head reads
    const T* kh = (const T*)p.k + (int64_t)hc * D;
    const T* vh = (const T*)p.v + (int64_t)hc * D;
    int pg0 = 0, e0 = 0, e1 = 0;
    if constexpr (MODE == 1) {
      pg0 = div_page(d.base);
      e0 = __builtin_amdgcn_readlane(e[0], 0);
      e1 = __builtin_amdgcn_readlane(e[0], 1);
    }
    if constexpr (OFF32) {
      // cache smaller than 4 GiB: a wave-uniform base plus a 32-bit byte offset
      // per lane, shared by K and V.  Lane rows are t_i = base + RPI*i + lr; a
      // row's offset steps by RPI rows per load, plus the page jump past bnd;
      // rows past the item's end reread its last row.
      const char* kb8 = (const char*)p.k;
      const char* vb8 = (const char*)p.v;
      const uint32_t rowb = (uint32_t)(row_elems * sizeof(T));
      const int lr = lane / CHP, c = lcol;
      const uint32_t lane_off = (uint32_t)hc * (uint32_t)(D * sizeof(T)) + (uint32_t)c * 16u;
      const int tl = d.te - 1;
      if constexpr (MODE == 2) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int t = min(d.base + RPI * i + lr, tl);
          int row = e[i] * page + (t - div_page(t) * page);
          if (!d.ok) row = 0;
          const uint32_t off = (uint32_t)row * rowb + lane_off;
          if constexpr (swap) put(i, kr, vr);
          kr[i] = *(const u32x4*)(kb8 + off);
          vr[i] = *(const u32x4*)(vb8 + off);
        }
      } else {
        int d0, dd, bnd;                      // row(t) = t + d0 below bnd, t + d0 + dd from bnd on
        page_rows(d, e, d0, dd, bnd);
        const int tlast = (tl < bnd ? tl + d0 : tl + d0 + dd);
        const uint32_t off_last = d.ok ? (uint32_t)tlast * rowb + lane_off : lane_off;
        const int t0 = d.base + lr;
        const uint32_t off0 = d.ok ? (uint32_t)(t0 + d0) * rowb + lane_off : lane_off;
        const uint32_t jump = (uint32_t)dd * rowb, stepb = (uint32_t)RPI * rowb;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int t = t0 + RPI * i;
          uint32_t off = off0 + (uint32_t)i * stepb + (t >= bnd ? jump : 0u);
          if (t > tl || !d.ok) off = d.ok ? off_last : lane_off;
          if constexpr (swap) put(i, kr, vr);
          kr[i] = *(const u32x4*)(kb8 + off);
          vr[i] = *(const u32x4*)(vb8 + off);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int r = RPI * i + lane / CHP, c = lcol;
        const int t = min(d.base + r, d.te - 1);
        int64_t row;
        if constexpr (MODE == 0) {
          row = (int64_t)b * page + t;
        } else if constexpr (MODE == 1) {
          const int off = t - pg0 * page;
          row = off < page ? (int64_t)e0 * page + off : (int64_t)e1 * page + (off - page);
        } else {
          row = (int64_t)e[i] * page + (t - div_page(t) * page);
        }
        if (!d.ok) row = 0;
        if constexpr (swap) put(i, kr, vr);
        kr[i] = *(const u32x4*)(kh + row * row_elems + c * 8);
        vr[i] = *(const u32x4*)(vh + row * row_elems + c * 8);
      }
    }
    issue_q(d, qs, sls);
  };
  // ---- per-item row state.  Row n sees tokens [rlo, rhi] of the item; every
  // live row sees [wlo, whi], so chunks inside it need no masking.
  V8 qb[KSTEP];
  f32x4 o[DBK];
  float m = kNegInf, lx = 0.f, slope = 0.f, ipf = 0.f;
  int rlo = 0, rhi = -1, wlo = 0, whi = -1;

  auto begin_item = [&](const DecodeChunk& d, const u32x4 (&qs)[KSTEP], float sls) __attribute__((always_inline)) {
    // the row's query sits in its own cache head's elements, zeros elsewhere, so
    // the scores take only that head's keys
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks)
      qb[ks] = __builtin_bit_cast(V8, live && ((ks * 32 + q4 * 8) >> p.head_shift) == hrow ? qs[ks] : u32x4{});
    slope = (p.alibi && live) ? sls * kLog2e : 0.f;
    const int ip = sqi + d.len - p.Sq;     // bottom-right aligned position of the row
    ipf = (float)ip;
    rlo = p.wl >= 0 ? max(0, ip - p.wl) : 0;
    rhi = d.te - 1;
    if (p.causal) rhi = min(rhi, ip);
    if (p.wr >= 0) rhi = min(rhi, ip + p.wr);
    if (!live) rhi = -1;
    // rows 0 and Sq-1 bound the others (positions grow with the row)
    const int ip0 = d.len - p.Sq, ipl = d.len - 1;
    wlo = p.wl >= 0 ? max(0, ipl - p.wl) : 0;
    whi = d.te - 1;
    if (p.causal) whi = min(whi, ip0);
    if (p.wr >= 0) whi = min(whi, ip0 + p.wr);
    m = kNegInf;
    lx = 0.f;
#pragma unroll
    for (int db = 0; db < DBK; ++db) o[db] = f32x4{};
  };

  // kk: with KD, the chunk's K operands in registers (K[token 16g + n][d = 32ks +
  // 8q4 ..] in kk[g * KSTEP + ks]); vt: the LDS tile holding the chunk's V rows
  // after_scores runs once S^T has been formed (the KD pipeline loads the next
  // K operands into kk there)
  auto compute = [&](const DecodeChunk& d, const u32x4* kk, const T* vt, auto&& after_scores)
      __attribute__((always_inline)) {
    const int base = d.base;
    // S^T = K Q^T; A operand: lane holds K[token 16g + n][d = 32ks + 8q4 .. +7]
    f32x4 s[NG];
    const T* kb_ = kbuf + n * KROW + q4 * 8;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      s[g] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks) {
        if constexpr (KD) s[g] = E::mfma16(__builtin_bit_cast(V8, kk[g * KSTEP + ks]), qb[ks], s[g]);
        else s[g] = E::mfma16(*(const V8*)(kb_ + 16 * g * KROW + ks * 32), qb[ks], s[g]);
      }
    }
    after_scores();
    // scores of tokens base + 16g + 4q4 + r for row n; times mult they are in
    // log2 units (plain scores keep the scale folded into the exp argument)
    const bool plain = !(p.softcap > 0.f) && !p.alibi;
    const float mult = plain ? sl2 : 1.f;
    if (p.softcap > 0.f) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2_fast(s[g][r] * cap_in);
          s[g][r] = fmaf(-2.f * cap_l2, __builtin_amdgcn_rcpf(e + 1.f), cap_l2);
        }
    } else if (p.alibi) {
#pragma unroll
      for (int g = 0; g < NG; ++g) s[g] *= sl2;
    }
    if (p.alibi) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[g][r] = fmaf(-slope, fabsf(ipf - (float)(base + 16 * g + 4 * q4 + r)), s[g][r]);
    }
    if (!(base >= wlo && base + C - 1 <= whi)) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = base + 16 * g + 4 * q4 + r;
          if (t < rlo || t > rhi) s[g][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int g = 0; g < NG; ++g) mx = fmaxf(mx, fmaxf(fmaxf(s[g][0], s[g][1]), fmaxf(s[g][2], s[g][3])));
    mx = max_halves(max_xor16(mx)) * mult;           // the row's four lanes: l, l^16, l^32, l^48
    const float m_new = fmaxf(m, mx);
    if (__any(m_new > m + kTauD)) {
      const float alpha = m_new == kNegInf ? 1.f : exp2_fast(m - m_new);
      m = m_new;
      lx *= alpha;
#pragma unroll
      for (int db = 0; db < DBK; ++db) o[db] *= alpha;
    }
    const float m_use = m == kNegInf ? 0.f : m;
    // O^T += V^T P^T per 32 tokens: B operand element 4g' + r of lane (n, q4) is
    // P of token 32h + 16g' + 4q4 + r
    // P goes in two rounded parts, hi = RN(P) and lo = RN(P - hi), each through
    // its own product, so O carries P to about 2^-22 relative instead of the
    // half ulp of the input type that rounding P alone would leave.  The extra
    // products ride on matrix cores that the memory stream leaves idle.
#pragma unroll
    for (int hh = 0; hh < NG / 2; ++hh) {
      V8 bop, blo;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = exp2_fast(fmaf(s[2 * hh + g][r], mult, -m_use));
          const float p1 = exp2_fast(fmaf(s[2 * hh + g][r + 1], mult, -m_use));
          const V2 pp = E::pack(p0, p1);
          bop[4 * g + r] = pp[0];
          bop[4 * g + r + 1] = pp[1];
          const V2 pl = E::pack(p0 - E::to_f32(pp[0]), p1 - E::to_f32(pp[1]));
          blo[4 * g + r] = pl[0];
          blo[4 * g + r + 1] = pl[1];
          lx += p0 + p1;
        }
      // V^T operand rows: 32h + 16g' + 4q4 + (n / 4), columns 16db + 4(n % 4)
      const T* vrow = vt + (32 * hh + 4 * q4 + (n >> 2)) * VROW + 4 * (n & 3);
#pragma unroll
      for (int db = 0; db < DBK; ++db) {
        const i16x4 x0 = lds_read_tr16(vrow + db * 16);
        const i16x4 x1 = lds_read_tr16(vrow + 16 * VROW + db * 16);
        const V8 a = __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = E::mfma16(a, bop, o[db]);
        o[db] = E::mfma16(a, blo, o[db]);
      }
    }
    if (d.last) {
      // the four lanes of a row hold partial sums over their own tokens
      const float lxt = sum_halves(sum_xor16(lx));
      if (live) {
        const int64_t prow = prow_of(d);
        const float inv = lxt > 0.f ? 1.f / lxt : 0.f;
        // only the row's own cache head's elements of O are its output
        float* dst = p.out_partial + prow * p.head_dim + 4 * q4;
#pragma unroll
        for (int db = 0; db < DBK; ++db)
          if (((db * 16) >> p.head_shift) == hrow) *(f32x4*)(dst + db * 16 - hrow * p.head_dim) = o[db] * inv;
        if (q4 == 0) p.lse_partial[prow] = lxt > 0.f ? (m + __log2f(lxt)) * kLn2 : kNegInf;
      }
    }
  };

  // ---- KD pipeline (D = 128, pages of >= 64 tokens, cache under 4 GiB).  K of
  // a chunk is loaded straight into the A operands of S^T = K Q^T (16 loads of
  // 16 tokens x 64 contiguous bytes: the same d order as Q, so the same
  // products), so only V passes through LDS, in two tiles.  Two register sets
  // hold K of two chunks, so while chunk c is computed, K of c+1 and c+2 and V
  // of c+1 are in flight (48 KB per wave against the 32 KB of one chunk).
  // Step c (s = c % 2):
  //   a. begin the item of c;  b. request the pages of c+3;  c. load q of c+1;
  //   d. S^T of c from kreg[s];  e. load K of c+2 into kreg[s];
  //   f. softmax and P V of c from tile s;
  //   g. store V of c+1 to tile s^1, loading V of c+2 into the freed registers.
  // V of c+1 is stored only after c is computed: waiting for it earlier would
  // also wait for K of c+1 (loads complete in order) and empty the queue.
  auto kd_pipeline = [&]() __attribute__((always_inline)) {
    if constexpr (KD) {
      static_assert(MODE == 1 && OFF32 && NL * RPI == C, "KD: paged cache under 4 GiB");
      constexpr int NK = NG * KSTEP;
      const char* kb8 = (const char*)p.k;
      const char* vb8 = (const char*)p.v;
      const uint32_t rowb = (uint32_t)(row_elems * sizeof(T));
      auto issue_k = [&](const DecodeChunk& d, const int (&e)[NE], u32x4 (&kk)[NK]) __attribute__((always_inline)) {
        const int hc = (d.ok ? d.hk : 0) / p.kv_split;
        const uint32_t lane_off = (uint32_t)hc * (uint32_t)(D * sizeof(T)) + (uint32_t)q4 * 16u;
        int d0, dd, bnd;
        page_rows(d, e, d0, dd, bnd);
        const int tl = d.te - 1;
        const uint32_t off_last = d.ok ? (uint32_t)(tl < bnd ? tl + d0 : tl + d0 + dd) * rowb + lane_off : lane_off;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int t = d.base + 16 * g + n;
          uint32_t off = (uint32_t)(t + d0) * rowb + lane_off + (t >= bnd ? (uint32_t)dd * rowb : 0u);
          if (t > tl || !d.ok) off = d.ok ? off_last : lane_off;
#pragma unroll
          for (int ks = 0; ks < KSTEP; ++ks) kk[g * KSTEP + ks] = *(const u32x4*)(kb8 + off + ks * 64);
        }
      };
      // V rows of chunk d; with Swap the registers' chunk is first stored to the
      // tile vdst piece by piece, each register reloaded right after its store
      auto issue_v = [&](const DecodeChunk& d, const int (&e)[NE], u32x4 (&vv)[NL], T* vdst, auto Swap)
          __attribute__((always_inline)) {
        constexpr bool swap = decltype(Swap)::value;
        const int hc = (d.ok ? d.hk : 0) / p.kv_split;
        const uint32_t lane_off = (uint32_t)hc * (uint32_t)(D * sizeof(T)) + (uint32_t)lcol * 16u;
        int d0, dd, bnd;
        page_rows(d, e, d0, dd, bnd);
        const int tl = d.te - 1;
        const uint32_t off_last = d.ok ? (uint32_t)(tl < bnd ? tl + d0 : tl + d0 + dd) * rowb + lane_off : lane_off;
        const int t0 = d.base + lane / CHP;
        const uint32_t off0 = d.ok ? (uint32_t)(t0 + d0) * rowb + lane_off : lane_off;
        const uint32_t jump = (uint32_t)dd * rowb, stepb = (uint32_t)RPI * rowb;
        T* const vs = vdst + (lane / CHP) * VROW + lcol * 8;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int t = t0 + RPI * i;
          uint32_t off = off0 + (uint32_t)i * stepb + (t >= bnd ? jump : 0u);
          if (t > tl || !d.ok) off = d.ok ? off_last : lane_off;
          if constexpr (swap) {
            if (piece_ok) *(u32x4*)(vs + i * RPI * VROW) = vv[i];
          }
          vv[i] = *(const u32x4*)(vb8 + off);
        }
      };
      DecodeChunk dc, d1, d2, d3;
      int ev[2][NE], e0v[NE];
      u32x4 kreg[2][NK];
      u32x4 vv[NL];
      u32x4 qs[KSTEP];
      float sl = 0.f;
      next_item(dc);
      request(dc, e0v);                                 // pages of c0
      d1 = dc;
      advance(d1);
      request(d1, ev[1]);                               // pages of c1
      issue_q(dc, qs, sl);
      issue_k(dc, e0v, kreg[0]);
      issue_v(dc, e0v, vv, vbuf, std::false_type{});
      d2 = d1;
      advance(d2);
      request(d2, ev[0]);                               // pages of c2
      issue_k(d1, ev[1], kreg[1]);
      issue_v(d1, ev[1], vv, vbuf, std::true_type{});   // V of c0 to tile 0, load V of c1
      auto step = [&](auto S) __attribute__((always_inline)) -> bool {
        constexpr int s0 = decltype(S)::value, s1 = s0 ^ 1;
        if (dc.first) begin_item(dc, qs, sl);
        d3 = d2;
        advance(d3);
        request(d3, ev[s1]);                            // pages of c+3
        issue_q(d1, qs, sl);                            // q of c+1
        compute(dc, kreg[s0], vbuf + s0 * C * VROW, [&] { issue_k(d2, ev[s0], kreg[s0]); });
        issue_v(d2, ev[s0], vv, vbuf + s1 * C * VROW, std::true_type{});
        dc = d1;
        d1 = d2;
        d2 = d3;
        return dc.ok;
      };
      if (dc.ok) {
        for (;;) {
          if (!step(std::integral_constant<int, 0>{})) break;
          if (!step(std::integral_constant<int, 1>{})) break;
        }
      }
    }
  };
  if constexpr (KD) {
    kd_pipeline();
    return;
  }
  // ---- pipeline.  Step j: request the pages of c_{j+2}; store chunk c_j to
  // the LDS tile while loading c_{j+1} into the registers it leaves; compute c_j
  // from LDS while c_{j+1} is in flight.  One chunk in flight per wave reads HBM
  // faster than a deeper trickle of loads.  Page numbers are requested before
  // the loads of the chunk ahead of them, so waiting for them only waits for
  // consumed chunks.  The LDS tile is reused at once: a wave's LDS accesses
  // complete in order.
  DecodeChunk dq[2], dc;      // chunks with pages requested (by j % 2) / the chunk in registers
  int ev[2][NE];
  u32x4 kr[NL], vr[NL];
  u32x4 qs[KSTEP];
  float sl = 0.f;

  next_item(dq[0]);
  request(dq[0], ev[0]);                              // c0
  dq[1] = dq[0];
  advance(dq[1]);
  request(dq[1], ev[1]);                              // c1
  issue(dq[0], ev[0], kr, vr, qs, sl, std::false_type{});
  dc = dq[0];
  // step j with s = j % 2: dq[s ^ 1] holds c_{j+1}
  auto step = [&](auto S) __attribute__((always_inline)) -> bool {
    constexpr int s0 = decltype(S)::value, s1 = s0 ^ 1;
    if (dc.first) begin_item(dc, qs, sl);
    dq[s0] = dq[s1];
    advance(dq[s0]);                                  // c_{j+2}
    request(dq[s0], ev[s0]);
    issue(dq[s1], ev[s1], kr, vr, qs, sl, std::true_type{});   // store c_j, load c_{j+1}
    compute(dc, kr, vbuf, [] {});
    dc = dq[s1];
    return dc.ok;
  };
  if (dc.ok) {
    for (;;) {
      if (!step(std::integral_constant<int, 0>{})) break;
      if (!step(std::integral_constant<int, 1>{})) break;
    }
  }
}

// 1: D = 128 on a paged cache under 4 GiB runs the KD form (K in operand
// registers, V in two LDS tiles); 0: the LDS form everywhere
#ifndef FA_DECODE_KD
#define FA_DECODE_KD 1
#endif
template <class E, int D, int MODE, bool OFF32, bool KD = FA_DECODE_KD && D == 128 && MODE == 1 && OFF32>
static hipError_t launch_dk(const DecodeParams& p, int cus, hipStream_t s) {
  // resident workgroups per CU (the same on every gfx950 device); computed once,
  // and a concurrent first call at worst computes the same value twice
  static std::atomic<int> cached{0};
  int per_cu = cached.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<E, D, MODE, OFF32, KD>, 64, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    per_cu = nb;
    cached.store(nb, std::memory_order_relaxed);
  }
  const int64_t items = (int64_t)p.B * p.num_splits * p.Hkv;
  const int grid = (int)std::min<int64_t>(items, (int64_t)cus * per_cu);
  hipLaunchKernelGGL((decode_kernel<E, D, MODE, OFF32, KD>), dim3(grid), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <class E, int D, int MODE>
static hipError_t launch_dm(const DecodeParams& p, int cus, hipStream_t s) {
  const int64_t bytes = p.cache_rows * p.kv_heads * D * (int64_t)sizeof(typename E::T);
  if (bytes <= ((int64_t)1 << 32)) return launch_dk<E, D, MODE, true>(p, cus, s);
  return launch_dk<E, D, MODE, false>(p, cus, s);
}

template <class E, int D>
static hipError_t launch_d(const DecodeParams& p, int cus, hipStream_t s) {
  if (!p.block_table) return launch_dm<E, D, 0>(p, cus, s);
  if (p.page_size >= decode_chunk<D>()) return launch_dm<E, D, 1>(p, cus, s);
  return launch_dm<E, D, 2>(p, cus, s);
}

hipError_t launch_decode(Dtype dt, int D, const DecodeParams& p, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (cus < 1) cus = 1;
  if (p.order) {
    hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(1024), 0, s, p.cache_seqlens, p.seqlen_add, p.B,
                       p.num_splits, p.order);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  switch (D) {
    case 32: return dt == kF16 ? launch_d<F16, 32>(p, cus, s) : launch_d<BF16, 32>(p, cus, s);
    case 64: return dt == kF16 ? launch_d<F16, 64>(p, cus, s) : launch_d<BF16, 64>(p, cus, s);
    case 96: return dt == kF16 ? launch_d<F16, 96>(p, cus, s) : launch_d<BF16, 96>(p, cus, s);
    case 256: return dt == kF16 ? launch_d<F16, 256>(p, cus, s) : launch_d<BF16, 256>(p, cus, s);
    default: return dt == kF16 ? launch_d<F16, 128>(p, cus, s) : launch_d<BF16, 128>(p, cus, s);
  }
}

}  // namespace fa
