// Backward kernels for gfx950: gradients of exact attention with respect to q,
// k and v, with the attention weights recomputed from q, k and the forward's
// log-sum-exp instead of being stored (xhh.club "flash attention" tag page, the
// summaries on recomputation in the backward pass; the skill page's overview of
// tiling plus recomputation).  Every result is produced by one workgroup in a
// fixed order, so repeated calls give identical bits (the deterministic mode of
// the Flash-Attention update notes, v2.4, and "FlashAttention 常用接口简单介绍",
// §5.3, here the only mode).
//
// Per (query row i, key j) of one head, with s the forward's final score in
// log2 units and L_i = lse_i·log2(e):
//   P = 2^(s - L_i),  dV_j += P dO_i,  dP = dO_i · V_j,
//   dS = P (dP - delta_i) with delta_i = dO_i · O_i (the row sum of P dP),
//   dU = dS (1 - t²) under softcap (t = tanh of the capped argument), else dS,
//   dQ_i += scale dU K_j,  dK_j += scale dU Q_i.
//
// Two kernels, the dQ kernel first:
//  * bwd_dkdv_kernel: one workgroup per (key tile, kv head, batch); each wave
//    owns 32 keys, keeps their K and V rows in registers and their dK and dV
//    accumulators in registers, and streams the query tiles of every query head
//    of its group through LDS.  S = Q Kᵀ and dP = dO Vᵀ put the key on the lane
//    (column) side, so P and dS are already in the A-operand layout of
//    dV += Pᵀ dO and dK += dSᵀ Q; dO and Q come out of LDS with the transposing
//    read ds_read_b64_tr_b16.
//  * bwd_dq_kernel: one workgroup per (query tile, query head, batch); each wave
//    owns 32 queries, keeps their Q and dO rows in registers, and streams K and V
//    tiles through LDS.  Sᵀ = K Qᵀ and dPᵀ = V dOᵀ put the query on the lane
//    side, so dS is in the A-operand layout of dQ += dS K, with K read
//    transposed.  It also forms delta_i from the dO row it holds and the O row,
//    and stores it in the workspace for the dK/dV kernel.
// Both streaming kernels hold their LDS tiles in an XOR-swizzled row-major
// layout (swz below) that serves the plain 16-byte operand reads and the
// transposing reads without bank conflicts.
#include <type_traits>
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// Element offset of 16-byte chunk c of row r in a [rows, D] LDS tile.  The chunk
// index is XORed with a function of the row such that
//  * 16 consecutive rows read at one chunk index land on 16 distinct 16-byte
//    bank groups (plain operand reads: lane <-> row), and
//  * rows 4a .. 4a+3 read at the four chunks of one 64-byte column block land on
//    four distinct 64-byte bank ranges (transposing reads).
//  (D = 32 and 96: row r starts at bank group 4*(r*D/32 mod 4), so rows
//  r .. r+3 already fall on distinct 64-byte ranges; XORing the low two chunk
//  bits with (r/4) mod 4 spreads 16 rows over all 16 groups and keeps every
//  chunk index below D/8.)
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "");
  if constexpr (D >= 128) return r * D + 8 * (c ^ (4 * (r & 3) + ((r >> 2) & 3)));
  else if constexpr (D == 64) return r * D + 8 * (c ^ (4 * ((r >> 1) & 1) + ((r >> 2) & 3)));
  else return r * D + 8 * (c ^ ((r >> 2) & 3));
}

// Score of one (query, key) pair in log2 units from the raw product x = q·k, and
// the factor 1 - t² that softcap puts on the gradient (1 without softcap).
template <bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ float score_l2(float x, float dist, float sl2, float cap_in, float cap_l2, float slope_l2,
                                          float& dcap) {
  float s;
  if constexpr (SOFTCAP) {
    const float e = exp2_fast(x * cap_in);                 // e^(2u/c), u = scale·x
    const float t = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
    s = cap_l2 * t;
    dcap = 1.f - t * t;
  } else {
    s = x * sl2;
    dcap = 1.f;
  }
  if constexpr (ALIBI) s = fmaf(-slope_l2, fabsf(dist), s);
  return s;
}

constexpr int kBig = 1 << 30;

// Workgroup shapes and register budgets (waves per SIMD the compiler targets).
#ifndef FA_BWD_KV_NW64
#define FA_BWD_KV_NW64 8
#endif
#ifndef FA_BWD_KV_WPE64
#define FA_BWD_KV_WPE64 2
#endif
#ifndef FA_BWD_KV_NW96
#define FA_BWD_KV_NW96 4
#endif
#ifndef FA_BWD_KV_NW128
#define FA_BWD_KV_NW128 4
#endif
#ifndef FA_BWD_KV_BMQ64
#define FA_BWD_KV_BMQ64 128
#endif
#ifndef FA_BWD_KV_BMQ96
#define FA_BWD_KV_BMQ96 64
#endif
#ifndef FA_BWD_KV_BMQ128
#define FA_BWD_KV_BMQ128 64
#endif
#ifndef FA_BWD_KV_WPE128
#define FA_BWD_KV_WPE128 1
#endif
#ifndef FA_BWD_Q_NW64
#define FA_BWD_Q_NW64 4
#endif
#ifndef FA_BWD_Q_NW128
#define FA_BWD_Q_NW128 8
#endif
#ifndef FA_BWD_Q_WPE64
#define FA_BWD_Q_WPE64 3
#endif
#ifndef FA_BWD_Q_WPE128
#define FA_BWD_Q_WPE128 2
#endif

// ---------------------------------------------------------------------------
// dK, dV: workgroup = NW waves x 32 keys; query tiles of BMQ rows through LDS.
// PART 0 accumulates both; at D = 256, where K, V, dK and dV of 32 keys do not
// fit one wave's registers, PART 1 accumulates dV only (S, then P^T dO) and
// PART 2 dK only (S, dP, then dS^T Q), in two launches; PART 2 keeps the V rows
// in LDS instead of registers (each lane reads back only what it wrote).
// ---------------------------------------------------------------------------
template <class E, int D, int NW, bool SOFTCAP, bool ALIBI, int PART>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D >= 96 ? FA_BWD_KV_WPE128 : FA_BWD_KV_WPE64)))
void bwd_dkdv_kernel(BackwardParams p) {
  constexpr bool DO_DV = PART != 2, DO_DK = PART != 1, V_LDS = PART == 2;
  using T = typename E::T;
  using V8 = typename E::V8;
  using V2 = typename E::V2;
  constexpr int BMQ = V_LDS ? 32 : D >= 128 ? FA_BWD_KV_BMQ128 : D >= 96 ? FA_BWD_KV_BMQ96 : FA_BWD_KV_BMQ64;   // query rows per LDS tile
  constexpr int BNK = NW * 32;            // keys per workgroup
  constexpr int CH = D / 8, DC = D / 16, DB = D / 32;
  constexpr int NT = NW * 64;
  constexpr int LQ = BMQ * CH / NT;       // 16-byte pieces per thread per tile, for Q and for dO
  static_assert(LQ * NT == BMQ * CH, "");
  __shared__ __attribute__((aligned(16))) T qsm[2][BMQ * D];
  __shared__ __attribute__((aligned(16))) T gsm[2][BMQ * D];     // dO
  __shared__ __attribute__((aligned(16))) float lsm[2][BMQ];     // lse in log2 units; +inf: row adds nothing
  __shared__ __attribute__((aligned(16))) float esm[2][BMQ];     // -delta
  __shared__ __attribute__((aligned(16))) T vsm[V_LDS ? NW * 32 * D : 8];   // V rows of each wave's keys

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (batch, kv head, key tile); the heads are spread over the XCDs
  // in contiguous ranges, and within a head the first key tiles (seen by the
  // most queries under a causal mask) go first
  int id = blockIdx.x;
  int head, kt;
  tile_order(id, (int)(gridDim.x / p.n_ktiles), p.n_ktiles, p.remap_xcd, p.order_group, head, kt);   // first key tiles: most queries
  const int b = head / p.Hkv, hk = head - b * p.Hkv;
  int sq = p.Sq, sk = p.Sk, qbase = 0, kbase = 0;
  if (p.cu_seqlens_q) {
    qbase = p.cu_seqlens_q[b];
    sq = p.cu_seqlens_q[b + 1] - qbase;
    kbase = p.cu_seqlens_k[b];
    sk = p.cu_seqlens_k[b + 1] - kbase;
  }
  const int shift = sk - sq;
  const int n0 = kt * BNK;
  if (n0 >= sk) return;                    // varlen: past this sequence's keys
  const int64_t bq = p.cu_seqlens_q ? 0 : (int64_t)b;

  // the lane's key and the query rows that may attend it: i in [a_j, b_j]
  const int j = n0 + wave * 32 + l32;
  const bool key_ok = j < sk;
  const int jc = min(j, sk - 1);
  int R = kBig;                            // key j allowed iff j <= i' + R (i' = i + shift) ...
  if (p.causal) R = 0;
  if (p.wr >= 0) R = min(R, p.wr);
  const int Lw = p.wl >= 0 ? p.wl : kBig;  // ... and j >= i' - Lw
  const int a_j = R == kBig ? 0 : max(0, j - shift - R);
  const int b_j = Lw == kBig ? sq - 1 : min(sq - 1, j - shift + Lw);
  // query range of the whole workgroup
  const int qlo = R == kBig ? 0 : max(0, n0 - shift - R);
  const int qhi = Lw == kBig ? sq : min(sq, min(n0 + BNK, sk) - 1 - shift + Lw + 1);
  const int t_lo = qlo / BMQ;
  const int nt = qhi > qlo ? (qhi + BMQ - 1) / BMQ - t_lo : 0;
  const int total = nt * p.group;

  // K and V rows of the lane's key: B operands of S = Q Kᵀ and dP = dO Vᵀ
  // (lane <-> key, d = 16dc + 8hi .. +7)
  V8 kr[DC], vr[DO_DK && !V_LDS ? DC : 1];
  T* const vw = vsm + (V_LDS ? wave * 32 * D : 0);   // the wave's V rows (V_LDS)
  {
    const T* kp = (const T*)p.k + bq * p.k_sb + (int64_t)(kbase + jc) * p.k_ss + (int64_t)hk * p.k_sh + hi * 8;
    const T* vp = (const T*)p.v + bq * p.v_sb + (int64_t)(kbase + jc) * p.v_ss + (int64_t)hk * p.v_sh + hi * 8;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      kr[dc] = *(const V8*)(kp + dc * 16);
      if constexpr (V_LDS) *(V8*)(vw + swz<D>(l32, 2 * dc + hi)) = *(const V8*)(vp + dc * 16);
      else if constexpr (DO_DK) vr[dc] = *(const V8*)(vp + dc * 16);
    }
  }
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_in = 2.f * p.scale * kLog2e / (SOFTCAP ? p.softcap : 1.f);

  // ---- global -> registers -> LDS staging of query tile `it` (rows past sq are
  // clamped to a real row and get lse = +inf, so their P is 0)
  u32x4 qst[LQ], gst[LQ];
  float lst = 0.f, est = 0.f;
  // a whole tile is read as a wave-uniform tile base plus a fixed 32-bit byte
  // offset per lane when a tile's rows span less than 2 GiB; the last, partial
  // tile (and huge strides) clamp row by row
  const bool off32 = (int64_t)BMQ * (p.q_ss > p.do_ss ? p.q_ss : p.do_ss) * (int64_t)sizeof(T) < ((int64_t)1 << 31) &&
                     p.q_ss >= 0 && p.do_ss >= 0;
  uint32_t qoff[LQ], goff[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
    qoff[i] = off32 ? (uint32_t)(((int64_t)r * p.q_ss + c * 8) * (int64_t)sizeof(T)) : 0u;
    goff[i] = off32 ? (uint32_t)(((int64_t)r * p.do_ss + c * 8) * (int64_t)sizeof(T)) : 0u;
  }
  auto gload = [&](int it) __attribute__((always_inline)) {
    const int g = it / nt, t = t_lo + (it - g * nt);
    const int hq = hk * p.group + g;
    const int r0 = t * BMQ;
    const T* qp = (const T*)p.q + bq * p.q_sb + (int64_t)qbase * p.q_ss + (int64_t)hq * p.q_sh;
    const T* gp = (const T*)p.dout + bq * p.do_sb + (int64_t)qbase * p.do_ss + (int64_t)hq * p.do_sh;
    if (off32 && r0 + BMQ <= sq) {
      const char* qt = (const char*)(qp + (int64_t)r0 * p.q_ss);
      const char* gt = (const char*)(gp + (int64_t)r0 * p.do_ss);
#pragma unroll
      for (int i = 0; i < LQ; ++i) {
        qst[i] = *(const u32x4*)(qt + qoff[i]);
        gst[i] = *(const u32x4*)(gt + goff[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LQ; ++i) {
        const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
        const int row = min(r0 + r, sq - 1);
        qst[i] = *(const u32x4*)(qp + (int64_t)row * p.q_ss + c * 8);
        gst[i] = *(const u32x4*)(gp + (int64_t)row * p.do_ss + c * 8);
      }
    }
    if (tid < BMQ) {
      const int row = r0 + tid;
      const int rc = min(row, sq - 1);
      const float l = p.lse[bq * p.lse_sb + (int64_t)hq * p.lse_sh + qbase + rc];
      const float d = p.delta[bq * p.dl_sb + (int64_t)hq * p.dl_sh + qbase + rc];
      lst = (row < sq && l != kNegInf) ? l * kLog2e : __builtin_inff();
      est = row < sq ? -d : 0.f;   // -delta: it starts the dP accumulation
    }
  };
  auto swrite = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
      const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
      *(u32x4*)(&qsm[buf][swz<D>(r, c)]) = qst[i];
      *(u32x4*)(&gsm[buf][swz<D>(r, c)]) = gst[i];
    }
    if (tid < BMQ) {
      lsm[buf][tid] = lst;
      esm[buf][tid] = est;
    }
  };

  f32x16 dk[DO_DK ? DB : 1], dv[DO_DV ? DB : 1];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    if constexpr (DO_DK) dk[db] = f32x16{};
    if constexpr (DO_DV) dv[db] = f32x16{};
  }

  // transposing-read addressing: lane (4a + g) of each 16-lane group reads row
  // 4hi + a (+8) of a 16-row chunk, elements 32db + 16((lane >> 4) & 1) + 4g .. +3
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_elem = 4 * (lane & 1);

  // one block of 32 queries (rows rb0 .. rb0+31 of the tile, first row i0) against
  // the wave's 32 keys
  auto block = [&](const T* qs, const T* gs, const float* ls, const float* es, int rb0, int i0, bool edge,
                   float slope_l2) __attribute__((always_inline)) {
    // register r of s holds query row rb0 + 8(r/4) + 4hi + r%4 for the lane's key;
    // dp starts from -delta of those rows, so it ends as dP - delta
    f32x4 L[4];
    f32x16 dp;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      L[t] = *(const f32x4*)(ls + rb0 + 8 * t + 4 * hi);
      const f32x4 nd = *(const f32x4*)(es + rb0 + 8 * t + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * t + e] = nd[e];
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int off = swz<D>(rb0 + l32, 2 * dc + hi);
      s = E::mfma32(*(const V8*)(qs + off), kr[dc], s);
      if constexpr (V_LDS) dp = E::mfma32(*(const V8*)(gs + off), *(const V8*)(vw + swz<D>(l32, 2 * dc + hi)), dp);
      else if constexpr (DO_DK) dp = E::mfma32(*(const V8*)(gs + off), vr[dc], dp);
    }
    V8 pa[2], sa[2];
    const float dist0 = (float)(i0 + 4 * hi + shift - j);
    // P and dS of every register, packed; then, in an edge block only, the
    // masked halves of the packed words are cleared under one uniform branch (a
    // mask test per element made the compiler branch on the edge flag at every
    // element).  Cleared bits are +0 whatever P was computed there.
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float pr[2], ds[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rr = r + u;
        const int qo = 8 * (rr >> 2) + (rr & 3);
        float dcap;
        const float x = score_l2<SOFTCAP, ALIBI>(s[rr], dist0 + (float)qo, sl2, cap_in, cap_l2, slope_l2, dcap);
        pr[u] = exp2_fast(x - L[rr >> 2][rr & 3]);
        ds[u] = DO_DK ? pr[u] * dp[rr] * dcap : 0.f;
      }
      const V2 pp = E::pack(pr[0], pr[1]);
      const V2 sp = E::pack(ds[0], ds[1]);
      pa[r >> 3][r & 7] = pp[0];
      pa[r >> 3][(r & 7) + 1] = pp[1];
      sa[r >> 3][r & 7] = sp[0];
      sa[r >> 3][(r & 7) + 1] = sp[1];
    }
    if (edge) {
      const int ilo = a_j - i0 - 4 * hi, ihi = b_j - i0 - 4 * hi;   // allowed row offsets
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 pw = __builtin_bit_cast(u32x4, pa[h]), sw = __builtin_bit_cast(u32x4, sa[h]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = 8 * h + 2 * w, q0 = 8 * (r >> 2) + (r & 3);   // rows of registers r, r+1
          const uint32_t keep = (q0 < ilo || q0 > ihi ? 0u : 0xffffu) | (q0 + 1 < ilo || q0 + 1 > ihi ? 0u : 0xffff0000u);
          pw[w] &= keep;
          sw[w] &= keep;
        }
        pa[h] = __builtin_bit_cast(V8, pw);
        sa[h] = __builtin_bit_cast(V8, sw);
      }
    }
    // dV += Pᵀ dO and dK += dSᵀ Q over two 16-query chunks; the contraction order
    // inside a chunk is the register order of P, matched by the transposing read
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int r1 = rb0 + 16 * c2 + tr_row, r2 = r1 + 8;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int o1 = swz<D>(r1, 4 * db + tr_chunk) + tr_elem;
        const int o2 = swz<D>(r2, 4 * db + tr_chunk) + tr_elem;
        if constexpr (DO_DV) {
          const i16x4 g0 = lds_read_tr16(gs + o1), g1 = lds_read_tr16(gs + o2);
          const V8 gb = __builtin_bit_cast(V8, __builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7));
          dv[db] = E::mfma32(pa[c2], gb, dv[db]);
        }
        if constexpr (DO_DK) {
          const i16x4 q0 = lds_read_tr16(qs + o1), q1 = lds_read_tr16(qs + o2);
          const V8 qb = __builtin_bit_cast(V8, __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7));
          dk[db] = E::mfma32(sa[c2], qb, dk[db]);
        }
      }
    }
  };

  if (total > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();
  // one step per query tile; the loop is unrolled by the two LDS buffers, so
  // every LDS address is a per-lane base plus an immediate
  auto step = [&](int it, auto Buf) __attribute__((always_inline)) {
    constexpr int buf = decltype(Buf)::value;
    if (it + 1 < total) gload(it + 1);
    const int g = it / nt, t = t_lo + (it - g * nt);
    const int hq = hk * p.group + g;
    const float slope_l2 = ALIBI ? p.alibi[hq] * kLog2e : 0.f;
#pragma unroll
    for (int blk = 0; blk < BMQ / 32; ++blk) {
      const int i0 = t * BMQ + blk * 32;
      const bool live = key_ok && max(a_j, i0) <= min(b_j, i0 + 31);
      if (!__any(live)) continue;
      const bool full = !key_ok || (a_j <= i0 && b_j >= i0 + 31);
      block(qsm[buf], gsm[buf], lsm[buf], esm[buf], blk * 32, i0, !__all(full), slope_l2);
    }
    if (it + 1 < total) swrite(buf ^ 1);
    __syncthreads();
  };
  for (int it = 0; it < total; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < total) step(it + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: register r of dk[db] / dv[db] is key n0 + 32w + 8(r/4) + 4hi + r%4,
  // column d = 32db + l32
  T* dkp = (T*)p.dk + bq * p.dk_sb + (int64_t)kbase * p.dk_ss + (int64_t)hk * p.dk_sh;
  T* dvp = (T*)p.dv + bq * p.dv_sb + (int64_t)kbase * p.dv_ss + (int64_t)hk * p.dv_sh;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = n0 + wave * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (key < sk) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (DO_DK) dkp[(int64_t)key * p.dk_ss + db * 32 + l32] = E::from_f32(dk[db][r] * p.scale);
        if constexpr (DO_DV) dvp[(int64_t)key * p.dv_ss + db * 32 + l32] = E::from_f32(dv[db][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = NW waves x 32 queries; key tiles of BN rows through LDS.  At
// D = 256 the dO rows of each wave's queries sit in LDS instead of registers
// (each lane reads back only what it wrote), so that Q, dQ and the products fit.
// ---------------------------------------------------------------------------
template <class E, int D, int NW, bool SOFTCAP, bool ALIBI>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : D >= 96 ? FA_BWD_Q_WPE128 : FA_BWD_Q_WPE64)))
void bwd_dq_kernel(BackwardParams p) {
  using T = typename E::T;
  using V8 = typename E::V8;
  using V2 = typename E::V2;
  constexpr bool G_LDS = D >= 256;
  constexpr int BN = D >= 256 ? 32 : 64;  // keys per LDS tile
  constexpr int BM = NW * 32;             // queries per workgroup
  constexpr int CH = D / 8, DC = D / 16, DB = D / 32;
  constexpr int NT = NW * 64;
  constexpr int LK = BN * CH / NT;
  static_assert(LK * NT == BN * CH, "");
  __shared__ __attribute__((aligned(16))) T ksm[2][BN * D];
  __shared__ __attribute__((aligned(16))) T vsm[2][BN * D];
  __shared__ __attribute__((aligned(16))) T gsm[G_LDS ? NW * 32 * D : 8];   // dO rows of each wave's queries

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int id = blockIdx.x;
  int head, rank;
  tile_order(id, (int)(gridDim.x / p.n_qtiles), p.n_qtiles, p.remap_xcd, p.order_group, head, rank);
  const int qt = p.n_qtiles - 1 - rank;      // last (longest) query tiles first
  const int b = head / p.Hq, hq = head - b * p.Hq;
  const int hk = hq / p.group;
  int sq = p.Sq, sk = p.Sk, qbase = 0, kbase = 0;
  if (p.cu_seqlens_q) {
    qbase = p.cu_seqlens_q[b];
    sq = p.cu_seqlens_q[b + 1] - qbase;
    kbase = p.cu_seqlens_k[b];
    sk = p.cu_seqlens_k[b + 1] - kbase;
  }
  const int shift = sk - sq;
  const int m0 = qt * BM;
  if (m0 >= sq) return;                    // varlen: past this sequence's queries
  const int64_t bq = p.cu_seqlens_q ? 0 : (int64_t)b;

  // the lane's query row and its allowed keys [j_lo, j_hi]
  const int i = m0 + wave * 32 + l32;
  const bool row_ok = i < sq;
  const int ic = min(i, sq - 1);
  const int ip = i + shift;
  int j_lo = 0, j_hi = sk - 1;
  if (p.wl >= 0) j_lo = max(j_lo, ip - p.wl);
  if (p.causal) j_hi = min(j_hi, ip);
  if (p.wr >= 0) j_hi = min(j_hi, ip + p.wr);
  // key range of the workgroup
  const int ip_first = m0 + shift, ip_last = min(m0 + BM, sq) - 1 + shift;
  int kv_lo = 0, kv_hi = sk;
  if (p.wl >= 0) kv_lo = max(0, ip_first - p.wl);
  if (p.causal) kv_hi = min(kv_hi, ip_last + 1);
  if (p.wr >= 0) kv_hi = min(kv_hi, ip_last + p.wr + 1);
  const int t_lo = kv_lo / BN;
  const int t_hi = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : t_lo;

  // Q and dO rows of the lane's query: B operands of Sᵀ = K Qᵀ and dPᵀ = V dOᵀ
  V8 qr[DC], gr[G_LDS ? 1 : DC];
  T* const gw = gsm + (G_LDS ? wave * 32 * D : 0);   // the wave's dO rows (G_LDS)
  // delta_i = dO_i · O_i of the lane's row: each lane holds half of the row's dO
  // and reads the same half of O, and the halves meet across lane ^ 32.  The
  // lane with hi = 0 also stores it for the dK/dV kernel, which runs after
  // this one.
  float Dl;
  {
    const T* qp = (const T*)p.q + bq * p.q_sb + (int64_t)(qbase + ic) * p.q_ss + (int64_t)hq * p.q_sh + hi * 8;
    const T* gp = (const T*)p.dout + bq * p.do_sb + (int64_t)(qbase + ic) * p.do_ss + (int64_t)hq * p.do_sh + hi * 8;
    const T* op = (const T*)p.out + bq * p.o_sb + (int64_t)(qbase + ic) * p.o_ss + (int64_t)hq * p.o_sh + hi * 8;
    float acc = 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      qr[dc] = *(const V8*)(qp + dc * 16);
      const V8 g = *(const V8*)(gp + dc * 16);
      const V8 o = *(const V8*)(op + dc * 16);
      if constexpr (G_LDS) *(V8*)(gw + swz<D>(l32, 2 * dc + hi)) = g;
      else gr[dc] = g;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
    acc += __shfl_xor(acc, 32);
    Dl = row_ok ? acc : 0.f;
    if (row_ok && hi == 0) p.delta[bq * p.dl_sb + (int64_t)hq * p.dl_sh + qbase + ic] = acc;
  }
  const float lse = p.lse[bq * p.lse_sb + (int64_t)hq * p.lse_sh + qbase + ic];
  const float L = (row_ok && lse != kNegInf) ? lse * kLog2e : __builtin_inff();
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_in = 2.f * p.scale * kLog2e / (SOFTCAP ? p.softcap : 1.f);
  const float slope_l2 = ALIBI ? p.alibi[hq] * kLog2e : 0.f;

  const T* kp = (const T*)p.k + bq * p.k_sb + (int64_t)kbase * p.k_ss + (int64_t)hk * p.k_sh;
  const T* vp = (const T*)p.v + bq * p.v_sb + (int64_t)kbase * p.v_ss + (int64_t)hk * p.v_sh;
  u32x4 kst[LK], vst[LK];
  // whole tiles: a uniform tile base plus a fixed 32-bit byte offset per lane
  // (see bwd_dkdv_kernel); the last, partial tile clamps row by row.  Not at
  // D = 64 with softcap or ALiBi, where the offsets' registers spill at the
  // budget of three waves per SIMD.
  constexpr bool kOff32 = D != 64 || !(SOFTCAP || ALIBI);
  const bool off32 = kOff32 &&
                     (int64_t)BN * (p.k_ss > p.v_ss ? p.k_ss : p.v_ss) * (int64_t)sizeof(T) < ((int64_t)1 << 31) &&
                     p.k_ss >= 0 && p.v_ss >= 0;
  uint32_t koff[LK], voff[LK];
#pragma unroll
  for (int u = 0; u < LK; ++u) {
    const int cid = tid + u * NT, r = cid / CH, c = cid - r * CH;
    koff[u] = off32 ? (uint32_t)(((int64_t)r * p.k_ss + c * 8) * (int64_t)sizeof(T)) : 0u;
    voff[u] = off32 ? (uint32_t)(((int64_t)r * p.v_ss + c * 8) * (int64_t)sizeof(T)) : 0u;
  }
  auto gload = [&](int t) __attribute__((always_inline)) {
    if (off32 && (t + 1) * BN <= sk) {
      const char* kt = (const char*)(kp + (int64_t)(t * BN) * p.k_ss);
      const char* vt = (const char*)(vp + (int64_t)(t * BN) * p.v_ss);
#pragma unroll
      for (int u = 0; u < LK; ++u) {
        kst[u] = *(const u32x4*)(kt + koff[u]);
        vst[u] = *(const u32x4*)(vt + voff[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < LK; ++u) {
        const int cid = tid + u * NT, r = cid / CH, c = cid - r * CH;
        const int row = min(t * BN + r, sk - 1);
        kst[u] = *(const u32x4*)(kp + (int64_t)row * p.k_ss + c * 8);
        vst[u] = *(const u32x4*)(vp + (int64_t)row * p.v_ss + c * 8);
      }
    }
  };
  auto swrite = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LK; ++u) {
      const int cid = tid + u * NT, r = cid / CH, c = cid - r * CH;
      *(u32x4*)(&ksm[buf][swz<D>(r, c)]) = kst[u];
      *(u32x4*)(&vsm[buf][swz<D>(r, c)]) = vst[u];
    }
  };

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_elem = 4 * (lane & 1);

  // keys kb0 .. kb0+31 of the tile (first key j0) against the wave's 32 queries
  auto block = [&](const T* ks, const T* vs, int kb0, int j0, bool edge) __attribute__((always_inline)) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int off = swz<D>(kb0 + l32, 2 * dc + hi);
      s = E::mfma32(*(const V8*)(ks + off), qr[dc], s);
      if constexpr (G_LDS) dp = E::mfma32(*(const V8*)(vs + off), *(const V8*)(gw + swz<D>(l32, 2 * dc + hi)), dp);
      else dp = E::mfma32(*(const V8*)(vs + off), gr[dc], dp);
    }
    // register r holds key j0 + 8(r/4) + 4hi + r%4 for the lane's query
    V8 sa[2];
    const float dist0 = (float)(ip - j0 - 4 * hi);
    // dS of every register, packed; in an edge block the masked halves are then
    // cleared under one uniform branch (see bwd_dkdv_kernel)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float ds[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rr = r + u;
        const int ko = 8 * (rr >> 2) + (rr & 3);
        float dcap;
        const float x = score_l2<SOFTCAP, ALIBI>(s[rr], dist0 - (float)ko, sl2, cap_in, cap_l2, slope_l2, dcap);
        const float pv = exp2_fast(x - L);
        ds[u] = pv * (dp[rr] - Dl) * dcap;
      }
      const V2 sp = E::pack(ds[0], ds[1]);
      sa[r >> 3][r & 7] = sp[0];
      sa[r >> 3][(r & 7) + 1] = sp[1];
    }
    if (edge) {
      const int jlo = j_lo - j0 - 4 * hi, jhi = j_hi - j0 - 4 * hi;   // allowed key offsets
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 sw = __builtin_bit_cast(u32x4, sa[h]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = 8 * h + 2 * w, k0 = 8 * (r >> 2) + (r & 3);   // keys of registers r, r+1
          sw[w] &= (k0 < jlo || k0 > jhi ? 0u : 0xffffu) | (k0 + 1 < jlo || k0 + 1 > jhi ? 0u : 0xffff0000u);
        }
        sa[h] = __builtin_bit_cast(V8, sw);
      }
    }
    // dQ += dS K over two 16-key chunks, K read transposed
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int r1 = kb0 + 16 * c2 + tr_row, r2 = r1 + 8;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 k0 = lds_read_tr16(ks + swz<D>(r1, 4 * db + tr_chunk) + tr_elem);
        const i16x4 k1 = lds_read_tr16(ks + swz<D>(r2, 4 * db + tr_chunk) + tr_elem);
        const V8 kb = __builtin_bit_cast(V8, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
        dq[db] = E::mfma32(sa[c2], kb, dq[db]);
      }
    }
  };

  if (t_hi > t_lo) {
    gload(t_lo);
    swrite(0);
  }
  __syncthreads();
  // one step per key tile, unrolled by the two LDS buffers (see bwd_dkdv_kernel)
  auto step = [&](int t, auto Buf) __attribute__((always_inline)) {
    constexpr int buf = decltype(Buf)::value;
    if (t + 1 < t_hi) gload(t + 1);
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      const int j0 = t * BN + kb * 32;
      const bool live = row_ok && max(j_lo, j0) <= min(j_hi, j0 + 31);
      if (!__any(live)) continue;
      const bool full = !row_ok || (j_lo <= j0 && j_hi >= j0 + 31);
      block(ksm[buf], vsm[buf], kb * 32, j0, !__all(full));
    }
    if (t + 1 < t_hi) swrite(buf ^ 1);
    __syncthreads();
  };
  for (int t = t_lo; t < t_hi; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < t_hi) step(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: register r of dq[db] is query m0 + 32w + 8(r/4) + 4hi + r%4, d = 32db + l32
  T* dqp = (T*)p.dq + bq * p.dq_sb + (int64_t)qbase * p.dq_ss + (int64_t)hq * p.dq_sh;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + wave * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (row < sq) {
#pragma unroll
      for (int db = 0; db < DB; ++db) dqp[(int64_t)row * p.dq_ss + db * 32 + l32] = E::from_f32(dq[db][r] * p.scale);
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int D> constexpr int bwd_dkdv_waves() { return D >= 128 ? FA_BWD_KV_NW128 : D >= 96 ? FA_BWD_KV_NW96 : FA_BWD_KV_NW64; }
template <int D> constexpr int bwd_dq_waves() { return D >= 256 ? 4 : D >= 128 ? FA_BWD_Q_NW128 : FA_BWD_Q_NW64; }

int backward_block_n(int D) { return (D >= 128 ? FA_BWD_KV_NW128 : D >= 96 ? FA_BWD_KV_NW96 : FA_BWD_KV_NW64) * 32; }
int backward_block_m(int D) { return (D >= 256 ? 4 : D >= 128 ? FA_BWD_Q_NW128 : FA_BWD_Q_NW64) * 32; }

template <class E, int D, bool SOFTCAP, bool ALIBI>
hipError_t launch_bwd_main(const BackwardParams& p, hipStream_t s) {
  // dQ first: it also computes delta = rowsum(dO * O) for its rows and stores it
  // in the workspace, where the dK/dV kernel reads it
  const int64_t gq = (int64_t)p.n_qtiles * p.B * p.Hq;
  if (gq > 0) {
    BackwardParams pq = p;
    pq.remap_xcd = ((int64_t)p.B * p.Hq) % 8 == 0;
    pq.order_group = order_group(p.causal != 0, (int64_t)p.B * p.Hq, p.n_qtiles, pq.remap_xcd);
    constexpr int NWQ = bwd_dq_waves<D>();
    hipLaunchKernelGGL((bwd_dq_kernel<E, D, NWQ, SOFTCAP, ALIBI>), dim3((unsigned)gq), dim3(NWQ * 64), 0, s, pq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int NWK = bwd_dkdv_waves<D>();
  const int64_t gk = (int64_t)p.n_ktiles * p.B * p.Hkv;
  if (gk > 0) {
    BackwardParams pk = p;
    pk.remap_xcd = ((int64_t)p.B * p.Hkv) % 8 == 0;
    pk.order_group = order_group(p.causal != 0, (int64_t)p.B * p.Hkv, p.n_ktiles, pk.remap_xcd);
    if constexpr (D >= 256) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, NWK, SOFTCAP, ALIBI, 1>), dim3((unsigned)gk), dim3(NWK * 64), 0, s, pk);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, NWK, SOFTCAP, ALIBI, 2>), dim3((unsigned)gk), dim3(NWK * 64), 0, s, pk);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, NWK, SOFTCAP, ALIBI, 0>), dim3((unsigned)gk), dim3(NWK * 64), 0, s, pk);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

template <class E, int D>
hipError_t launch_bwd_d(const BackwardParams& p, hipStream_t s) {
  const bool cap = p.softcap > 0.f, al = p.alibi != nullptr;
  if (cap && al) return launch_bwd_main<E, D, true, true>(p, s);
  if (cap) return launch_bwd_main<E, D, true, false>(p, s);
  if (al) return launch_bwd_main<E, D, false, true>(p, s);
  return launch_bwd_main<E, D, false, false>(p, s);
}

template <class E>
hipError_t launch_bwd_e(int D, const BackwardParams& p, hipStream_t s) {
  switch (D) {
    case 32: return launch_bwd_d<E, 32>(p, s);
    case 64: return launch_bwd_d<E, 64>(p, s);
    case 96: return launch_bwd_d<E, 96>(p, s);
    case 256: return launch_bwd_d<E, 256>(p, s);
    default: return launch_bwd_d<E, 128>(p, s);
  }
}

hipError_t launch_backward(Dtype dt, int D, const BackwardParams& p, hipStream_t s) {
  if (dt == kBF16) return launch_bwd_e<BF16>(D, p, s);
  return launch_bwd_e<F16>(D, p, s);
}

}  // namespace fa
