// Prefill forward kernel for gfx950: exact attention, tile by tile, with an
// online softmax, so the Sq x Sk score matrix never leaves the chip.
//
// The method: tiles of K and V are streamed through on-chip memory while each
// query row keeps a running maximum and running sum of its exponentiated
// scores; the partial output is rescaled whenever the maximum grows, and the
// log-sum-exp is written next to the output (xhh.club "flash attention" tag
// page, the tiling / online-softmax summaries; "FlashAttention 常用接口简单介绍",
// §1 and §3.1 for the interface and the lse output).  Masks and score
// transforms follow the Flash-Attention v2.0-v2.7 update notes (bottom-right
// causal, v2.3 local window, v2.4 ALiBi, v2.6 softcap).
//
// CDNA4 mapping (one workgroup = NW waves of 64 lanes, 32 query rows per wave):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: keys on the M side, so each
//    lane holds 16 scores of ONE query per 32-key block; lanes l and l^32 share
//    the query, so a row max / sum is in-lane work plus one permlane32 swap.
//  * O^T += V^T P^T on the same MFMA: P stays in registers as the B operand (the
//    score layout already is the B layout up to a fixed permutation of the
//    contraction index, applied identically to V); V^T comes out of LDS with the
//    transposing read ds_read_b64_tr_b16.
//  * K and V tiles are double-buffered in LDS with padded rows (conflict-free
//    reads, see k_stride / v_stride); the next tile's global loads are issued
//    before the current tile's math.
//  * scale·log2(e) is folded into the exp2 argument (one FMA + v_exp_f32 per score).
//  * tiles that are fully masked for a wave are skipped; mask arithmetic runs only
//    on tiles that straddle a mask edge.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

constexpr float kTau = 8.f;   // lazy-rescale threshold (log2 units)
constexpr float kTauPow = 256.f;   // 2^kTau
// |out| from which a wave recomputes its rows with P carried in two parts (see
// the epilogue of prefill_kernel).  Below it half an ulp of out leaves about
// half of the error bar to the rounding of P.  prefill_kernel normalises O by
// the fp32 sum of P, so rounding P perturbs out by up to u * sum_j w_j |v_j|
// (u the unit roundoff of P's type), and the bar is |out| >= 1 for both types.
// prefill_pp_kernel normalises by the sum of the rounded P, which makes out a
// convex combination of the rounded weights and the perturbation
// u * sum_j w_j |v_j - out|, smaller where |out| is large; there bf16 (half an
// ulp 3.9e-3 under 2, against 8e-3) recomputes from 2.
constexpr float kPreciseOut = 1.f;
template <class E> constexpr float precise_out_pp() { return std::is_same_v<E, BF16> ? 2.f : 1.f; }

// Head dims from which the ping-pong kernel is used.  With D = 64 the softmax
// phase outweighs the MFMA phase: the ping-pong kernel there, even with the
// lean softmax phase, runs at the main kernel's rate and not above it.
#ifndef FA_PREFILL_PINGPONG_MIN_D
#define FA_PREFILL_PINGPONG_MIN_D 128
#endif
// 1: the ping-pong kernel's lean softmax phase (lazy max, fp32 sum only) for
// plain masks; softcap and ALiBi keep the full phase (see prefill_pp_kernel)
#ifndef FA_PREFILL_TRANS_GROUPS
#define FA_PREFILL_TRANS_GROUPS 3    // VALU instructions placed before each exponential of P
#endif
#ifndef FA_PP_LEAN
#define FA_PP_LEAN 1
#endif
#ifndef FA_PREFILL_WAVES_PER_EU
#define FA_PREFILL_WAVES_PER_EU 2    // register budget: 256 VGPRs+AGPRs per wave
#endif

typedef short i16x8 __attribute__((ext_vector_type(8)));


// LDS row strides (elements) of the K and V tiles.  Padding instead of an XOR
// swizzle keeps every LDS read at "one base register + immediate offset":
//  * K rows of 2D+16 bytes: the 16 lanes of a 16-byte K read hit 16 different
//    rows, whose starts then fall on 16 distinct 16-byte bank groups;
//  * V rows of 192 bytes (D = 32, 64, 96) or 2D+64 bytes (D = 128): a transposing
//    read covers 4 rows x 64 bytes per 32 lanes, and row starts 64 bytes apart
//    modulo 256 map those rows to 4 disjoint bank ranges.
template <int D> constexpr int k_stride() { return D + 8; }
#ifndef FA_PREFILL_VPAD
#define FA_PREFILL_VPAD 32
#endif
template <int D> constexpr int v_stride() { return D + (D == 96 ? 0 : D == 32 ? 64 : FA_PREFILL_VPAD); }

// Register budgets (waves per SIMD): four for the plain kernels up to D = 64,
// except three for the 4-wave D = 64 instance (its two 16-byte K/V loads per
// thread and tile need about 155 registers; it runs the narrow windows, three
// workgroups per CU); one at D = 256 and for the 2-wave D >= 96 instances;
// FA_PREFILL_WAVES_PER_EU otherwise.
template <class E, int D, int BN, int NW, int RB, bool SOFTCAP, bool ALIBI, bool F8 = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D >= 256 || (NW <= 2 && D >= 96) ? 1 : D <= 64 && RB == 1 && !SOFTCAP && !ALIBI ? (D == 64 && NW == 4 ? 3 : 4) : FA_PREFILL_WAVES_PER_EU)))
void prefill_kernel(PrefillParams p) {
  using T = typename E::T;
  using V8 = typename E::V8;
  using V2 = typename E::V2;
  // F8: q, k, v are fp8 e4m3 (OCP); Q K^T runs on the fp8 MFMA, V is widened
  // exactly to bf16 (T) on its way into LDS, and P V, out and lse are as for bf16
  using TI = std::conditional_t<F8, uint8_t, T>;          // element type of q, k, v
  // operand of Q K^T: 8 elements (v_mfma_f32_32x32x16_{f16,bf16}) or, for fp8,
  // 32 (v_mfma_f32_32x32x64_f8f6f4: one instruction per 64 of the D products)
  using QV = std::conditional_t<F8, i32x8, V8>;
  using KST = std::conditional_t<F8, u32x2, u32x4>;       // 8 staged elements of K or V
  constexpr int BM = NW * 32 * RB;        // query rows per workgroup
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int KB = BN / 32;             // 32-key blocks per tile
  constexpr int DC = F8 ? D / 64 : D / 16;   // contraction steps of Q K^T
  constexpr int DW = F8 ? 64 : 16;        // elements of d per step
  constexpr int DB = D / 32;              // 32-wide blocks of the output
  constexpr int NT = NW * 64;
  constexpr int LOADS = (BN * CH + NT - 1) / NT;   // 16-byte loads per thread per tile, for K and for V
  // with D = 32 or 96 the last load round covers only the first waves (a whole
  // number of them, so the guard is wave-uniform)
  constexpr bool EVEN = LOADS * NT == BN * CH;
  static_assert(EVEN || (BN * CH) % 64 == 0, "partial load rounds must end on a wave boundary");
  constexpr bool PLAIN = !SOFTCAP && !ALIBI;

  constexpr int KS = k_stride<D>(), VS = v_stride<D>();
  // K row stride in elements of TI: fp8 rows of D+16 bytes keep the 16-byte
  // pieces of the 32-byte operand reads aligned, and 16 lanes on distinct banks
  constexpr int KSI = F8 ? D + 16 : KS;
  __shared__ __attribute__((aligned(16))) T ksm[2][BN * KS];   // K tiles, double-buffered
  __shared__ __attribute__((aligned(16))) T vsm[2][BN * VS];   // V tiles

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) index
  lds_poison(ksm, sizeof(ksm), tid, NT);
  lds_poison(vsm, sizeof(vsm), tid, NT);

  // ---- workgroup -> (batch, query head, query tile); heads are spread over the
  // 8 XCDs in contiguous ranges so the workgroups sharing K/V share an L2, and
  // within a head the longest (last) query tiles go first.
  int head, rank;
  tile_order(blockIdx.x, p.n_heads, p.n_qtiles, p.remap_xcd, p.order_group, head, rank);
  const int qt = p.n_qtiles - 1 - rank;      // the last query tiles see the most keys under a causal mask
  const int b = head / p.Hq, hq = head - b * p.Hq;
  const int hk = hq / p.group;

  int sq = p.Sq, sk = p.Sk, qbase = 0, kbase = 0;
  if (p.cu_seqlens_q) {
    qbase = p.cu_seqlens_q[b];
    sq = p.cu_seqlens_q[b + 1] - qbase;
    kbase = p.cu_seqlens_k[b];
    sk = p.cu_seqlens_k[b + 1] - kbase;
  }
  const int m0 = qt * BM;
  if (m0 >= sq) return;

  const int64_t bq = p.cu_seqlens_q ? 0 : (int64_t)b;
  const TI* qp = (const TI*)p.q + bq * p.q_sb + (int64_t)qbase * p.q_ss + (int64_t)hq * p.q_sh;
  const TI* kp = (const TI*)p.k + bq * p.k_sb + (int64_t)kbase * p.k_ss + (int64_t)hk * p.k_sh;
  const TI* vp = (const TI*)p.v + bq * p.v_sb + (int64_t)kbase * p.v_ss + (int64_t)hk * p.v_sh;
  T* op = (T*)p.out + bq * p.o_sb + (int64_t)qbase * p.o_ss + (int64_t)hq * p.o_sh;
  float* lp = p.lse + bq * p.lse_sb + (int64_t)hq * p.lse_sh + qbase;

  // ---- key range of the workgroup (bottom-right alignment: row i sits at i + sk - sq)
  const int shift = sk - sq;
  const int ip_first = m0 + shift, ip_last = min(m0 + BM, sq) - 1 + shift;
  int kv_lo = 0, kv_hi = sk;
  if (p.wl >= 0) kv_lo = max(0, ip_first - p.wl);
  if (p.causal) kv_hi = min(kv_hi, ip_last + 1);
  if (p.wr >= 0) kv_hi = min(kv_hi, ip_last + p.wr + 1);
  const int t_lo = kv_lo / BN;
  const int t_hi = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : t_lo;

  // ---- the wave owns RB blocks of 32 query rows; block rb covers rows
  // m0 + rb*(NW*32) + wave*32 + [0, 32), so at the causal diagonal every wave
  // holds one block from each half of the tile and the waves stay balanced.
  int qrow[RB], j_lo[RB], j_hi[RB];
  bool row_ok[RB];
  int lo_min[RB], lo_max[RB], hi_min[RB], hi_max[RB];   // bounds over the block's rows (scalar)
  bool blk_live[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int w0 = m0 + rb * NW * 32 + wave * 32;
    qrow[rb] = w0 + l32;
    row_ok[rb] = qrow[rb] < sq;
    const int ip = qrow[rb] + shift;
    j_lo[rb] = 0; j_hi[rb] = sk - 1;
    if (p.wl >= 0) j_lo[rb] = max(j_lo[rb], ip - p.wl);
    if (p.causal) j_hi[rb] = min(j_hi[rb], ip);
    if (p.wr >= 0) j_hi[rb] = min(j_hi[rb], ip + p.wr);
    const int w1 = min(w0 + 32, sq) - 1;
    blk_live[rb] = w0 < sq;
    lo_min[rb] = 0; lo_max[rb] = 0; hi_min[rb] = sk - 1; hi_max[rb] = sk - 1;
    if (p.wl >= 0) { lo_min[rb] = max(0, w0 + shift - p.wl); lo_max[rb] = max(0, w1 + shift - p.wl); }
    if (p.causal) { hi_min[rb] = min(hi_min[rb], w0 + shift); hi_max[rb] = min(hi_max[rb], w1 + shift); }
    if (p.wr >= 0) { hi_min[rb] = min(hi_min[rb], w0 + shift + p.wr); hi_max[rb] = min(hi_max[rb], w1 + shift + p.wr); }
    if (lo_min[rb] > hi_max[rb]) blk_live[rb] = false;   // no row of the block sees any key
  }

  // ---- Q operand (B of S^T = K Q^T): lane holds row qrow, d = DW*dc + (DW/2)*hi
  // .. +DW/2-1 (fp8 rows are only 8-byte aligned: read in 8-byte pieces)
  QV qr[RB][DC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const TI* qrp = qp + (int64_t)qrow[rb] * p.q_ss + dc * DW + hi * (DW / 2);
      if (!row_ok[rb]) {
        qr[rb][dc] = QV{};
      } else if constexpr (F8) {
        u32x2 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = *(const u32x2*)(qrp + 8 * u);
        qr[rb][dc] = i32x8{(int)w[0][0], (int)w[0][1], (int)w[1][0], (int)w[1][1],
                           (int)w[2][0], (int)w[2][1], (int)w[3][0], (int)w[3][1]};
      } else {
        qr[rb][dc] = *(const QV*)qrp;
      }
    }

  float slope_l2 = 0.f, ipf[RB];
  if constexpr (ALIBI) slope_l2 = p.alibi[hq] * kLog2e;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) ipf[rb] = (float)(qrow[rb] + shift);
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;                 // softcap in log2 units
  const float cap_in = 2.f * p.scale * kLog2e / (SOFTCAP ? p.softcap : 1.f);
  const float mult = PLAIN ? sl2 : 1.f;

  // ---- global -> register staging of one K/V tile (rows past sk are clamped to a
  // real row; their scores are masked, so their values only ever meet p = 0)
  // Whole tiles are addressed as a scalar tile base plus a fixed 32-bit byte offset
  // per lane; the last, partial tile clamps row by row.
  KST kst[LOADS], vst[LOADS];
  uint32_t koff[LOADS], voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
    koff[i] = (uint32_t)(r * p.k_ss + c * 8) * (uint32_t)sizeof(TI);
    voff[i] = (uint32_t)(r * p.v_ss + c * 8) * (uint32_t)sizeof(TI);
  }
  const bool off32 = p.k_ss >= 0 && p.v_ss >= 0 && p.k_ss < (1 << 24) / BN && p.v_ss < (1 << 24) / BN;
  auto gload = [&](int tile) __attribute__((always_inline)) {
    const int j0 = tile * BN;
    if (off32 && j0 + BN <= sk) {
      const char* kt = (const char*)(kp + (int64_t)j0 * p.k_ss);
      const char* vt = (const char*)(vp + (int64_t)j0 * p.v_ss);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        if (!EVEN && tid + i * NT >= BN * CH) continue;
        kst[i] = *(const KST*)(kt + koff[i]);
        vst[i] = *(const KST*)(vt + voff[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
        if (!EVEN && cid >= BN * CH) continue;
        const int j = min(j0 + r, sk - 1);
        kst[i] = *(const KST*)(kp + (int64_t)j * p.k_ss + c * 8);
        vst[i] = *(const KST*)(vp + (int64_t)j * p.v_ss + c * 8);
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
      if (!EVEN && cid >= BN * CH) continue;
      *(KST*)(reinterpret_cast<TI*>(ksm[buf]) + r * KSI + c * 8) = kst[i];
      if constexpr (F8) {
        // 8 fp8 values -> 8 bf16 (exact: every e4m3 value is a bf16 value)
        u32x4 w;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)vst[i][h], false);
          const f32x2 hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vst[i][h], true);
          w[2 * h] = __builtin_bit_cast(uint32_t, E::pack(lo[0], lo[1]));
          w[2 * h + 1] = __builtin_bit_cast(uint32_t, E::pack(hi2[0], hi2[1]));
        }
        *(u32x4*)(&vsm[buf][r * VS + c * 8]) = w;
      } else {
        *(u32x4*)(&vsm[buf][r * VS + c * 8]) = vst[i];
      }
    }
  };

  f32x16 o[RB][DB];
  // Running row max m (log2 units) and row sum lx of the fp32 P over this lane's
  // keys (the other half is added at the end).  lx normalises out and gives an
  // lse free of the rounding of P; m is lazy (see step): O and lx are rescaled
  // only when m moves, which leaves the result exact.
  float m[RB], lx[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x16{};
    m[rb] = kNegInf; lx[rb] = 0.f;
  }

  // S^T = K Q^T for one tile: s[rb][kb][r] is key j0 + 32kb + 8(r/4) + 4hi + (r%4) of
  // row qrow[rb]; each K operand read from LDS feeds the RB row blocks.  Softcap and
  // ALiBi turn the scores into log2 units; masked scores become -inf when edge is set.
  auto scores = [&](bool edge, int j0, const T* Ks, f32x16 (&s)[RB][KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[rb][kb] = f32x16{};
    const TI* kbase = reinterpret_cast<const TI*>(Ks) + l32 * KSI + hi * (DW / 2);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        QV a;
        if constexpr (F8) {
          const u32x4 a0 = *(const u32x4*)(kbase + kb * 32 * KSI + dc * DW);
          const u32x4 a1 = *(const u32x4*)(kbase + kb * 32 * KSI + dc * DW + 16);
          a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        } else {
          a = *(const QV*)(kbase + kb * 32 * KSI + dc * DW);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          // fp8 e4m3 (format 0) for both operands, no block scales
          if constexpr (F8) s[rb][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qr[rb][dc], s[rb][kb], 0, 0, 0, 0, 0, 0);
          else s[rb][kb] = E::mfma32(a, qr[rb][dc], s[rb][kb]);
        }
      }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (!PLAIN) {
        const float dj0 = (float)(j0 + 4 * hi) - ipf[rb];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = s[rb][kb][r];
            if constexpr (SOFTCAP) {
              const float e = exp2_fast(x * cap_in);
              x = fmaf(-2.f * cap_l2, __builtin_amdgcn_rcpf(e + 1.f), cap_l2);
            } else {
              x *= sl2;
            }
            if constexpr (ALIBI) {
              const float dist = dj0 + (float)(kb * 32 + (r >> 2) * 8 + (r & 3));
              x = fmaf(-slope_l2, fabsf(dist), x);
            }
            s[rb][kb][r] = x;
          }
      }
      if (edge) {
        // key j is kept iff j_lo <= j <= j_hi, i.e. iff j - j_lo, taken unsigned,
        // is below the row's key count (0 for a row without keys): one add, one
        // compare and one select per score
        const int base = j0 + 4 * hi - j_lo[rb];
        const uint32_t cnt = (uint32_t)max(j_hi[rb] - j_lo[rb] + 1, 0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t x = (uint32_t)(base + kb * 32 + (r >> 2) * 8 + (r & 3));
            if (x >= cnt) s[rb][kb][r] = kNegInf;
          }
      }
    }
  };

  // P = exp2(s * mult - mu), rounded for the P V product, and this lane's sum of
  // the unrounded fp32 P (lxs) of each row block
  auto probs = [&](f32x16 (&s)[RB][KB], const float (&mu)[RB], V2 (&pk)[RB][KB][8],
                   float (&lxs)[RB]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float ax = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = exp2_fast(fmaf(s[rb][kb][r], mult, -mu[rb]));
          const float p1 = exp2_fast(fmaf(s[rb][kb][r + 1], mult, -mu[rb]));
          pk[rb][kb][r >> 1] = E::pack(p0, p1);
          ax += p0 + p1;
        }
      lxs[rb] = ax;
    }
    // 8-wave workgroups only: the 4-wave (window, D = 96) instances measured
    // 1-3% slower with the exponentials spread
    spread_exponentials<RB * KB * 16, NW == 8 ? FA_PREFILL_TRANS_GROUPS : 0>();
  };

  // One tile for the wave's RB row blocks; mask arithmetic runs only when edge is set.
  // The row max is not taken on every tile: once every row of the wave has a running
  // max m, P is formed against it and kept when no lane's partial sum of P exceeds
  // 2^kTau (then no single P does, and the rounded P stays far from overflow).
  // Otherwise (first tile of a row, or a score more than about kTau above m) the
  // tile is redone: the scores are recomputed, m moves to the exact new max, and O,
  // l, lx are rescaled.  Any m not below the true max gives the same exact result.
  auto step = [&](bool edge, int j0, const T* Ks, const T* Vs) __attribute__((always_inline)) {
    f32x16 s[RB][KB];
    V2 pk[RB][KB][8];
    float lxs[RB];
    bool unset = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) unset |= m[rb] == kNegInf;
    bool redo = true;
    if (!__any(unset)) {
      scores(edge, j0, Ks, s);
      probs(s, m, pk, lxs);
      bool big = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) big |= lxs[rb] > kTauPow;
      redo = __any(big);
    }
    if (redo) {
      scores(edge, j0, Ks, s);
      float mu[RB];
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          mx0 = fmaxf(fmaxf(mx0, s[rb][0][r]), s[rb][0][r + 1]);
          mx1 = fmaxf(fmaxf(mx1, s[rb][KB - 1][r]), s[rb][KB - 1][r + 1]);
        }
#pragma unroll
        for (int kb = 1; kb + 1 < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx0 = fmaxf(fmaxf(mx0, s[rb][kb][r]), s[rb][kb][r + 1]);
        const float mx = max_halves(fmaxf(mx0, mx1)) * mult;
        mu[rb] = fmaxf(m[rb], mx);
        grow |= mu[rb] > m[rb];
      }
      if (__any(grow)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float alpha = mu[rb] == kNegInf ? 1.f : exp2_fast(m[rb] - mu[rb]);
          m[rb] = mu[rb];
          lx[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[rb][db] *= alpha;
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) mu[rb] = m[rb] == kNegInf ? 0.f : m[rb];
      probs(s, mu, pk, lxs);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lx[rb] += lxs[rb];

    // O^T += V^T P^T over 16-key chunks; each V operand read feeds the RB blocks.
    // Transposing read: lane (g = lane % 16) of each 16-lane group addresses row
    // 16c + 4hi + g/4 (+8 for the second half), columns 32db + 16((lane/16)%2) + 4(g%4).
    const T* vbase = Vs + (hi * 4 + ((lane & 15) >> 2)) * VS + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    // the V operands of two 16-key chunks are read ahead of their MFMAs (all
    // four chunks at once do not fit the register budget)
    V8 vop[BN / 16][DB];
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
      if ((c & 1) == 0) {
#pragma unroll
        for (int cc = c; cc < c + 2 && cc < BN / 16; ++cc)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const i16x4 x0 = lds_read_tr16(vbase + cc * 16 * VS + db * 32);
            const i16x4 x1 = lds_read_tr16(vbase + (cc * 16 + 8) * VS + db * 32);
            vop[cc][db] = __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        __builtin_amdgcn_sched_barrier(0);
      }
      const int kb = c >> 1, c2 = c & 1;
      V8 bop[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bop[rb][2 * e] = pk[rb][kb][4 * c2 + e][0];
          bop[rb][2 * e + 1] = pk[rb][kb][4 * c2 + e][1];
        }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][db] = E::mfma32(vop[c][db], bop[rb], o[rb][db]);
      }
    }
  };

  // One tile of the precise pass (see the epilogue): P against the final m, split
  // into two rounded parts that both go through P V; lx sums the fp32 P.
  auto step_precise = [&](bool edge, int j0, const T* Ks, const T* Vs) __attribute__((always_inline)) {
    f32x16 s[RB][KB];
    scores(edge, j0, Ks, s);
    float mu[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mu[rb] = m[rb] == kNegInf ? 0.f : m[rb];
    const T* vbase = Vs + (hi * 4 + ((lane & 15) >> 2)) * VS + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
      const int kb = c >> 1, c2 = c & 1;
      V8 bh[RB], bl[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = exp2_fast(fmaf(s[rb][kb][8 * c2 + e], mult, -mu[rb]));
          const T h = E::from_f32(pv);
          bh[rb][e] = h;
          bl[rb][e] = E::from_f32(pv - E::to_f32(h));
          lx[rb] += pv;
        }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 x0 = lds_read_tr16(vbase + c * 16 * VS + db * 32);
        const i16x4 x1 = lds_read_tr16(vbase + (c * 16 + 8) * VS + db * 32);
        const V8 a = __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          o[rb][db] = E::mfma32(a, bh[rb], o[rb][db]);
          o[rb][db] = E::mfma32(a, bl[rb], o[rb][db]);
        }
      }
    }
  };

  // ---- tiles in ascending key order.  Liveness and the need for masks are
  // decided per wave from its own rows, so a wave's arithmetic does not depend
  // on how many rows its workgroup holds.
  if (t_lo < t_hi) {
    gload(t_lo);
    swrite(0);
  }
  wait_vmem_all();   // Q operands ready: the loop waits only for its own tile loads
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    if (t + 1 < t_hi) gload(t + 1);
    const int j0 = t * BN;
    bool any_live = false, all_full = true;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool live = blk_live[rb] && j0 + BN - 1 >= lo_min[rb] && j0 <= hi_max[rb];
      any_live |= live;
      all_full &= live && j0 >= lo_max[rb] && j0 + BN - 1 <= hi_min[rb];
    }
    if (any_live) step(!all_full, j0, ksm[buf], vsm[buf]);
    if (t + 1 < t_hi) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: out = O / lx, lse = ln(sum exp(scores)) = (m + log2 lx) * ln 2
  auto write_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float lxt = sum_halves(lx[rb]);
      if (row_ok[rb]) {
        const float inv = lxt > 0.f ? p.out_scale / lxt : 0.f;
        T* orow = op + (int64_t)qrow[rb] * p.o_ss;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            V2 a = E::pack(o[rb][db][4 * gq] * inv, o[rb][db][4 * gq + 1] * inv);
            V2 c = E::pack(o[rb][db][4 * gq + 2] * inv, o[rb][db][4 * gq + 3] * inv);
            u32x2 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c)};
            *(u32x2*)(orow + db * 32 + gq * 8 + hi * 4) = w;
          }
        if (hi == 0) lp[qrow[rb]] = lxt > 0.f ? (m[rb] + __log2f(lxt)) * kLn2 : kNegInf;
      }
    }
  };

  // Rounding P to the input type before P V perturbs each weight by up to half
  // an ulp of that type.  Where |out| >= 2 half an ulp of out itself nearly
  // fills the error bar, so a wave with an output element of magnitude
  // kPreciseOut or more walks its tiles again: P is taken against the final
  // row max m (every P <= 2^kTau), split into hi = RN(P) and lo = RN(P - hi),
  // and O accumulates V hi + V lo, which carries P to about 2^-22 relative.
  bool need = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lt = sum_halves(lx[rb]);
    float om = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) om = fmaxf(om, fabsf(o[rb][db][r]));
    need |= row_ok[rb] && lt > 0.f && om * (p.out_scale / lt) >= kPreciseOut;
  }
  const bool wave_need = __any(need);
  if (!wave_need) write_rows();
  if (__syncthreads_or(wave_need)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[rb][db] = f32x16{};
      lx[rb] = 0.f;
    }
    if (t_lo < t_hi) {
      gload(t_lo);
      swrite(0);
    }
    __syncthreads();
    for (int t = t_lo; t < t_hi; ++t) {
      const int buf = (t - t_lo) & 1;
      if (t + 1 < t_hi) gload(t + 1);
      const int j0 = t * BN;
      bool any_live = false, all_full = true;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bool live = blk_live[rb] && j0 + BN - 1 >= lo_min[rb] && j0 <= hi_max[rb];
        any_live |= live;
        all_full &= live && j0 >= lo_max[rb] && j0 + BN - 1 <= hi_min[rb];
      }
      if (wave_need && any_live) step_precise(!all_full, j0, ksm[buf], vsm[buf]);
      if (t + 1 < t_hi) swrite(buf ^ 1);
      __syncthreads();
    }
    if (wave_need) write_rows();
  }
}

// ---------------------------------------------------------------------------
// Ping-pong variant.  The 8 waves form two groups (waves w and w+4 share a
// SIMD).  Each wave alternates a GEMM phase (Q K^T of tile j on MFMA, then
// P V of tile j-1) and a softmax phase (scores of tile j -> P on VALU and the
// transcendental unit), and group 1 runs one phase behind group 0, so on every
// SIMD one wave keeps the matrix cores busy while the other does the
// exponentials.  Phases end at workgroup barriers; K/V tiles rotate through
// three LDS stages, each wave staging its share of tile j+1 during GEMM phase
// j-1 and storing it during GEMM phase j.
// LEAN selects the softmax phase of prefill_kernel (P against the running max
// without a max reduction, the fp32 sum of P normalising out); otherwise the
// max is taken on every tile and out is normalised by the sum of the rounded
// P, which suits softcap and ALiBi: steep ALiBi slopes raise the max within
// most tiles, and the rounded-P normalisation lets bf16 rows up to |out| = 2
// skip the precise pass.
// ---------------------------------------------------------------------------
template <class E, int D, int BN, bool SOFTCAP, bool ALIBI, bool LEAN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(FA_PREFILL_WAVES_PER_EU)))
void prefill_pp_kernel(PrefillParams p) {
  using T = typename E::T;
  using V8 = typename E::V8;
  using V2 = typename E::V2;
  constexpr int NW = 8;
  constexpr int BM = NW * 32;
  constexpr int CH = D / 8;
  constexpr int KB = BN / 32;
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int NT = NW * 64;
  constexpr int LOADS = BN * CH / NT;
  static_assert(LOADS * NT == BN * CH, "tile must split evenly over the workgroup");
  constexpr bool PLAIN = !SOFTCAP && !ALIBI;
  constexpr int KS = k_stride<D>(), VS = v_stride<D>();
  __shared__ __attribute__((aligned(16))) T ksm[3][BN * KS];
  __shared__ __attribute__((aligned(16))) T vsm[3][BN * VS];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  lds_poison(ksm, sizeof(ksm), tid, NT);
  lds_poison(vsm, sizeof(vsm), tid, NT);

  int head, rank;
  tile_order(blockIdx.x, p.n_heads, p.n_qtiles, p.remap_xcd, p.order_group, head, rank);
  const int qt = p.n_qtiles - 1 - rank;      // the last query tiles see the most keys under a causal mask
  const int b = head / p.Hq, hq = head - b * p.Hq;
  const int hk = hq / p.group;

  int sq = p.Sq, sk = p.Sk, qbase = 0, kbase = 0;
  if (p.cu_seqlens_q) {
    qbase = p.cu_seqlens_q[b];
    sq = p.cu_seqlens_q[b + 1] - qbase;
    kbase = p.cu_seqlens_k[b];
    sk = p.cu_seqlens_k[b + 1] - kbase;
  }
  const int m0 = qt * BM;
  if (m0 >= sq) return;

  const int64_t bq = p.cu_seqlens_q ? 0 : (int64_t)b;
  const T* qp = (const T*)p.q + bq * p.q_sb + (int64_t)qbase * p.q_ss + (int64_t)hq * p.q_sh;
  const T* kp = (const T*)p.k + bq * p.k_sb + (int64_t)kbase * p.k_ss + (int64_t)hk * p.k_sh;
  const T* vp = (const T*)p.v + bq * p.v_sb + (int64_t)kbase * p.v_ss + (int64_t)hk * p.v_sh;
  T* op = (T*)p.out + bq * p.o_sb + (int64_t)qbase * p.o_ss + (int64_t)hq * p.o_sh;
  float* lp = p.lse + bq * p.lse_sb + (int64_t)hq * p.lse_sh + qbase;

  const int shift = sk - sq;
  const int ip_first = m0 + shift, ip_last = min(m0 + BM, sq) - 1 + shift;
  int kv_lo = 0, kv_hi = sk;
  if (p.wl >= 0) kv_lo = max(0, ip_first - p.wl);
  if (p.causal) kv_hi = min(kv_hi, ip_last + 1);
  if (p.wr >= 0) kv_hi = min(kv_hi, ip_last + p.wr + 1);
  const int t_lo = kv_lo / BN;
  const int n_t = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN - t_lo : 0;

  const int w0 = m0 + wave * 32;
  const int qrow = w0 + l32;
  const bool row_ok = qrow < sq;
  const int ip = qrow + shift;
  int j_lo = 0, j_hi = sk - 1;
  if (p.wl >= 0) j_lo = max(j_lo, ip - p.wl);
  if (p.causal) j_hi = min(j_hi, ip);
  if (p.wr >= 0) j_hi = min(j_hi, ip + p.wr);
  const int w1 = min(w0 + 32, sq) - 1;
  int lo_max = 0, hi_min = sk - 1;
  if (p.wl >= 0) lo_max = max(0, w1 + shift - p.wl);
  if (p.causal) hi_min = min(hi_min, w0 + shift);
  if (p.wr >= 0) hi_min = min(hi_min, w0 + shift + p.wr);
  // the wave's key range: [j_lo of its first row, j_hi of its last]
  int j_lo_min = 0, j_hi_max = sk - 1;
  if (p.wl >= 0) j_lo_min = max(0, w0 + shift - p.wl);
  if (p.causal) j_hi_max = min(j_hi_max, w1 + shift);
  if (p.wr >= 0) j_hi_max = min(j_hi_max, w1 + shift + p.wr);

  V8 qr[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    if (row_ok) qr[dc] = *(const V8*)(qp + (int64_t)qrow * p.q_ss + dc * 16 + hi * 8);
    else qr[dc] = V8{};
  }
  float slope_l2 = 0.f;
  if constexpr (ALIBI) slope_l2 = p.alibi[hq] * kLog2e;
  const float ipf = (float)ip;
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_in = 2.f * p.scale * kLog2e / (SOFTCAP ? p.softcap : 1.f);
  const float mult = PLAIN ? sl2 : 1.f;

  u32x4 kst[LOADS], vst[LOADS];
  auto gload = [&](int i) {
    const int j0 = (t_lo + i) * BN;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int cid = tid + u * NT, r = cid / CH, c = cid - r * CH;
      const int j = min(j0 + r, sk - 1);
      kst[u] = *(const u32x4*)(kp + (int64_t)j * p.k_ss + c * 8);
      vst[u] = *(const u32x4*)(vp + (int64_t)j * p.v_ss + c * 8);
    }
  };
  auto swrite = [&](int st) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int cid = tid + u * NT, r = cid / CH, c = cid - r * CH;
      *(u32x4*)(&ksm[st][r * KS + c * 8]) = kst[u];
      *(u32x4*)(&vsm[st][r * VS + c * 8]) = vst[u];
    }
  };
  // LDS writes of this wave complete, then all 8 waves meet
  auto barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  // running row max m (log2 units), sum l of the rounded P that feeds P V (it
  // normalises out; not kept by the lean phase, which normalises by lx) and sum
  // lx of the fp32 P (it gives lse)
  float m = kNegInf, l = 0.f, lx = 0.f;
  f32x16 s[KB];
  V2 pk[KB][8];

  if (n_t > 0) { gload(0); swrite(0); }
  if (n_t > 1) { gload(1); swrite(1); }
  wait_vmem_all();   // Q operands ready: the loop waits only for its own tile loads
  if (n_t > 2) gload(2);
  barrier();
  if (grp == 1) barrier();                 // group 1 runs one phase behind

  int st_q = 0;                            // stage of tile j (K read by this GEMM phase)
  // not unrolled: copies of the loop body for the three stages would not fit
  // the register budget (the plain and ALiBi-only variants then spill)
#pragma nounroll
  for (int j = 0; j <= n_t; ++j) {
    const int st_p = st_q == 0 ? 2 : st_q - 1;      // stage of tile j-1 (V read by P V)
    const int st_w = st_q == 2 ? 0 : st_q + 1;      // stage of tile j+1 (written now)
    // ---------------- GEMM phase j
    __builtin_amdgcn_s_setprio(1);
    if (j >= 1 && j + 1 < n_t) swrite(st_w);
    if (j >= 1 && j + 2 < n_t) gload(j + 2);
    {
    if (j < n_t) {
      const T* kb_ = ksm[st_q] + l32 * KS + hi * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        if (D > 64 && (dc & 1) == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const V8 a = *(const V8*)(kb_ + kb * 32 * KS + dc * 16);
          s[kb] = E::mfma32(a, qr[dc], s[kb]);
        }
      }
    }
    if (j >= 1) {
      const T* vb_ = vsm[st_p] + (hi * 4 + ((lane & 15) >> 2)) * VS + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
        // keep the operand reads of one 16-key chunk in flight at a time (bounds registers)
        if (D > 64) __builtin_amdgcn_sched_barrier(0);
        const int kb = c >> 1, c2 = c & 1;
        V8 bop;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bop[2 * e] = pk[kb][4 * c2 + e][0];
          bop[2 * e + 1] = pk[kb][4 * c2 + e][1];
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 x0 = lds_read_tr16(vb_ + c * 16 * VS + db * 32);
          const i16x4 x1 = lds_read_tr16(vb_ + (c * 16 + 8) * VS + db * 32);
          const V8 a = __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = E::mfma32(a, bop, o[db]);
        }
      }
    }
    }
    __builtin_amdgcn_s_setprio(0);
    barrier();
    if (j == n_t) break;
    // ---------------- softmax phase j
    const int j0 = (t_lo + j) * BN;
    const bool edge = !(j0 >= lo_max && j0 + BN - 1 <= hi_min);
    if constexpr (!PLAIN) {
      const float dj0 = (float)(j0 + 4 * hi) - ipf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r];
          if constexpr (SOFTCAP) {
            const float e = exp2_fast(x * cap_in);
            x = fmaf(-2.f * cap_l2, __builtin_amdgcn_rcpf(e + 1.f), cap_l2);
          } else {
            x *= sl2;
          }
          if constexpr (ALIBI) {
            const float dist = dj0 + (float)(kb * 32 + (r >> 2) * 8 + (r & 3));
            x = fmaf(-slope_l2, fabsf(dist), x);
          }
          s[kb][r] = x;
        }
    }
    if (edge) {
      // one unsigned compare per score, as in prefill_kernel
      const int base = j0 + 4 * hi - j_lo;
      const uint32_t cnt = (uint32_t)max(j_hi - j_lo + 1, 0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t x = (uint32_t)(base + kb * 32 + (r >> 2) * 8 + (r & 3));
          if (x >= cnt) s[kb][r] = kNegInf;
        }
    }
    if constexpr (LEAN) {
      // P against the running max m without a max reduction, kept when no
      // lane's sum of the tile's P exceeds 2^kTau; otherwise (a row without a
      // max yet, or scores well above m) m moves to the exact new max, O and lx
      // are rescaled and P is formed again from the scores still in registers.
      float lxs = 0.f;
      bool redo = __any(m == kNegInf);
      if (!redo) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = exp2_fast(fmaf(s[kb][r], mult, -m));
            const float p1 = exp2_fast(fmaf(s[kb][r + 1], mult, -m));
            pk[kb][r >> 1] = E::pack(p0, p1);
            lxs += p0 + p1;
          }
        redo = __any(lxs > kTauPow);
      }
      if (redo) {
        float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            mx0 = fmaxf(fmaxf(mx0, s[kb][r]), s[kb][r + 1]);
            mx1 = fmaxf(fmaxf(mx1, s[kb][r + 2]), s[kb][r + 3]);
          }
        const float m_new = fmaxf(m, max_halves(fmaxf(mx0, mx1)) * mult);
        if (__any(m_new > m)) {
          const float alpha = m_new == kNegInf ? 1.f : exp2_fast(m - m_new);
          m = m_new;
          lx *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= alpha;
        }
        const float m_use = m == kNegInf ? 0.f : m;
        lxs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = exp2_fast(fmaf(s[kb][r], mult, -m_use));
            const float p1 = exp2_fast(fmaf(s[kb][r + 1], mult, -m_use));
            pk[kb][r >> 1] = E::pack(p0, p1);
            lxs += p0 + p1;
          }
      }
      lx += lxs;
      barrier();
      st_q = st_w;
      continue;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
    mx = max_halves(mx) * mult;
    const float m_new = fmaxf(m, mx);
    if (__any(m_new > m + kTau)) {
      const float alpha = m_new == kNegInf ? 1.f : exp2_fast(m - m_new);
      m = m_new;
      l *= alpha;
      lx *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    const float m_use = m == kNegInf ? 0.f : m;
    float ls = 0.f, lxs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_fast(fmaf(s[kb][r], mult, -m_use));
        const float p1 = exp2_fast(fmaf(s[kb][r + 1], mult, -m_use));
        pk[kb][r >> 1] = E::pack(p0, p1);
        ls = E::sum2(pk[kb][r >> 1], ls);
        lxs += p0 + p1;
      }
    l += ls;
    lx += lxs;
    barrier();
    st_q = st_w;
  }
  if (grp == 0) barrier();                 // matches group 1's initial offset

  // out = O / norm (l; lx in the lean phase and after the precise pass, whose O is the product with
  // P itself), lse = (m + log2 lx) * ln 2
  auto write_row = [&](float norm) __attribute__((always_inline)) {
    const float lt = sum_halves(norm);
    const float lxt = sum_halves(lx);
    if (row_ok) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      T* orow = op + (int64_t)qrow * p.o_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          V2 a = E::pack(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv);
          V2 c = E::pack(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv);
          u32x2 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c)};
          *(u32x2*)(orow + db * 32 + gq * 8 + hi * 4) = w;
        }
      if (hi == 0) lp[qrow] = lxt > 0.f ? (m + __log2f(lxt)) * kLn2 : kNegInf;
    }
  };

  // The precise pass of prefill_kernel, here as a plain loop over one LDS stage:
  // waves with an output element of magnitude precise_out_pp<E>() or more recompute
  // their row with P split into RN(P) and RN(P - RN(P)) against the final m.
  bool need = false;
  {
    const float lt = sum_halves(l);
    float om = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) om = fmaxf(om, fabsf(o[db][r]));
    const float lnorm = LEAN ? sum_halves(lx) : lt;
    need = row_ok && lnorm > 0.f && om / lnorm >= (LEAN ? kPreciseOut : precise_out_pp<E>());
  }
  const bool wave_need = __any(need);
  if (!wave_need) write_row(LEAN ? lx : l);
  if (__syncthreads_or(wave_need)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    lx = 0.f;
    const float mu = m == kNegInf ? 0.f : m;
    const T* kb_ = ksm[0] + l32 * KS + hi * 8;
    const T* vb_ = vsm[0] + (hi * 4 + ((lane & 15) >> 2)) * VS + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    for (int i = 0; i < n_t; ++i) {
      gload(i);
      barrier();                             // every wave is done with the previous tile
      swrite(0);
      barrier();                             // the tile is in LDS
      if (!wave_need) continue;
      const int j0 = (t_lo + i) * BN;
      if (j0 + BN - 1 < j_lo_min || j0 > j_hi_max) continue;   // no row of the wave sees the tile
      f32x16 sp[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sp[kb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sp[kb] = E::mfma32(*(const V8*)(kb_ + kb * 32 * KS + dc * 16), qr[dc], sp[kb]);
      const float dj0 = (float)(j0 + 4 * hi) - ipf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sp[kb][r];
          if constexpr (SOFTCAP) {
            const float e = exp2_fast(x * cap_in);
            x = fmaf(-2.f * cap_l2, __builtin_amdgcn_rcpf(e + 1.f), cap_l2);
          } else if constexpr (ALIBI) {
            x *= sl2;
          }
          if constexpr (ALIBI) x = fmaf(-slope_l2, fabsf(dj0 + (float)(kb * 32 + (r >> 2) * 8 + (r & 3))), x);
          const int jj = j0 + 4 * hi + kb * 32 + (r >> 2) * 8 + (r & 3);
          sp[kb][r] = (jj < j_lo || jj > j_hi) ? kNegInf : x;
        }
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
        const int kb = c >> 1, c2 = c & 1;
        V8 bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = exp2_fast(fmaf(sp[kb][8 * c2 + e], mult, -mu));
          const T h = E::from_f32(pv);
          bh[e] = h;
          bl[e] = E::from_f32(pv - E::to_f32(h));
          lx += pv;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 x0 = lds_read_tr16(vb_ + c * 16 * VS + db * 32);
          const i16x4 x1 = lds_read_tr16(vb_ + (c * 16 + 8) * VS + db * 32);
          const V8 a = __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = E::mfma32(a, bh, o[db]);
          o[db] = E::mfma32(a, bl, o[db]);
        }
      }
    }
    if (wave_need) write_row(lx);
  }
}

// Tile shapes: 8 waves of one 32-row block each, i.e. 256 query rows per
// workgroup and 64-key tiles, for both head dims.  (RB = 2 blocks per wave
// shares every K/V operand read between two MFMAs but needs more than the
// 256-register budget of two waves per SIMD.)
template <int D> struct Shape { static constexpr int NW = 8, RB = 1, BN = 64; };
// D = 256: O alone takes 128 registers per lane, so one wave per SIMD (4 per
// workgroup) with up to 512 registers, and 32-key tiles to bound the staging
template <> struct Shape<256> { static constexpr int NW = 4, RB = 1, BN = 32; };
template <> struct Shape<64> { static constexpr int NW = FA_PREFILL_NW64, RB = FA_PREFILL_RB64, BN = 64; };
template <> struct Shape<128> { static constexpr int NW = FA_PREFILL_NW128, RB = FA_PREFILL_RB128, BN = 64; };

// Query rows per workgroup.  The main kernel with 8 waves of 32 rows takes 256;
// when B*Hq*ceil(Sq/256) workgroups would fill fewer than two per CU it drops
// to 4 waves (128 rows) or 2 waves (64 rows), so more CUs get work (each wave
// still owns 32 rows; the workgroups share K/V tiles among fewer waves).
template <int D> static int block_m_of(int64_t heads, int max_sq, int cus, int span) {
  using S = Shape<D>;
  if (D >= FA_PREFILL_PINGPONG_MIN_D && (D == 64 || D == 128)) return 8 * 32;
  if (S::NW != 8 || S::RB != 1) return S::NW * 32 * S::RB;
  auto wgs = [&](int bm) { return heads * ((max_sq + bm - 1) / bm); };
  // D = 64 under a narrow window (a row sees at most 512 keys besides its own):
  // a 256-row workgroup walks 256 + span keys of which each wave needs 32 +
  // span, so 128-row workgroups (3 per CU, 3 waves per SIMD) waste fewer
  // barrier steps: B=4, S=4096, H=32 window (256,0) 336 -> 366 TFLOP/s,
  // (256,256) 530 -> 540
  if (D == 64 && span >= 0 && span <= 512 && wgs(128) >= (int64_t)cus) return 128;
  // D = 96: 4-wave workgroups measured faster even on full grids (656 against
  // 615 TFLOP/s at B=4, S=4096, H=32 causal), 8 waves splitting its 12-piece
  // rows less evenly
  if (D != 96 && wgs(256) >= 2 * (int64_t)cus) return 256;
  if (wgs(128) >= (int64_t)cus) return 128;
  return 64;
}

int prefill_block_m(int D, int64_t heads, int max_sq, int cus, int span) {
  switch (D) {
    case 32: return block_m_of<32>(heads, max_sq, cus, span);
    case 64: return block_m_of<64>(heads, max_sq, cus, span);
    case 96: return block_m_of<96>(heads, max_sq, cus, span);
    case 256: return block_m_of<256>(heads, max_sq, cus, span);
    default: return block_m_of<128>(heads, max_sq, cus, span);
  }
}

// One workgroup per (head, query tile) unit.
template <auto Kern>
static void launch_k(int threads, const PrefillParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.n_heads;
  hipLaunchKernelGGL(Kern, dim3(grid), dim3(threads), 0, s, p);
}

template <class E, int D, bool SC, bool AL>
static hipError_t launch_one(const PrefillParams& p, hipStream_t s) {
  using S = Shape<D>;
  if constexpr (D >= FA_PREFILL_PINGPONG_MIN_D && (D == 64 || D == 128)) {
    launch_k<prefill_pp_kernel<E, D, 64, SC, AL, FA_PP_LEAN && !SC && !AL>>(512, p, s);
  } else if constexpr (S::NW == 8 && S::RB == 1) {
    // fewer rows per workgroup when the grid would leave CUs idle (see prefill_block_m)
    if (p.block_m == 64)
      launch_k<prefill_kernel<E, D, S::BN, 2, 1, SC, AL>>(128, p, s);
    else if (p.block_m == 128)
      launch_k<prefill_kernel<E, D, S::BN, 4, 1, SC, AL>>(256, p, s);
    else
      launch_k<prefill_kernel<E, D, S::BN, 8, 1, SC, AL>>(512, p, s);
  } else {
    launch_k<prefill_kernel<E, D, S::BN, S::NW, S::RB, SC, AL>>(S::NW * 64, p, s);
  }
  return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_d(const PrefillParams& p, hipStream_t s) {
  const bool sc = p.softcap > 0.f, al = p.alibi != nullptr;
  if (sc && al) return launch_one<E, D, true, true>(p, s);
  if (sc) return launch_one<E, D, true, false>(p, s);
  if (al) return launch_one<E, D, false, true>(p, s);
  return launch_one<E, D, false, false>(p, s);
}

template <class E>
static hipError_t launch_e(int D, const PrefillParams& p, hipStream_t s) {
  switch (D) {
    case 32: return launch_d<E, 32>(p, s);
    case 64: return launch_d<E, 64>(p, s);
    case 96: return launch_d<E, 96>(p, s);
    case 256: return launch_d<E, 256>(p, s);
    default: return launch_d<E, 128>(p, s);
  }
}

// fp8 inputs: the main kernel (8 waves of 32 rows, 64-key tiles) for both head dims
int prefill_block_m_fp8(int) { return 8 * 32; }

template <int D, bool SC, bool AL>
static hipError_t launch_f8(const PrefillParams& p, hipStream_t s) {
  launch_k<prefill_kernel<BF16, D, 64, 8, 1, SC, AL, true>>(512, p, s);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f8d(const PrefillParams& p, hipStream_t s) {
  const bool sc = p.softcap > 0.f, al = p.alibi != nullptr;
  if (sc && al) return launch_f8<D, true, true>(p, s);
  if (sc) return launch_f8<D, true, false>(p, s);
  if (al) return launch_f8<D, false, true>(p, s);
  return launch_f8<D, false, false>(p, s);
}

hipError_t launch_prefill_fp8(int D, const PrefillParams& p, hipStream_t s) {
  return D == 64 ? launch_f8d<64>(p, s) : launch_f8d<128>(p, s);
}

hipError_t launch_prefill(Dtype dt, int D, const PrefillParams& p, hipStream_t s) {
  return dt == kF16 ? launch_e<F16>(D, p, s) : launch_e<BF16>(D, p, s);
}

}  // namespace fa
