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
//  * K and V tiles are double-buffered in LDS with XOR-swizzled 16-byte chunks;
//    the next tile's global loads are issued before the current tile's math.
//  * scale·log2(e) is folded into the exp2 argument (one FMA + v_exp_f32 per score).
//  * tiles that are fully masked for a wave are skipped; mask arithmetic runs only
//    on tiles that straddle a mask edge.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

typedef short i16x8 __attribute__((ext_vector_type(8)));

// 16-byte chunk c of tile row r is stored at chunk kswz / vswz (bank-conflict
// free for the K row reads and the transposing V reads respectively).
template <int D>
__device__ __forceinline__ int kswz(int r, int c) {
  return D == 64 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15));
}
template <int D>
__device__ __forceinline__ int vswz(int r, int c) {
  return D == 64 ? (c ^ (((r >> 1) & 1) << 2)) : (c ^ ((r & 3) << 2));
}

template <class E, int D, int BN, int NW, bool SOFTCAP, bool ALIBI>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillParams p) {
  using T = typename E::T;
  using V8 = typename E::V8;
  using V2 = typename E::V2;
  constexpr int BM = NW * 32;
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int KB = BN / 32;             // 32-key blocks per tile
  constexpr int DC = D / 16;              // contraction steps of Q K^T
  constexpr int DB = D / 32;              // 32-wide blocks of the output
  constexpr int NT = NW * 64;
  constexpr int LOADS = BN * CH / NT;     // 16-byte loads per thread per tile, for K and for V
  static_assert(LOADS * NT == BN * CH, "tile must split evenly over the workgroup");
  constexpr bool PLAIN = !SOFTCAP && !ALIBI;

  __shared__ __attribute__((aligned(16))) T smem[2][2][BN * D];   // [buffer][K, V][row * D]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;

  // ---- workgroup -> (batch, query head, query tile); heads are spread over the
  // 8 XCDs in contiguous ranges so the workgroups sharing K/V share an L2, and
  // within a head the longest (last) query tiles go first.
  int id = blockIdx.x;
  if (p.remap_xcd) id = (id & 7) * (int)(gridDim.x >> 3) + (id >> 3);
  const int head = id / p.n_qtiles;
  const int qt = p.n_qtiles - 1 - (id - head * p.n_qtiles);
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

  // ---- key range of the workgroup (bottom-right alignment: row i sits at i + sk - sq)
  const int shift = sk - sq;
  const int ip_first = m0 + shift, ip_last = min(m0 + BM, sq) - 1 + shift;
  int kv_lo = 0, kv_hi = sk;
  if (p.wl >= 0) kv_lo = max(0, ip_first - p.wl);
  if (p.causal) kv_hi = min(kv_hi, ip_last + 1);
  if (p.wr >= 0) kv_hi = min(kv_hi, ip_last + p.wr + 1);
  const int t_lo = kv_lo / BN;
  const int t_hi = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : t_lo;

  // ---- this lane's query row and its allowed key interval [j_lo, j_hi]
  const int qrow = m0 + wave * 32 + l32;
  const bool row_ok = qrow < sq;
  const int ip = qrow + shift;
  int j_lo = 0, j_hi = sk - 1;
  if (p.wl >= 0) j_lo = max(j_lo, ip - p.wl);
  if (p.causal) j_hi = min(j_hi, ip);
  if (p.wr >= 0) j_hi = min(j_hi, ip + p.wr);

  // the same bounds over the wave's rows, to classify tiles as empty / full / edge
  const int w0 = m0 + wave * 32, w1 = min(w0 + 32, sq) - 1;
  const bool wave_live = w0 < sq;
  int lo_min = 0, lo_max = 0, hi_min = sk - 1, hi_max = sk - 1;
  if (p.wl >= 0) { lo_min = max(0, w0 + shift - p.wl); lo_max = max(0, w1 + shift - p.wl); }
  if (p.causal) { hi_min = min(hi_min, w0 + shift); hi_max = min(hi_max, w1 + shift); }
  if (p.wr >= 0) { hi_min = min(hi_min, w0 + shift + p.wr); hi_max = min(hi_max, w1 + shift + p.wr); }

  // ---- Q operand (B of S^T = K Q^T): lane holds row qrow, d = 16*dc + 8*hi .. +7
  V8 qr[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    if (row_ok) qr[dc] = *(const V8*)(qp + (int64_t)qrow * p.q_ss + dc * 16 + hi * 8);
    else qr[dc] = V8{};
  }

  float slope_l2 = 0.f, ipf = 0.f;
  if constexpr (ALIBI) { slope_l2 = p.alibi[hq] * kLog2e; ipf = (float)ip; }
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;                 // softcap in log2 units
  const float cap_in = 2.f * p.scale * kLog2e / (SOFTCAP ? p.softcap : 1.f);

  // ---- global -> register staging of one K/V tile (rows past sk are clamped to a
  // real row; their scores are masked, so their values only ever meet p = 0)
  u32x4 kst[LOADS], vst[LOADS];
  auto gload = [&](int tile) {
    const int j0 = tile * BN;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
      const int j = min(j0 + r, sk - 1);
      kst[i] = *(const u32x4*)(kp + (int64_t)j * p.k_ss + c * 8);
      vst[i] = *(const u32x4*)(vp + (int64_t)j * p.v_ss + c * 8);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int cid = tid + i * NT, r = cid / CH, c = cid - r * CH;
      *(u32x4*)(&smem[buf][0][r * D + kswz<D>(r, c) * 8]) = kst[i];
      *(u32x4*)(&smem[buf][1][r * D + vswz<D>(r, c) * 8]) = vst[i];
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegInf;     // running row max, log2 units
  // running row sums over this lane's keys (the other half is added at the end):
  // l of the rounded P that feeds the P V product (normalises out, so out is an
  // exact convex combination of the rounded weights), lx of the unrounded fp32 P
  // (gives an lse free of the P rounding)
  float l = 0.f, lx = 0.f;

  if (t_lo < t_hi) {
    gload(t_lo);
    swrite(0);
  }
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    if (t + 1 < t_hi) gload(t + 1);
    const int j0 = t * BN;
    const bool empty = !wave_live || lo_min > hi_max || j0 + BN - 1 < lo_min || j0 > hi_max;
    if (!empty) {
      const bool full = j0 >= lo_max && j0 + BN - 1 <= hi_min;
      const T* Ks = smem[buf][0];
      const T* Vs = smem[buf][1];

      // S^T = K Q^T : s[kb][r] is key j0 + 32kb + 8(r/4) + 4hi + (r%4) of row qrow
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x16{};
        const int r = kb * 32 + l32;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const V8 a = *(const V8*)(Ks + r * D + kswz<D>(r, dc * 2 + hi) * 8);
          s[kb] = E::mfma32(a, qr[dc], s[kb]);
        }
      }

      // score transforms into log2 units (the plain path folds the scale into exp2)
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
      if (!full) {
        const int jb = j0 + 4 * hi;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = jb + kb * 32 + (r >> 2) * 8 + (r & 3);
            if (j < j_lo || j > j_hi) s[kb][r] = kNegInf;
          }
      }

      // online softmax
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_halves(mx);
      const float mult = PLAIN ? sl2 : 1.f;
      const float m_new = fmaxf(m, mx * mult);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      V2 pk[KB][8];
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
      l = fmaf(l, alpha, ls);
      lx = fmaf(lx, alpha, lxs);
      m = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;

      // O^T += V^T P^T over 16-key chunks
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
        const int kb = c >> 1, c2 = c & 1;
        V8 bop;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bop[2 * e] = pk[kb][4 * c2 + e][0];
          bop[2 * e + 1] = pk[kb][4 * c2 + e][1];
        }
        const int g = lane & 15;
        const int row = c * 16 + hi * 4 + (g >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + ((lane >> 4) & 1) * 16 + (g & 3) * 4;
          const int cc = col >> 3, co = col & 7;
          const i16x4 x0 = lds_read_tr16(Vs + row * D + vswz<D>(row, cc) * 8 + co);
          const i16x4 x1 = lds_read_tr16(Vs + (row + 8) * D + vswz<D>(row + 8, cc) * 8 + co);
          const i16x8 xa = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = E::mfma32(__builtin_bit_cast(V8, xa), bop, o[db]);
        }
      }
    }
    if (t + 1 < t_hi) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: out = O / l, lse = ln(sum exp(scores)) = (m + log2 lx) * ln 2
  const float lt = sum_halves(l);
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
}

template <class E, int D, bool SC, bool AL>
static hipError_t launch_one(const PrefillParams& p, hipStream_t s) {
  constexpr int NW = 4, BN = 64;
  static_assert(NW * 32 == kPrefillBlockM, "");
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.Hq * (unsigned)p.B;
  hipLaunchKernelGGL((prefill_kernel<E, D, BN, NW, SC, AL>), dim3(grid), dim3(NW * 64), 0, s, p);
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

hipError_t launch_prefill(Dtype dt, int D, const PrefillParams& p, hipStream_t s) {
  if (dt == kF16) return D == 64 ? launch_d<F16, 64>(p, s) : launch_d<F16, 128>(p, s);
  return D == 64 ? launch_d<BF16, 64>(p, s) : launch_d<BF16, 128>(p, s);
}

}  // namespace fa
