// Split-KV decode kernel for gfx950: new queries against a (paged) KV cache.
//
// Flash-decoding, as the Flash-Attention v2.0-v2.7 update notes describe it
// (v2.2): instead of one workgroup walking the whole cache, the cache is cut
// along the sequence into num_splits contiguous chunks, each chunk is attended
// by its own workgroup, and a separate reduction kernel merges the chunks by
// their log-sum-exp (combine.hip).  The cache may be paged (v2.5): token t of
// sequence b lives in page block_table[b, t / page_size], row t % page_size.
//
// Decode reads every K/V byte once and does ~4 FLOP per byte, so the kernel is
// bound by HBM bandwidth.  Layout choices:
//  * grid = (split, kv head, batch); the workgroup owns every query row of its
//    GQA group (G = Hq/Hkv heads x Sq positions), so each K/V row is read once
//    and used for all G*Sq rows;
//  * D/8 lanes per token, 16 bytes per lane per K or V row: one coalesced
//    dwordx4 load per lane, 2-4 tokens in flight per lane;
//  * each token slot (lane group) keeps its own running max / sum / partial
//    output, so the hot loop has no cross-slot reduction; slots are merged once
//    at the end (cross-lane, then through LDS);
//  * the split's partial output and lse go to the fp32 workspace.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

#ifndef FA_DECODE_U
#define FA_DECODE_U 4
#endif
constexpr int kPageWindow = 1024;   // block-table entries staged in LDS per segment
constexpr float kTauD = 8.f;        // lazy-rescale threshold (log2 units)
#ifndef FA_DECODE_MFMA
#define FA_DECODE_MFMA 1
#endif

// bf16 / fp16 pair <-> fp32
template <class E>
__device__ __forceinline__ void unpack8(const u32x4& w, float (&x)[8]);
template <>
__device__ __forceinline__ void unpack8<BF16>(const u32x4& w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack8<F16>(const u32x4& w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // copy the element out first: a bit_cast applied to a vector element
    // expression directly read element 0 regardless of i
    const uint32_t wi = w[i];
    const f16x2 h = __builtin_bit_cast(f16x2, wi);
    x[2 * i] = (float)h[0];
    x[2 * i + 1] = (float)h[1];
  }
}

// sum over groups of G lanes (G = 8 or 16), every lane of the group gets the total
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)); // 7 - i in 8
  if constexpr (G == 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)); // 15 - i
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) {
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, x)));
}

template <class E, int D, int R>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  using T = typename E::T;
  constexpr int LPT = D / 8;            // lanes per token
  constexpr int TPW = 64 / LPT;         // token slots per wave
  constexpr int NW = 4;
  constexpr int SLOTS = TPW * NW;       // token slots per workgroup
  constexpr int U = R <= 4 ? FA_DECODE_U : (R == 8 ? 2 : 1);   // tokens per slot per iteration
  constexpr int STEP = SLOTS * U;

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slot = wave * TPW + lane / LPT, dc = lane % LPT;

  const int len = p.cache_seqlens[b];
  const int chunk = (len + p.num_splits - 1) / p.num_splits;
  const int t0 = min(len, split * chunk), t1 = min(len, t0 + chunk);
  const int rows = p.group * p.Sq;      // live query rows (<= R)

  // query rows: r = sqi * G + g  ->  head hk*G + g, position sqi
  float q[R][8];
  int jlo[R], jhi[R];
  float slope[R], ipf[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int sqi = r / p.group, g = r - sqi * p.group;
    const bool live = r < rows;
    const int hq = hk * p.group + g;
    if (live) {
      const u32x4 w = *(const u32x4*)((const T*)p.q + (((int64_t)b * p.Sq + sqi) * p.Hq + hq) * D + dc * 8);
      unpack8<E>(w, q[r]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[r][i] = 0.f;
    }
    const int ip = sqi + len - p.Sq;    // bottom-right aligned position
    int lo = 0, hi = len - 1;
    if (p.wl >= 0) lo = max(lo, ip - p.wl);
    if (p.causal) hi = min(hi, ip);
    if (p.wr >= 0) hi = min(hi, ip + p.wr);
    jlo[r] = lo;
    jhi[r] = live ? hi : -1;
    slope[r] = (p.alibi && live) ? p.alibi[hq] * kLog2e : 0.f;
    ipf[r] = (float)ip;
  }
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_in = p.softcap > 0.f ? 2.f * p.scale * kLog2e / p.softcap : 0.f;

  const int64_t row_elems = (int64_t)p.Hkv * D;
  const T* kbase = (const T*)p.k + (int64_t)hk * D + dc * 8;
  const T* vbase = (const T*)p.v + (int64_t)hk * D + dc * 8;
  const int* bt = p.block_table ? p.block_table + (int64_t)b * p.bt_stride : nullptr;

  float m[R], l[R], o[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[r][i] = 0.f;
  }

  // The split's page numbers are staged in LDS (kPageWindow at a time), so the
  // per-token page lookup is an LDS read: a block-table load in the global
  // queue would make every wait for it also wait for the K/V loads in flight.
  __shared__ int s_pages[kPageWindow];
  const int page = p.page_size;
  const int pg_first = bt ? t0 / page : 0;
  const int pg_last = bt ? (t1 > t0 ? (t1 - 1) / page : pg_first - 1) : 0;

  u32x4 kr[U], vr[U];
  for (int seg = pg_first; t0 < t1 && seg <= pg_last; seg += kPageWindow) {
    int ts = t0, te = t1;
    if (bt) {
      const int n = min(kPageWindow, pg_last + 1 - seg);
      __syncthreads();                                   // previous segment's lookups are done
      for (int i = tid; i < n; i += NW * 64) s_pages[i] = bt[seg + i];
      __syncthreads();
      ts = max(t0, seg * page);
      te = min(t1, (seg + n) * page);
    }
    auto token_row = [&](int t) -> int64_t {    // cache row index of token t
      if (!bt) return (int64_t)b * page + t;
      const int pg = p.log2_page >= 0 ? (t >> p.log2_page) : t / page;
      const int in = t - pg * page;
      return (int64_t)s_pages[pg - seg] * page + in;
    };
    auto issue = [&](int base) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = min(base + u * SLOTS + slot, te - 1);    // clamp: a real token, masked below
        const int64_t row = token_row(t);
        kr[u] = __builtin_nontemporal_load((const u32x4*)(kbase + row * row_elems));
        vr[u] = __builtin_nontemporal_load((const u32x4*)(vbase + row * row_elems));
      }
    };

    issue(ts);
    for (int base = ts; base < te; base += STEP) {
      u32x4 kc[U], vc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) { kc[u] = kr[u]; vc[u] = vr[u]; }
      if (base + STEP < te) issue(base + STEP);

      float s[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kx[8];
        unpack8<E>(kc[u], kx);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc = fmaf(q[r][i], kx[i], acc);
          s[u][r] = group_sum<LPT>(acc);
        }
      }
      // transforms (log2 units) and masks
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = base + u * SLOTS + slot;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float x = s[u][r];
          if (p.softcap > 0.f) {
            const float e = exp2_fast(x * cap_in);
            x = fmaf(-2.f * cap_l2, __builtin_amdgcn_rcpf(e + 1.f), cap_l2);
          } else {
            x *= sl2;
          }
          x = fmaf(-slope[r], fabsf(ipf[r] - (float)t), x);
          if (t >= te || t < jlo[r] || t > jhi[r]) x = kNegInf;
          s[u][r] = x;
        }
      }
      float vx[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) unpack8<E>(vc[u], vx[u]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float mx = s[0][r];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][r]);
        const float m_new = fmaxf(m[r], mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = exp2_fast(m[r] - m_use);
        float ps[U];
        float lsum = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) { ps[u] = exp2_fast(s[u][r] - m_use); lsum += ps[u]; }
        l[r] = fmaf(l[r], alpha, lsum);
        m[r] = m_new;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float acc = o[r][i] * alpha;
#pragma unroll
          for (int u = 0; u < U; ++u) acc = fmaf(ps[u], vx[u][i], acc);
          o[r][i] = acc;
        }
      }
    }
    if (!bt) break;
  }

  // ---- merge the token slots of each wave (lane groups at distance LPT, 2*LPT, ...)
#pragma unroll
  for (int dist = LPT; dist < 64; dist *= 2) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float mo = shfl_xor_f(m[r], dist);
      const float lo_ = shfl_xor_f(l[r], dist);
      const float m_new = fmaxf(m[r], mo);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float a = exp2_fast(m[r] - m_use), ao = exp2_fast(mo - m_use);
      l[r] = l[r] * a + lo_ * ao;
      m[r] = m_new;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float oo = shfl_xor_f(o[r][i], dist);
        o[r][i] = o[r][i] * a + oo * ao;
      }
    }
  }

  // ---- merge the waves through LDS
  __shared__ float s_o[NW][R][D];
  __shared__ float s_ml[NW][R][2];
  if (lane < LPT) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_o[wave][r][dc * 8 + i] = o[r][i];
      if (dc == 0) { s_ml[wave][r][0] = m[r]; s_ml[wave][r][1] = l[r]; }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < rows * D; idx += NW * 64) {
    const int r = idx / D, d = idx - r * D;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_ml[w][r][0]);
    const float m_use = mm == kNegInf ? 0.f : mm;
    float lt = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = exp2_fast(s_ml[w][r][0] - m_use);
      lt += s_ml[w][r][1] * a;
      acc += s_o[w][r][d] * a;
    }
    const int sqi = r / p.group, g = r - sqi * p.group;
    const int64_t prow = (((int64_t)b * p.Sq + sqi) * p.Hq + hk * p.group + g) * p.num_splits + split;
    p.out_partial[prow * D + d] = lt > 0.f ? acc / lt : 0.f;
    if (d == 0) p.lse_partial[prow] = lt > 0.f ? (mm + __log2f(lt)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// MFMA decode.  One wave per (split, kv head, batch).  The query rows of the
// GQA group (G heads x Sq positions, at most 16) sit on the N side of
// v_mfma_f32_16x16x32, so both contractions run on the matrix cores:
//   S^T = K Q^T : the A operand (lane = token % 16, 8 consecutive d) is read
//                 from the K tile in LDS, Q^T is a register-resident B operand;
//   O^T += V^T P^T : P stays in registers as the B operand (its contraction
//                 index is a fixed permutation of the chunk's tokens, applied
//                 identically to V), V^T comes from LDS through the
//                 transposing read ds_read_b64_tr_b16.
// Lane l holds query row l % 16; the four lanes sharing a row exchange their
// chunk maxima with two shuffles, so P of a chunk shares one reference max.
// Tokens are processed in chunks of 32 whose K and V rows are read as whole
// 256-byte rows (16 lanes per row, full cache lines) into registers and then
// stored to LDS, from where the MFMA operands are read; two chunks are in
// flight while one is computed.
// ---------------------------------------------------------------------------
constexpr int kDecodeChunk = 32;
constexpr int kPageWindowM = 256;

// MODE: 0 = dense cache, 1 = paged with a power-of-two page size, 2 = other page sizes
template <class E, int D, int MODE>
__global__ __launch_bounds__(64) void decode_mfma_kernel(DecodeParams p) {
  using T = typename E::T;
  using V8 = typename E::V8;
  using V2 = typename E::V2;
  constexpr int KSTEP = D / 32;           // MFMA K-steps of Q K^T
  constexpr int DBK = D / 16;             // 16-wide d blocks of O^T
  constexpr int VROW = D + 16;            // V LDS row stride (elements): 2D + 32 bytes, conflict-free tr reads
  constexpr int KROW = D + 8;             // K LDS row stride: 2D + 16 bytes, conflict-free 16-byte reads
  constexpr int CH = D / 8;               // 16-byte chunks per K/V row
  constexpr int VLD = kDecodeChunk * CH / 64;   // 16-byte loads per lane per chunk, for K and for V
  static_assert(VLD * 64 == kDecodeChunk * CH, "");
  __shared__ __attribute__((aligned(16))) T vbuf[2][kDecodeChunk * VROW];
  __shared__ __attribute__((aligned(16))) T kbuf[2][kDecodeChunk * KROW];
  __shared__ int s_pages[kPageWindowM];

  const int lane = threadIdx.x, n = lane & 15, q4 = lane >> 4;
  // kv head fastest: the workgroups reading the Hkv slices of the same token rows
  // run at the same time, which keeps those DRAM rows open
  const int hk = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
  const int len = p.cache_seqlens[b];
  const int chunk = (len + p.num_splits - 1) / p.num_splits;
  const int t0 = min(len, split * chunk), t1 = min(len, t0 + chunk);
  const int rows = p.group * p.Sq;

  // ---- query row n of the group: position sqi, head hk*G + g
  const int sqi = n / p.group, gq = n - sqi * p.group;
  const bool live = n < rows;
  const int hq = hk * p.group + gq;
  V8 qb[KSTEP];
#pragma unroll
  for (int ks = 0; ks < KSTEP; ++ks) {
    if (live) qb[ks] = *(const V8*)((const T*)p.q + (((int64_t)b * p.Sq + sqi) * p.Hq + hq) * D + ks * 32 + q4 * 8);
    else qb[ks] = V8{};
  }
  const int ip = sqi + len - p.Sq;        // bottom-right aligned position of the row
  int jlo = 0, jhi = len - 1;
  if (p.wl >= 0) jlo = max(jlo, ip - p.wl);
  if (p.causal) jhi = min(jhi, ip);
  if (p.wr >= 0) jhi = min(jhi, ip + p.wr);
  if (!live) jhi = -1;
  const float slope = (p.alibi && live) ? p.alibi[hq] * kLog2e : 0.f;
  const float ipf = (float)ip;
  const float sl2 = p.scale * kLog2e;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_in = p.softcap > 0.f ? 2.f * p.scale * kLog2e / p.softcap : 0.f;

  const int64_t row_elems = (int64_t)p.Hkv * D;
  const T* kh = (const T*)p.k + (int64_t)hk * D;
  const T* vh = (const T*)p.v + (int64_t)hk * D;
  const int* bt = MODE ? p.block_table + (int64_t)b * p.bt_stride : nullptr;
  const int page = p.page_size;

  f32x4 o[DBK];
#pragma unroll
  for (int db = 0; db < DBK; ++db) o[db] = f32x4{};
  float m = kNegInf, l = 0.f, lx = 0.f;

  const int pg_first = MODE ? t0 / page : 0;
  const int pg_last = MODE ? (t1 > t0 ? (t1 - 1) / page : pg_first - 1) : 0;
  for (int seg = pg_first; t0 < t1 && seg <= pg_last; seg += kPageWindowM) {
    int ts = t0, te = t1;
    if constexpr (MODE != 0) {
      const int np = min(kPageWindowM, pg_last + 1 - seg);
      __syncthreads();
      for (int i = lane; i < np; i += 64) s_pages[i] = bt[seg + i];
      __syncthreads();
      ts = max(t0, seg * page);
      te = min(t1, (seg + np) * page);
    }
    auto token_row = [&](int t) -> int64_t {
      if constexpr (MODE == 0) return (int64_t)b * page + t;
      const int pg = MODE == 1 ? (t >> p.log2_page) : t / page;
      return (int64_t)s_pages[pg - seg] * page + (t - pg * page);
    };
    // this lane's share of the chunk's K and V rows: whole 256-byte rows per 16
    // lanes (full cache lines), staged in LDS
    auto load = [&](int base, u32x4 (&kr)[VLD], u32x4 (&vr)[VLD]) {
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int slot = i * 64 + lane, r = slot / CH, c = slot - r * CH;
        const int64_t row = token_row(min(base + r, te - 1));
        kr[i] = *(const u32x4*)(kh + row * row_elems + c * 8);
        vr[i] = *(const u32x4*)(vh + row * row_elems + c * 8);
      }
    };
    auto store_kv = [&](int buf, const u32x4 (&kr)[VLD], const u32x4 (&vr)[VLD]) {
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int slot = i * 64 + lane, r = slot / CH, c = slot - r * CH;
        *(u32x4*)(&kbuf[buf][r * KROW + c * 8]) = kr[i];
        *(u32x4*)(&vbuf[buf][r * VROW + c * 8]) = vr[i];
      }
    };
    auto compute = [&](int base, int buf) {
      // S^T = K Q^T; A operand: lane holds K[token 16g + n][d = 32ks + 8q4 .. +7]
      f32x4 s[2];
      const T* kb_ = kbuf[buf] + n * KROW + q4 * 8;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        s[g] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks)
          s[g] = E::mfma16(*(const V8*)(kb_ + 16 * g * KROW + ks * 32), qb[ks], s[g]);
      }
      // scores of tokens base + 16g + 4q4 + r for row n, in log2 units
      float mx = kNegInf;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = base + 16 * g + 4 * q4 + r;
          float x = s[g][r];
          if (p.softcap > 0.f) {
            const float e = exp2_fast(x * cap_in);
            x = fmaf(-2.f * cap_l2, __builtin_amdgcn_rcpf(e + 1.f), cap_l2);
          } else {
            x *= sl2;
          }
          x = fmaf(-slope, fabsf(ipf - (float)t), x);
          if (t >= te || t < jlo || t > jhi) x = kNegInf;
          s[g][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      if (__any(m_new > m + kTauD)) {
        const float alpha = m_new == kNegInf ? 1.f : exp2_fast(m - m_new);
        m = m_new;
        l *= alpha;
        lx *= alpha;
#pragma unroll
        for (int db = 0; db < DBK; ++db) o[db] *= alpha;
      }
      const float m_use = m == kNegInf ? 0.f : m;
      V8 bop;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = exp2_fast(s[g][r] - m_use), p1 = exp2_fast(s[g][r + 1] - m_use);
          const V2 pp = E::pack(p0, p1);
          bop[4 * g + r] = pp[0];
          bop[4 * g + r + 1] = pp[1];
          l = E::sum2(pp, l);
          lx += p0 + p1;
        }
      // V^T operand rows: 16g + 4q4 + (n / 4), columns 16db + 4(n % 4)
      const T* vb = vbuf[buf] + (4 * q4 + (n >> 2)) * VROW + 4 * (n & 3);
#pragma unroll
      for (int db = 0; db < DBK; ++db) {
        const i16x4 x0 = lds_read_tr16(vb + db * 16);
        const i16x4 x1 = lds_read_tr16(vb + 16 * VROW + db * 16);
        const V8 a = __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = E::mfma16(a, bop, o[db]);
      }
    };

    // Two chunks in flight: chunk i+2 is requested right after chunk i is
    // consumed, before the wait for chunk i+1, so every load has about two
    // chunk periods to arrive.  Register sets A/B and LDS buffers 0/1 alternate.
    u32x4 ka[VLD], va[VLD], kb2[VLD], vb2[VLD];
    constexpr int C = kDecodeChunk;
    const int nch = (te - ts + C - 1) / C;
    load(ts, ka, va);
    if (nch > 1) load(ts + C, kb2, vb2);
    store_kv(0, ka, va);
    for (int ci = 0; ci < nch; ci += 2) {
      const int base = ts + ci * C;
      compute(base, 0);
      if (ci + 2 < nch) load(base + 2 * C, ka, va);
      if (ci + 1 < nch) {
        store_kv(1, kb2, vb2);
        compute(base + C, 1);
        if (ci + 3 < nch) load(base + 3 * C, kb2, vb2);
        if (ci + 2 < nch) store_kv(0, ka, va);
      }
    }
    if constexpr (MODE == 0) break;
  }

  // ---- the four lanes of a row hold partial sums over their own tokens
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  lx += __shfl_xor(lx, 16, 64);
  lx += __shfl_xor(lx, 32, 64);
  if (live) {
    const int64_t prow = (((int64_t)b * p.Sq + sqi) * p.Hq + hq) * p.num_splits + split;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = p.out_partial + prow * D;
#pragma unroll
    for (int db = 0; db < DBK; ++db) {
      f32x4 w = o[db] * inv;
      *(f32x4*)(dst + db * 16 + 4 * q4) = w;
    }
    if (q4 == 0) p.lse_partial[prow] = lx > 0.f ? (m + __log2f(lx)) * kLn2 : kNegInf;
  }
}

template <class E, int D>
static hipError_t launch_d(const DecodeParams& p, hipStream_t s) {
#if FA_DECODE_MFMA
  const dim3 g(p.Hkv, p.num_splits, p.B);
  if (!p.block_table) hipLaunchKernelGGL((decode_mfma_kernel<E, D, 0>), g, dim3(64), 0, s, p);
  else if (p.log2_page >= 0) hipLaunchKernelGGL((decode_mfma_kernel<E, D, 1>), g, dim3(64), 0, s, p);
  else hipLaunchKernelGGL((decode_mfma_kernel<E, D, 2>), g, dim3(64), 0, s, p);
  return hipGetLastError();
#endif
  const dim3 grid(p.num_splits, p.Hkv, p.B), block(256);
  const int rows = p.group * p.Sq;
  if (rows <= 1) hipLaunchKernelGGL((decode_kernel<E, D, 1>), grid, block, 0, s, p);
  else if (rows <= 2) hipLaunchKernelGGL((decode_kernel<E, D, 2>), grid, block, 0, s, p);
  else if (rows <= 4) hipLaunchKernelGGL((decode_kernel<E, D, 4>), grid, block, 0, s, p);
  else if (rows <= 8) hipLaunchKernelGGL((decode_kernel<E, D, 8>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((decode_kernel<E, D, 16>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode(Dtype dt, int D, const DecodeParams& p, hipStream_t s) {
  if (dt == kF16) return D == 64 ? launch_d<F16, 64>(p, s) : launch_d<F16, 128>(p, s);
  return D == 64 ? launch_d<BF16, 64>(p, s) : launch_d<BF16, 128>(p, s);
}

}  // namespace fa
