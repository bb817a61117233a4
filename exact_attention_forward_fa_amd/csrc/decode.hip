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
  constexpr int U = 2;                  // tokens per slot per iteration
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

  auto token_row = [&](int t) -> int64_t {    // cache row index of token t
    if (!bt) return (int64_t)b * p.page_size + t;
    const int pg = p.log2_page >= 0 ? (t >> p.log2_page) : t / p.page_size;
    const int in = p.log2_page >= 0 ? (t & (p.page_size - 1)) : t - pg * p.page_size;
    return (int64_t)bt[pg] * p.page_size + in;
  };

  float m[R], l[R], o[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[r][i] = 0.f;
  }

  u32x4 kr[U], vr[U];
  auto issue = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(base + u * SLOTS + slot, t1 - 1);    // clamp: a real token, masked below
      const int64_t row = token_row(t);
      kr[u] = *(const u32x4*)(kbase + row * row_elems);
      vr[u] = *(const u32x4*)(vbase + row * row_elems);
    }
  };

  if (t0 < t1) issue(t0);
  for (int base = t0; base < t1; base += STEP) {
    u32x4 kc[U], vc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { kc[u] = kr[u]; vc[u] = vr[u]; }
    if (base + STEP < t1) issue(base + STEP);

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
        if (t >= t1 || t < jlo[r] || t > jhi[r]) x = kNegInf;
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

template <class E, int D>
static hipError_t launch_d(const DecodeParams& p, hipStream_t s) {
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
