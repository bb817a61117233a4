// LSE-weighted combine of split partial results (gfx950).
//
// Each split attended a disjoint key chunk and produced its own softmax
// average out_s and log normaliser lse_s (Flash-Attention v2.0-v2.7 update
// notes, v2.2: a separate kernel merges the chunks).  With M = max_s lse_s and
// w_s = exp(lse_s - M), the merged result is out = Σ w_s out_s / Σ w_s and
// lse = M + ln Σ w_s; a row whose splits are all empty (lse = -inf) gets 0 and
// -inf.  Shapes follow "FlashAttention 常用接口简单介绍", §3.4
// (out_partial [B, S, H, D, splits], lse_partial [B, S, H, splits]); any
// element strides are accepted, so the decode workspace order also works.
//
// One wave per (b, s, h) row: lane s reads lse_s (splits <= 64) and two wave
// reductions give M and Σ w; then combine_rows_kernel (decode workspace layout)
// or combine_kernel (any strides, any D) accumulates the weighted partials.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <class E>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  using T = typename E::T;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)p.B * p.S * p.H;
  if (row >= nrows) return;
  const int h = (int)(row % p.H);
  const int s = (int)((row / p.H) % p.S);
  const int b = (int)(row / ((int64_t)p.H * p.S));

  const float* lp = p.lse_partial + b * p.lp_sb + s * p.lp_ss + h * p.lp_sh;
  const float* opp = p.out_partial + b * p.op_sb + s * p.op_ss + h * p.op_sh;
  const float my = lane < p.num_splits ? lp[lane * p.lp_sn] : kNegInf;
  const float M = wave_max(my);
  const float Mu = M == kNegInf ? 0.f : M;
  const float w = lane < p.num_splits ? __expf(my - Mu) : 0.f;
  const float W = wave_sum(w);
  const float inv = W > 0.f ? 1.f / W : 0.f;

  T* orow = (T*)p.out + b * p.o_sb + s * p.o_ss + h * p.o_sh;
  // Each lane owns up to kCombineCols columns; the loads of all splits are issued
  // before they are consumed.  Splits with weight 0 (empty, lse = -inf) are
  // never read, so their partials may hold anything.
  constexpr int kCombineCols = 4;
  for (int d0 = 0; d0 < p.D; d0 += 64 * kCombineCols) {
    float acc[kCombineCols] = {};
    for (int sp = 0; sp < p.num_splits; ++sp) {
      const float ws = __shfl(w, sp, 64);
      if (ws == 0.f) continue;                       // uniform across the wave
      const float* src = opp + sp * p.op_sn;
#pragma unroll
      for (int c = 0; c < kCombineCols; ++c) {
        const int d = d0 + c * 64 + lane;
        if (d < p.D) acc[c] = fmaf(ws, src[d * p.op_sd], acc[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < kCombineCols; ++c) {
      const int d = d0 + c * 64 + lane;
      if (d < p.D) orow[d] = E::from_f32(acc[c] * inv);
    }
  }
  if (p.lse && lane == 0)
    p.lse[b * p.l_sb + s * p.l_ss + h * p.l_sh] = W > 0.f ? M + __logf(W) : kNegInf;
}

// Fast path for D in {64, 128} with unit d stride and 16-byte aligned split rows
// (the decode workspace layout).  Lane l reads columns 4c .. 4c+3, c = l % (D/4),
// of splits g, g + SG, g + 2 SG, ... with g = l / (D/4) and SG = 64 / (D/4); the
// loads of up to 8 splits are issued together before any is consumed (a lane
// past the last split re-reads an existing one and weighs it 0), and the SG partial sums
// of a column are added across lanes at the end.
template <class E, int D>
__global__ __launch_bounds__(256) void combine_rows_kernel(CombineParams p) {
  using T = typename E::T;
  constexpr int CL = D / 4;       // lanes per split row
  constexpr int SG = 64 / CL;     // splits read side by side
  constexpr int UB = 8;           // splits per lane in flight
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)p.B * p.S * p.H;
  if (row >= nrows) return;
  const int h = (int)(row % p.H);
  const int s = (int)((row / p.H) % p.S);
  const int b = (int)(row / ((int64_t)p.H * p.S));
  const int ns = p.num_splits;

  const float* lp = p.lse_partial + b * p.lp_sb + s * p.lp_ss + h * p.lp_sh;
  const int c = lane % CL, g = lane / CL;
  // lanes whose first split does not exist read split 0 (weight 0)
  const float* src = p.out_partial + b * p.op_sb + s * p.op_ss + h * p.op_sh + (g < ns ? g : 0) * p.op_sn + 4 * c;
  const float my = lane < ns ? lp[lane * p.lp_sn] : kNegInf;
  const float M = wave_max(my);
  const float Mu = M == kNegInf ? 0.f : M;
  const float e = lane < ns ? __expf(my - Mu) : 0.f;
  const float W = wave_sum(e);

  const int rounds = (ns + SG - 1) / SG;
  f32x4 acc = f32x4{};
  for (int r0 = 0; r0 < rounds; r0 += UB) {
    f32x4 x[UB];
    float wt[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int sp = (r0 + u) * SG + g;
      const bool in = sp < ns;
      x[u] = *(const f32x4*)(src + (in ? (int64_t)(r0 + u) * SG * p.op_sn : 0));
      wt[u] = __shfl(e, in ? sp : 0, 64);
      if (!in) wt[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < UB; ++u)
      if (wt[u] > 0.f) acc += wt[u] * x[u];   // weight 0: the split may hold anything
  }
#pragma unroll
  for (int m = CL; m < 64; m <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], m, 64);
  }
  if (g == 0) {
    const float inv = W > 0.f ? 1.f / W : 0.f;
    T* orow = (T*)p.out + b * p.o_sb + s * p.o_ss + h * p.o_sh + 4 * c;
    typedef T T4 __attribute__((ext_vector_type(4)));
    T4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = E::from_f32(acc[i] * inv);
    *(T4*)orow = v;
  }
  if (p.lse && lane == 0)
    p.lse[b * p.l_sb + s * p.l_ss + h * p.l_sh] = W > 0.f ? M + __logf(W) : kNegInf;
}

hipError_t launch_combine(Dtype dt, const CombineParams& p, hipStream_t s) {
  const int64_t nrows = (int64_t)p.B * p.S * p.H;
  const dim3 grid((unsigned)((nrows + 3) / 4)), block(256);
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  auto a8 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 7u) == 0; };
  const bool rows_ok = (p.D == 64 || p.D == 128) && p.op_sd == 1 && a16(p.out_partial) &&
                       p.op_sb % 4 == 0 && p.op_ss % 4 == 0 && p.op_sh % 4 == 0 && p.op_sn % 4 == 0 &&
                       a8(p.out) && p.o_sb % 4 == 0 && p.o_ss % 4 == 0 && p.o_sh % 4 == 0;
  if (rows_ok) {
    if (dt == kF16) {
      if (p.D == 64) hipLaunchKernelGGL((combine_rows_kernel<F16, 64>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((combine_rows_kernel<F16, 128>), grid, block, 0, s, p);
    } else {
      if (p.D == 64) hipLaunchKernelGGL((combine_rows_kernel<BF16, 64>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((combine_rows_kernel<BF16, 128>), grid, block, 0, s, p);
    }
  } else if (dt == kF16) {
    hipLaunchKernelGGL((combine_kernel<F16>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((combine_kernel<BF16>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace fa
