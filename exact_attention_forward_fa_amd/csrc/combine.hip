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
// One wave per (b, s, h) row: lane s reads lse_s (splits <= 64), two wave
// reductions give M and Σ w, then each lane accumulates its D/64 columns.
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

hipError_t launch_combine(Dtype dt, const CombineParams& p, hipStream_t s) {
  const int64_t nrows = (int64_t)p.B * p.S * p.H;
  const dim3 grid((unsigned)((nrows + 3) / 4)), block(256);
  if (dt == kF16) hipLaunchKernelGGL((combine_kernel<F16>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((combine_kernel<BF16>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
