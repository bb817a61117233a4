// Device helpers for the gfx950 (CDNA4) attention kernels: element types,
// MFMA wrappers, conversions, exp2 and cross-lane operations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Element traits: storage type, 8-wide MFMA operand vector, packed pair.
struct F16 {
  typedef _Float16 T;
  typedef f16x8 V8;
  typedef f16x2 V2;
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // round-to-nearest-even pack of two floats (v_cvt_pk_f16_f32)
  static __device__ __forceinline__ V2 pack(float a, float b) {
    V2 r; r[0] = (T)a; r[1] = (T)b; return r;
  }
  // fp32 accumulate of the pair's sum: a.x*1 + a.y*1 + c (v_dot2c_f32_f16)
  static __device__ __forceinline__ float sum2(V2 a, float c) {
    const V2 one = {(T)1.0f, (T)1.0f};
    return __builtin_amdgcn_fdot2(a, one, c, false);
  }
  static __device__ __forceinline__ float to_f32(T x) { return (float)x; }
  static __device__ __forceinline__ T from_f32(float x) { return (T)x; }
};

struct BF16 {
  typedef __bf16 T;
  typedef bf16x8 V8;
  typedef bf16x2 V2;
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ V2 pack(float a, float b) {
    V2 r; r[0] = (T)a; r[1] = (T)b; return r;
  }
  static __device__ __forceinline__ float sum2(V2 a, float c) {
    const V2 one = {(T)1.0f, (T)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(a, one, c, false);
  }
  static __device__ __forceinline__ float to_f32(T x) { return (float)x; }
  static __device__ __forceinline__ T from_f32(float x) { return (T)x; }
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Scheduling of a block that forms N values of P: each exponential (a TRANS
// instruction) is placed after G other VALU instructions, so the wave's
// exponentials are spread among its FMAs, packs and adds instead of issuing in
// runs; the transcendental unit then works beside the VALU.  Changes only the
// order of independent instructions.
template <int N, int G>
__device__ __forceinline__ void spread_exponentials() {
  if constexpr (G > 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x002, G, 0);   // VALU (not TRANS, not MFMA)
      __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);   // TRANS
    }
  }
}

// s_waitcnt vmcnt(0): every vector-memory access issued so far has completed.
// Placed before a loop, it tells the compiler that registers loaded before the
// loop are ready, so waits inside the loop count only the loop's own loads.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Value of x held by the lane in the other 32-lane half (lane l <-> l ^ 32).
__device__ __forceinline__ float other_half(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0..31 receive the upper half's value in r[1]; lanes 32..63 in r[0]
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// max / sum of x over the pair of lanes {l, l ^ 32}
__device__ __forceinline__ float max_halves(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max / sum of x over the pair of lanes {l, l ^ 16} (v_permlane16_swap: the two
// results hold the lane's own value and its partner's, in some order)
__device__ __forceinline__ float max_xor16(float x) {
  u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup order over (unit, tile) pairs, a unit being a (batch, head) with
// n_tiles tiles: workgroup id takes the tile of rank `rank` (0 = dispatched
// first) of unit `unit`.
//  * group > 0: the units go in groups of `group`, and inside a group ranks go
//    slowest, so the tiles of equal rank of the group's units are dispatched
//    together.  A caller that maps rank 0 to its longest tile (the last query
//    tile, or the first key tile, under a causal mask) then gets longest-first
//    within each group; a group that spans at least the workgroups resident on
//    an XCD keeps the tail short, and a small group keeps few heads' K/V in
//    flight for the L2.  Unit by unit (group 1), the long tiles of the last
//    units would start late and stretch the tail.
//  * group == 0: units go slowest (all tiles of one unit together), the order
//    for tiles of equal length.
// With xcd set (n_units a multiple of 8), the workgroups the hardware deals to
// XCD id % 8 cover a contiguous eighth of the units, whose K/V then stay in
// that XCD's L2.
__device__ __forceinline__ void tile_order(int id, int n_units, int n_tiles, bool xcd, int group, int& unit,
                                           int& rank) {
  int k = id, u0 = 0, nu = n_units;
  if (xcd) {
    nu = n_units >> 3;
    u0 = (id & 7) * nu;
    k = id >> 3;
  }
  if (group > 0) {
    const int per = group * n_tiles;               // workgroups of a full group
    const int g = k / per;
    const int gu = min(group, nu - g * group);     // units of this group (the last may have fewer)
    const int w = k - g * per;
    rank = w / gu;
    unit = u0 + g * group + (w - rank * gu);
  } else {
    const int uu = k / n_tiles;
    rank = k - uu * n_tiles;
    unit = u0 + uu;
  }
}

// Debug build (FA_LDS_POISON=1): fill an LDS staging buffer with all-ones bits
// (NaN in fp16, bf16 and fp32) and wait for the whole workgroup, before any tile
// is stored.  A read that a missing wait or barrier lets run ahead of its tile's
// store then carries NaN into the output.  The ordinary build does nothing.
#ifndef FA_LDS_POISON
#define FA_LDS_POISON 0
#endif
__device__ __forceinline__ void lds_poison(void* lds, size_t bytes, int tid, int nthreads) {
  if constexpr (FA_LDS_POISON) {
    uint32_t* w = static_cast<uint32_t*>(lds);
    for (size_t i = tid; i < bytes / 4; i += nthreads) w[i] = 0xffffffffu;
    __syncthreads();
  }
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunk addressed by lane
// 4*j + i/4, for j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p));
}

}  // namespace fa
