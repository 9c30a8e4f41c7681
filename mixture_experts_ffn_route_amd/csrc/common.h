// Shared device-side types and wavefront helpers for the gfx950 MoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Lane exchange across the wavefront at distance M (xor pattern).  Distances
// 1 and 2 use DPP quad permutes, 4..16 the ds_swizzle bit-mask mode (xor
// within 32-lane halves), 32 a bpermute across the halves.
template <int M>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);   // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);   // quad_perm 2,3,0,1
  } else if constexpr (M < 32) {
    return __builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1F);
  } else {
    return __shfl_xor(v, 32);
  }
}

template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  return __int_as_float(xor_lane<M>(__float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lane<1>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<8>(v));
  v = fmaxf(v, xor_lane<16>(v));
  v = fmaxf(v, xor_lane<32>(v));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane<1>(v);
  v += xor_lane<2>(v);
  v += xor_lane<4>(v);
  v += xor_lane<8>(v);
  v += xor_lane<16>(v);
  v += xor_lane<32>(v);
  return v;
}

__device__ __forceinline__ float bf16_to_f32(bf16 v) { return (float)v; }

// SwiGLU of one gate / up pair, with the clamp when L > 0 (gate capped at L,
// up clamped to [-L, L]).  SiLU divides by the hardware reciprocal (v_rcp_f32,
// 1 ulp) instead of the correctly rounded division sequence: the value is
// rounded to bf16 or E4M3 right after, and 1 + e^-g >= 1 keeps the reciprocal
// away from zero and denormals (e^-g = inf gives 0, the limit).
__device__ __forceinline__ float swiglu_pair(float g, float u, float L) {
  if (L > 0.f) {
    g = fminf(g, L);
    u = fminf(fmaxf(u, -L), L);
  }
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

}  // namespace moe
