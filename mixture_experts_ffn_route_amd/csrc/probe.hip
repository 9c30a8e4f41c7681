// Roofline probes (moe_probe_read, moe_probe_mfma): the achievable HBM read
// bandwidth and bf16 / FP8 MFMA rates of this GPU, measured with the same
// instruction forms the layer kernels use, as second denominators next to
// the data-sheet peaks.  The caller times them on its stream.

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

// Each wave streams its own contiguous 1/(4*grid) of the buffer, 1 KB per
// nontemporal load instruction (the form decode-height GEMM tiles stream
// their weights with, and the faster one for a pure stream) and eight
// instructions in flight; the loaded words feed a
// value that is stored only if it matches a constant, so no load is dead.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4 *p, int64_t n16,
                                                         uint32_t *out) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t per = n16 / waves;
  const u32x4 *q = p + w * per;
  uint32_t acc = 0;
  int64_t k = lane;
  for (; k + 7 * 64 < per; k += 8 * 64) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(q + k + u * 64);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][u & 3];
  }
  for (; k < per; k += 64) acc ^= q[k][0];
  if (w == 0)
    for (int64_t j = waves * per + lane; j < n16; j += 64) acc ^= p[j][0];
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

// Independent MFMA chains per wave, `iters` rounds: 8 chains of 16x16x32 bf16
// (shape 0) or 32x32x16 bf16 (shape 1), or 16 chains of the scaled
// 16x16x128 form the MXFP8 kernels use, E4M3 x E2M1 (shape 2) or E4M3 x E4M3
// (shape 3), unit scales; the host counts the flops.
typedef int i32x8_p __attribute__((ext_vector_type(8)));
template <int SHAPE>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *out) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (bf16)(0.002f * (float)((lane * 3 + i) & 7));
  }
  float s = 0.f;
  if constexpr (SHAPE == 1) {
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][15];
  } else if constexpr (SHAPE == 0) {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    // small E4M3 values (0x30 ~ 0.5) and E2M1 codes, exponent 127 = scale 1
    i32x8_p qa, qb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[i] = 0x30303030 ^ ((lane + i) & 7);
      qb[i] = SHAPE == 2 ? (0x22222222 ^ ((lane * 3 + i) & 7)) : (0x28282828 ^ ((lane * 3 + i) & 7));
    }
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, qb, acc[j], 0,
                                                                 SHAPE == 2 ? 4 : 0, 0, 127, 0, 127);
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][3];
  }
  if (s == 1234.5f) out[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_probe_read(const void *buf, int64_t bytes, uint32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(1024), dim3(256), 0, s, (const u32x4 *)buf,
                     bytes / 16, out);
  return hipGetLastError();
}

// 2048 workgroups x 4 waves (eight waves per SIMD), 8 chains each (16 for
// the scaled shapes).
int64_t probe_mfma_flops(int iters, int shape) {
  const int64_t per_mfma = shape == 1 ? 32 * 32 * 16 * 2 : shape == 0 ? 16 * 16 * 32 * 2
                                                                     : 16 * 16 * 128 * 2;
  return (int64_t)2048 * 4 * iters * (shape >= 2 ? 16 : 8) * per_mfma;
}

hipError_t launch_probe_mfma(int iters, int shape, float *out, hipStream_t s) {
  switch (shape) {
    case 0: hipLaunchKernelGGL(probe_mfma_kernel<0>, dim3(2048), dim3(256), 0, s, iters, out); break;
    case 1: hipLaunchKernelGGL(probe_mfma_kernel<1>, dim3(2048), dim3(256), 0, s, iters, out); break;
    case 2: hipLaunchKernelGGL(probe_mfma_kernel<2>, dim3(2048), dim3(256), 0, s, iters, out); break;
    case 3: hipLaunchKernelGGL(probe_mfma_kernel<3>, dim3(2048), dim3(256), 0, s, iters, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
