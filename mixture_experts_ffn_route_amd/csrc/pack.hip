// Tiled storage of the expert matrices (moe_pack_weights).
//
// The grouped GEMMs give each lane of a wave one MFMA B operand per load:
// 16 output columns x 8 consecutive inputs (bf16), or 16 columns x 16
// consecutive inputs (FP4 codes) plus their scale.  In the row layout those
// 64 operands sit on 16 rows 2K bytes apart; the tiled layout stores each
// 16-column x 32-input (bf16) or 16-column x 64-input (FP4) tile as one
// contiguous block in exactly that lane order, so every load of the GEMM reads
// a contiguous 1 KB (bf16) or 512 B (FP4 codes) and consecutive K stages of a
// column block follow each other in memory.  Values are only moved.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace moe {
namespace {

// One thread per 16-byte group (bf16) of the destination: tile t = group / 64,
// lane l = group % 64 holds row (t / (K/32))*16 + l%16, inputs
// (t % (K/32))*32 + (l/16)*8 .. +7.
__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint4 *__restrict__ src,
                                                        uint4 *__restrict__ dst, int64_t groups,
                                                        int64_t N, int64_t K) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  const int64_t per_mat = N * K / 8;       // 16-byte groups per expert matrix
  const int64_t e = g / per_mat;
  const int64_t r = g - e * per_mat;
  const int64_t tile = r >> 6;
  const int lane = (int)(r & 63);
  const int64_t kt = K / 32;
  const int64_t nb = tile / kt, kb = tile - nb * kt;
  const int64_t n = nb * 16 + (lane & 15);
  const int64_t k0 = kb * 32 + (lane >> 4) * 8;
  dst[g] = src[e * per_mat + (n * K + k0) / 8];
}

// FP4 codes: one thread per 8-byte group; tile = 16 rows x 32 bytes (64 inputs).
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint2 *__restrict__ src,
                                                       uint2 *__restrict__ dst, int64_t groups,
                                                       int64_t N, int64_t K) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  const int64_t KB = K / 2;                // bytes per row
  const int64_t per_mat = N * KB / 8;
  const int64_t e = g / per_mat;
  const int64_t r = g - e * per_mat;
  const int64_t tile = r >> 6;
  const int lane = (int)(r & 63);
  const int64_t kt = K / 64;
  const int64_t nb = tile / kt, kb = tile - nb * kt;
  const int64_t n = nb * 16 + (lane & 15);
  const int64_t b0 = kb * 32 + (lane >> 4) * 8;
  dst[g] = src[e * per_mat + (n * KB + b0) / 8];
}

// E8M0 scales: one thread per byte; tile = 16 rows x 2 scale blocks (32 bytes).
__global__ __launch_bounds__(256) void pack_scale_kernel(const uint8_t *__restrict__ src,
                                                         uint8_t *__restrict__ dst, int64_t bytes,
                                                         int64_t N, int64_t K) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= bytes) return;
  const int64_t KS = K / 32;               // scales per row
  const int64_t per_mat = N * KS;
  const int64_t e = i / per_mat;
  const int64_t r = i - e * per_mat;
  const int64_t tile = r >> 5;
  const int j = (int)(r & 31);
  const int64_t kt = K / 64;
  const int64_t nb = tile / kt, kb = tile - nb * kt;
  const int64_t n = nb * 16 + (j >> 1);
  const int64_t c = kb * 2 + (j & 1);
  dst[i] = src[e * per_mat + n * KS + c];
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_pack_matrix(const void *src, void *dst, int64_t count, int64_t N, int64_t K,
                              int dtype, bool scales, hipStream_t s) {
  if (!src || count <= 0) return hipSuccess;
  if (scales) {
    const int64_t bytes = count * N * (K / 32);
    hipLaunchKernelGGL(pack_scale_kernel, dim3(blocks_for(bytes)), dim3(256), 0, s,
                       (const uint8_t *)src, (uint8_t *)dst, bytes, N, K);
  } else if (dtype == MOE_DTYPE_FP4_E2M1) {
    const int64_t groups = count * N * (K / 2) / 8;
    hipLaunchKernelGGL(pack_fp4_kernel, dim3(blocks_for(groups)), dim3(256), 0, s,
                       (const uint2 *)src, (uint2 *)dst, groups, N, K);
  } else {
    const int64_t groups = count * N * K / 8;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(blocks_for(groups)), dim3(256), 0, s,
                       (const uint4 *)src, (uint4 *)dst, groups, N, K);
  }
  return hipGetLastError();
}

}  // namespace moe
