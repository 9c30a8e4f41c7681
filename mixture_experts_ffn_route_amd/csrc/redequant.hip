// FP4 -> FP8 re-dequantisation of expert weights ("From One Giant FFN to 384
// Tiny Experts", Ch.11.6): FP4 (E2M1) codes with one E8M0 scale per 32 inputs
// become E4M3 codes with one E8M0 scale per 128 x 128 block.  E4M3 has two
// more exponent bits than E2M1, so the ratio between a sub-block's scale and
// the block's goes into the element's exponent: the block scale is the
// largest scale among the block's sub-blocks that hold a nonzero code, over
// 2^6 (6 x 2^6 = 384 fits E4M3), and an element is e2m1 x 2^(s - B).  That is
// exact while s is at most 14 below the largest (the smallest E2M1 magnitude
// 0.5 x 2^-8 is E4M3's smallest step); larger spreads round to nearest, ties
// to even, and the block is reported lossy.
//
// Output layout (what the FP8 grouped GEMM copies into LDS and reads as MFMA
// operands): per matrix, column block nb (16 rows) and 128-input stage st, a
// 2 KB block whose byte ((h*4 + q)*16 + c)*16 + i is the element of row
// 16nb + c, input 128st + 64h + 16q + i.  Lane (c, q) of the MFMA then reads
// its two 16-byte operand halves at (q*16 + c)*16 and 1024 + (q*16 + c)*16.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8.h"
#include "internal.h"

namespace moe {
namespace {

// One workgroup per 128 x 128 block; thread t converts the sub-blocks
// (row 2t/4.., part (2t)%4 ..) -- two 32-input sub-blocks per thread.
__global__ __launch_bounds__(256) void redequant_fp8_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int N, int K, uint8_t *__restrict__ out,
                                                            uint8_t *__restrict__ bscale,
                                                            uint8_t *__restrict__ lossy) {
  __shared__ int red[256];
  const int nbi = N / 128, nbj = K / 128;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / ((int64_t)nbi * nbj);
  const int rest = (int)(blk - mat * nbi * nbj);
  const int bi = rest / nbj, bj = rest - bi * nbj;
  const int t = threadIdx.x;
  const int KB = K / 2, KS = K / 32;

  uint4 cw[2];
  int sc[2];
  int smax = -1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sub = 2 * t + j, row = sub >> 2, part = sub & 3;
    const int64_t n = (int64_t)bi * 128 + row;
    cw[j] = *(const uint4 *)(codes + (mat * N + n) * KB + bj * 64 + part * 16);
    sc[j] = scales[(mat * N + n) * KS + bj * 4 + part];
    // a sub-block with a nonzero magnitude bit in any nibble sets the maximum
    const uint32_t any = (cw[j].x | cw[j].y | cw[j].z | cw[j].w) & 0x77777777u;
    if (any) smax = smax > sc[j] ? smax : sc[j];
  }
  red[t] = smax;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] = red[t] > red[t + w] ? red[t] : red[t + w];
    __syncthreads();
  }
  const int top = red[0] < 0 ? 127 : red[0];
  const int B = top - 6 > 0 ? top - 6 : 0;

  int bad = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sub = 2 * t + j, row = sub >> 2, part = sub & 3;
    const int n = bi * 128 + row, nb = n >> 4, c = n & 15;
    const int h = part >> 1, q0 = 2 * (part & 1);
    const uint32_t w4[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
    uint32_t o[8];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) {            // nibble b of word wd: input 8*wd + b
        const uint32_t nib = w4[wd] >> (4 * b);
        const float v = ldexpf(e2m1_value(nib), sc[j] - B);
        const uint32_t e8 = e4m3_code(v);
        // (a nonzero code that underflows fp32 -- a spread beyond 2^140 -- is lossy too)
        bad |= (e4m3_value(e8) != v) | ((nib & 7u) != 0 && v == 0.f);
        if (b < 4) lo |= e8 << (8 * b); else hi |= e8 << (8 * (b - 4));
      }
      o[2 * wd] = lo;
      o[2 * wd + 1] = hi;
    }
    // inputs 32*part + 0..15 -> q = q0, 16..31 -> q = q0 + 1
    uint8_t *dst = out + ((mat * (N / 16) + nb) * nbj + bj) * 2048;
    *(uint4 *)(dst + ((h * 4 + q0) * 16 + c) * 16) = uint4{o[0], o[1], o[2], o[3]};
    *(uint4 *)(dst + ((h * 4 + q0 + 1) * 16 + c) * 16) = uint4{o[4], o[5], o[6], o[7]};
  }
  bad = __syncthreads_or(bad);
  if (t == 0) {
    const int64_t bo = (mat * nbi + bi) * nbj + bj;
    bscale[bo] = (uint8_t)B;
    lossy[bo] = bad ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_redequant_fp8(const uint8_t *codes, const uint8_t *scales, int64_t n_mat, int N,
                                int K, uint8_t *out, uint8_t *bscale, uint8_t *lossy,
                                hipStream_t s) {
  const int64_t blocks = n_mat * (N / 128) * (K / 128);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(redequant_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales,
                     N, K, out, bscale, lossy);
  return hipGetLastError();
}

}  // namespace moe
