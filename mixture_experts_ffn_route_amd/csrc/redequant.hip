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

// Every element of a 32-input sub-block is one of the eight E2M1 magnitudes
// times 2^d (d = the sub-block's scale minus the block's) with the code's
// sign.  Byte m of the pair (lo, hi) is the E4M3 code of magnitude m times 2^d
// (bytes 0..3 in lo), byte m of (badlo, badhi) is 1 where that code is not
// exact (or a nonzero magnitude underflows fp32).
__device__ __forceinline__ void e4m3_table(int d, uint32_t &lo, uint32_t &hi, uint32_t &badlo,
                                           uint32_t &badhi) {
  lo = hi = badlo = badhi = 0;
#pragma unroll
  for (uint32_t m = 0; m < 8; ++m) {
    const float v = ldexpf(e2m1_value(m), d);
    const uint32_t e8 = e4m3_code(v);
    const uint32_t bad = (e4m3_value(e8) != v) | (m != 0 && v == 0.f);
    if (m < 4) {
      lo |= e8 << (8 * m);
      badlo |= bad << (8 * m);
    } else {
      hi |= e8 << (8 * (m - 4));
      badhi |= bad << (8 * (m - 4));
    }
  }
}

// E4M3 codes of the four E2M1 nibbles in the low 16 bits of x (byte k: nibble
// k), by a byte select from the sub-block's table; *bad collects the inexact
// flags of the magnitudes present.
__device__ __forceinline__ uint32_t e4m3_of_nibbles(uint32_t x, uint32_t lo, uint32_t hi,
                                                    uint32_t badlo, uint32_t badhi,
                                                    uint32_t *bad) {
  uint32_t t = x & 0xFFFFu;
  t = (t | (t << 8)) & 0x00FF00FFu;
  t = (t | (t << 4)) & 0x0F0F0F0Fu;            // byte k = nibble k
  const uint32_t sel = t & 0x07070707u;        // magnitude index per byte
  *bad |= __builtin_amdgcn_perm(badhi, badlo, sel);
  return __builtin_amdgcn_perm(hi, lo, sel) | ((t & 0x08080808u) << 4);
}

// One workgroup per 128 x 128 block.  Thread t converts the 32-input
// sub-blocks (row t/4 + 64j, part t%4), j = 0, 1: four lanes cover a row's 64
// bytes of codes, so a wave reads 16 rows per load and writes 256 contiguous
// bytes per output quarter.  The block maximum is taken per wave by lane
// shuffles, then over the four waves through LDS (one barrier).
__global__ __launch_bounds__(256) void redequant_fp8_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int N, int K, uint8_t *__restrict__ out,
                                                            uint8_t *__restrict__ bscale,
                                                            uint8_t *__restrict__ lossy) {
  __shared__ int red[4];
  const int nbi = N / 128, nbj = K / 128;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / ((int64_t)nbi * nbj);
  const int rest = (int)(blk - mat * nbi * nbj);
  const int bi = rest / nbj, bj = rest - bi * nbj;
  const int t = threadIdx.x;
  const int KB = K / 2, KS = K / 32;
  const int part = t & 3;

  uint4 cw[2];
  int sc[2];
  int smax = -1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (t >> 2) + 64 * j;
    const int64_t n = (int64_t)bi * 128 + row;
    cw[j] = *(const uint4 *)(codes + (mat * N + n) * KB + bj * 64 + part * 16);
    sc[j] = scales[(mat * N + n) * KS + bj * 4 + part];
    // a sub-block with a nonzero magnitude bit in any nibble sets the maximum
    const uint32_t any = (cw[j].x | cw[j].y | cw[j].z | cw[j].w) & 0x77777777u;
    if (any) smax = smax > sc[j] ? smax : sc[j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int o = __shfl_xor(smax, off);
    smax = smax > o ? smax : o;
  }
  if ((t & 63) == 0) red[t >> 6] = smax;
  __syncthreads();
  int top = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) top = top > red[w] ? top : red[w];
  top = top < 0 ? 127 : top;
  const int B = top - 6 > 0 ? top - 6 : 0;

  int bad = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (t >> 2) + 64 * j;
    const int n = bi * 128 + row, nb = n >> 4, c = n & 15;
    const int h = part >> 1, q0 = 2 * (part & 1);
    const uint32_t w4[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
    uint32_t lo, hi, badlo, badhi, badv = 0;
    // (a nonzero code that underflows fp32 -- a spread beyond 2^140 -- is lossy too)
    e4m3_table(sc[j] - B, lo, hi, badlo, badhi);
    uint32_t o[8];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {           // nibble b of word wd: input 8*wd + b
      o[2 * wd] = e4m3_of_nibbles(w4[wd], lo, hi, badlo, badhi, &badv);
      o[2 * wd + 1] = e4m3_of_nibbles(w4[wd] >> 16, lo, hi, badlo, badhi, &badv);
    }
    bad |= badv != 0;
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
