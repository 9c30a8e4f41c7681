// Dense bf16 GEMM on v_mfma_f32_32x32x16_bf16 for the dense parts of the
// layer: the shared expert of the FP4 layers ("DeepSeek V4.1 - Add shared":
// the always-on expert every token passes through) and the router's score
// GEMM z = x Wg^T ("DeepSeek-V3.2-Exp - Routing weights", gate-forward).
//
// C[M, N] = A[M, K] B[N, K]^T with fp32 accumulation; B is one or two [N, K]
// matrices (row layout, or the tiled layout of moe_pack_weights).  The
// 32x32x16 form does twice the work of 16x16x32 per instruction at about the
// same cycle count (2.46 vs 1.38 PFLOP/s measured), which matters for these
// dense, compute-heavy GEMMs.  Operand layout (lane l, r = l % 32, h = l / 32):
//   A: row r, inputs 8h .. 8h+7 of the 16-input step; B: column r, same inputs
//   D: 16 floats, column r, rows 8(e/4) + 4h + e%4 for e = 0..15
//
// Workgroup tile: 128 rows x 128 columns of each matrix, 4 waves as 2 x 2,
// each 64 rows x 64 columns (2 x 2 blocks of 32 x 32 per matrix).  K runs in
// 64-input stages through an LDS copy ring: activations and row-layout
// weights as full-line units (8 rows x 128 bytes, lane l of unit u takes row
// l/8, 16-byte chunk (l%8) ^ (l/8) ^ (bit 1 of u)), tiled weights as their
// 1 KB tiles, the two 16-column blocks of a 32-column block 1 KB apart.  Both
// placements keep a half-wave's 16-byte operand reads on distinct LDS banks:
// on this GPU those banks follow address bits 4..8 with bit 10 folded into
// bit 8, so two units 2 KB apart collide unless their chunks are permuted
// (2-way conflicts before: 25-50 % of these kernels' LDS cycles).  Both weight layouts give the
// MFMAs the same operands in the same order, so the results are identical.
//
// Epilogues: SwiGLU of the two matrices (clamped as the routed experts) to
// bf16 rows; one matrix to fp32, one partial sum per split of K (the router's
// scores; the selection kernel adds the parts).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "gemm.h"

namespace moe {
namespace {

struct DenseArgs {
  const bf16 *A;           // [M, K]
  int64_t M;
  int K, N;
  const bf16 *B[2];        // [N, K] each
  int tiled;               // B in the tiled layout
  int k_parts;             // splits of K (fp32 output only)
  bf16 *C;                 // NB = 2: bf16 output [M, N], SwiGLU of the two
  float *Cf;               // NB = 1: fp32 output [k_parts, M, N]
  float limit;             // SwiGLU clamp; <= 0: none
};

// LDS: one object per ring slot (see BfRing in experts.hip).
struct DenseRing {
  uint8_t *s[4];
};

template <int NB, int NS>
__device__ __forceinline__ void dense_tile(const DenseArgs &g, int64_t m0, int n0, int part,
                                           const DenseRing &ring) {
  constexpr int BK = 64;
  constexpr int UA = 16;                       // activation units per stage (128 rows / 8)
  constexpr int UB = 16;                       // weight units per stage and matrix
  constexpr int UNITS = UA + NB * UB;
  constexpr int VM = UNITS / 4;                // copies per wave and stage
  static_assert(UNITS % 4 == 0, "units split evenly over the waves");
  static_assert(NS >= 2 && NS <= 4 && (NS - 2) * VM <= 63, "ring depth");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = g.K, N = g.N;
  const int64_t M = g.M;
  const bool tiled = g.tiled != 0;

  // copy sources: unit q of this wave is unit u = wave + 4q of the stage
  const uint8_t *src[VM];
#pragma unroll
  for (int q = 0; q < VM; ++q) {
    const int u = wave + 4 * q;
    if (u < UA) {
      int64_t r = m0 + u * 8 + (lane >> 3);
      r = r < M ? r : M - 1;
      src[q] = (const uint8_t *)(g.A + r * K) + 16 * ((lane & 7) ^ (lane >> 3) ^ ((u >> 1) & 1));
    } else {
      const int ub = u - UA, b = ub / UB, j = ub - b * UB;
      const bf16 *Bm = g.B[b];
      if (tiled) {
        // unit j = 4t + 2k + c: 32-input tile k of the stage of 16-column
        // block 2t + c of the slab (the two column blocks a 32-column read
        // spans sit 1 KB apart, on different banks)
        const int64_t nb = (n0 >> 4) + 2 * (j >> 2) + (j & 1);
        src[q] = (const uint8_t *)(Bm + (nb * (K / 32) + ((j >> 1) & 1)) * 512) + 16 * lane;
      } else {
        const int64_t n = n0 + j * 8 + (lane >> 3);
        src[q] = (const uint8_t *)(Bm + n * K) + 16 * ((lane & 7) ^ (lane >> 3) ^ ((j >> 1) & 1));
      }
    }
  }
  // bytes between stages: 128 in the rows of A and row-layout B; 2 tiles of 1 KB tiled
  const int64_t bstride = tiled ? 2048 : 128;

  // operand reads, k-step s = 0..3 of a stage: A row block rb (rows 32rb ..), B column
  // block cb (32 columns) of matrix b
  const int r32 = lane & 31, h = lane >> 5, rr = lane & 7;
  int aoff[4], boff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = 2 * s + h;                   // 16-byte chunk of the 128-byte row
    aoff[s] = (r32 >> 3) * 1024 + (rr * 8 + (c ^ rr ^ ((r32 >> 4) & 1))) * 16;
    boff[s] = tiled ? ((s >> 1) * 2 + (r32 >> 4)) * 1024 + ((r32 & 15) + 16 * (2 * (s & 1) + h)) * 16
                    : aoff[s];
  }
  const int wr = wave >> 1, wc = wave & 1;

  f32x16 acc[2][NB][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][b][j][e] = 0.f;

  const int nst_all = K / BK;
  const int st0 = (int)((int64_t)nst_all * part / g.k_parts);
  const int nst = (int)((int64_t)nst_all * (part + 1) / g.k_parts) - st0;
  const int last = nst - 1;
  auto issue = [&](int SL, int ST, int q) {
    const int u = wave + 4 * q;
    const int64_t step = u < UA ? 128 : bstride;
    dma16(src[q] + (int64_t)(st0 + ST) * step, ring.s[SL] + u * 1024);
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
#pragma unroll
    for (int q = 0; q < VM; ++q) issue(p, p < last ? p : last, q);

  auto compute_stage = [&](int p, int nx) {
    const int nslot = (p + NS - 1) % NS;
    const uint8_t *A = ring.s[p];
    const uint8_t *Bs = ring.s[p] + UA * 1024;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 av[2], bv[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *(const bf16x8 *)(A + (2 * wr + i) * 4096 + aoff[s]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bv[b][j] = *(const bf16x8 *)(Bs + b * UB * 1024 + (2 * wc + j) * 4096 + boff[s]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[b][j], acc[i][b][j],
                                                                   0, 0, 0);
      // this k-step's share of the refill of the slot stage st-1 used
#pragma unroll
      for (int q = s * ((VM + 3) / 4); q < (s + 1) * ((VM + 3) / 4) && q < VM; ++q)
        issue(nslot, nx, q);
      // keep them here: the scheduler otherwise sinks every copy below the
      // stage's MFMAs, a stage less of prefetch
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nfull = nst - nst % NS;
  for (int s0 = 0; s0 < nfull; s0 += NS) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      const int st = s0 + p;
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT((NS - 2) * VM));
      __builtin_amdgcn_s_barrier();
      compute_stage(p, st + NS - 1 < last ? st + NS - 1 : last);
    }
  }
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) {
    const int st = nfull + p;
    if (st < nst) {
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
      __builtin_amdgcn_s_barrier();
      compute_stage(p, st + NS - 1 < last ? st + NS - 1 : last);
    }
  }
  __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));

  // epilogue: lane holds column n0 + 64wc + 32j + r32, rows m0 + 64wr + 32i + 8(e/4) + 4h + e%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = m0 + 64 * wr + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + 64 * wc + 32 * j + r32;
        if constexpr (NB == 2) {
          g.C[row * N + col] = (bf16)swiglu_pair(acc[i][0][j][e], acc[i][1][j][e], g.limit);
        } else {
          g.Cf[((int64_t)part * M + row) * N + col] = acc[i][0][j][e];
        }
      }
    }
}

// Items (row tile, column tile, K part) are dealt to the 8 XCDs in contiguous
// runs, column tiles fastest, so the column tiles of one row tile share an L2.
// The one-matrix form (router scores: short K parts, latency-bound) runs a
// 2-stage ring in 64 KB of LDS so that two workgroups share a CU and cover
// each other's waits; the two-matrix form keeps one workgroup per CU.
template <int NB, int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 2 : 1,
                                                                     NB == 1 ? 2 : 1)))
void dense_gemm(const DenseArgs g) {
  constexpr int SLOT = (16 + NB * 16) * 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t L0[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t L1[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t L2[NS > 2 ? SLOT : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t L3[NS > 3 ? SLOT : 1];
  const DenseRing ring{{L0, L1, L2, L3}};
  const int n_nt = g.N / 128;
  const int64_t n_mt = (g.M + 127) / 128;
  const int64_t items = n_mt * n_nt * g.k_parts;
  const int64_t per = (items + 7) / 8;
  const int64_t item = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if ((blockIdx.x >> 3) >= per || item >= items) return;
  const int nt = (int)(item % n_nt);
  const int64_t rest = item / n_nt;
  const int part = (int)(rest % g.k_parts);
  const int64_t mt = rest / g.k_parts;
  dense_tile<NB, NS>(g, mt * 128, nt * 128, part, ring);
}

template <int NB, int NS>
hipError_t run_dense(const DenseArgs &g, hipStream_t s) {
  const int64_t items = ((g.M + 127) / 128) * (g.N / 128) * g.k_parts;
  if (items <= 0) return hipSuccess;
  const int64_t blocks = 8 * ((items + 7) / 8);
  hipLaunchKernelGGL((dense_gemm<NB, NS>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_swiglu(const void *A, int64_t M, int K, int N, const void *Bg,
                               const void *Bu, bool tiled, float limit, void *H, hipStream_t s) {
  if (N % 128 || K % 64) return hipErrorInvalidValue;
  DenseArgs g = {};
  g.A = (const bf16 *)A; g.M = M; g.K = K; g.N = N;
  g.B[0] = (const bf16 *)Bg; g.B[1] = (const bf16 *)Bu;
  g.tiled = tiled ? 1 : 0; g.k_parts = 1; g.C = (bf16 *)H; g.limit = limit;
  return run_dense<2, 3>(g, s);
}

hipError_t launch_dense_f32_parts(const void *A, int64_t M, int K, int N, const void *B,
                                  int k_parts, float *Cf, hipStream_t s) {
  if (N % 128 || K % 64 || k_parts < 1 || k_parts > K / 64) return hipErrorInvalidValue;
  DenseArgs g = {};
  g.A = (const bf16 *)A; g.M = M; g.K = K; g.N = N;
  g.B[0] = (const bf16 *)B;
  g.tiled = 0; g.k_parts = k_parts; g.Cf = Cf;
  return run_dense<1, 2>(g, s);
}

}  // namespace moe
