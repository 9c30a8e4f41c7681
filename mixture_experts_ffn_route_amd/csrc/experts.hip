// Expert computation for gfx950: grouped SwiGLU GEMMs and the combine.
//
// The layer ("DeepSeek V4.1 - Add shared", V4.1 MoE class; "From One Giant
// FFN to 384 Tiny Experts" Ch.1 SwiGLU, Ch.4 routed + shared, Ch.11.4 clamp,
// Ch.11.6 FP4 experts) is computed as:
//   GEMM1  H[r] = SiLU(min(x[tok(r)] W_gate[e]^T, L)) * clamp(x[tok(r)] W_up[e]^T, -L, L)
//   GEMM2  Y[r] = w(r) * (H[r] W_down[e]^T)
//   combine y[t] = sum_j Y[inverse[t, j]] + Y[shared row of t]
// where r runs over the permuted rows (all rows of one expert are adjacent)
// and the shared expert owns T extra rows with weight 1.
//
// Grouped GEMM kernel.  A work item is (tile, slab): a tile is up to BM rows
// of one expert (or of the shared expert), a slab WAVES*NCB*16 output
// columns of each weight matrix.  The weight slab is streamed from HBM
// exactly once per tile -- one tile normally holds all rows of an expert, so
// the routed weights are read once per forward -- straight into registers
// in the MFMA operand layout (no LDS hop for the streamed operand) with a
// PF-1 stage prefetch ring.  The gathered activation rows are staged through
// a double-buffered, XOR-swizzled LDS tile shared by the four waves.  MFMA
// is v_mfma_f32_16x16x32_bf16 (fp32 accumulate).  FP4 weights are loaded as
// 32 codes + one E8M0 scale per lane per 128-deep stage and expanded to bf16
// in registers with v_cvt_scalef32_pk_bf16_fp4.
//
// The workgroup -> work item map is XCD aware: consecutive workgroups land on
// different XCDs, so each XCD is given a contiguous range of items (all
// slabs of the same tiles), and the gathered rows of an expert stay in that
// XCD's L2 while its slabs stream.

#include "common.h"
#include "internal.h"

namespace moe {

struct GemmArgs {
  const bf16 *A;             // activation rows [*, K]
  const int32_t *a_rows;     // source row of each permuted row, or null (identity)
  int K, N;
  const void *B[2];          // routed weights [E, N, K] bf16 or FP4 bytes [E, N, K/2]
  const uint8_t *S[2];       // FP4 scales [E, N, K/32]
  const bf16 *SB[2];         // shared expert weights [N, K]
  int E;                     // group id E = shared expert
  bf16 *C;                   // output rows [*, N]
  const int32_t *tiles, *tile_count;
  int tile_begin, tile_end;  // tile_end < 0: end = *tile_count
  int n_slabs;
  float limit;               // SwiGLU clamp (two-matrix form); <= 0: none
  const float *route_w;      // one-matrix form: gate value of each (token, slot)
  const int32_t *sorted_tok, *sorted_slot;
  int k;
  int64_t routed_rows;       // T * k: rows at or above this belong to the shared expert
};

template <int NB, int NCB, int MB, bool FP4, int PF>
__global__ __launch_bounds__(256) void grouped_gemm(const GemmArgs g) {
  constexpr int WAVES = 4;
  constexpr int BK = FP4 ? 128 : 64;       // K per LDS stage
  constexpr int SUBS = BK / 32;            // MFMA k-steps per stage
  constexpr int CPR = BK / 8;              // 16-byte chunks per A row per stage
  constexpr int BM = MB * 16;
  constexpr int ACH = BM * CPR;
  constexpr int ACH_T = (ACH + 255) / 256;
  constexpr int NQ = FP4 ? 1 : SUBS;       // 16-byte B loads per (matrix, block) per stage
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * BK];

  // ---- work item (XCD-aware) ----
  const int tend = g.tile_end >= 0 ? g.tile_end : *g.tile_count;
  const int64_t work = (int64_t)(tend - g.tile_begin) * g.n_slabs;
  const int xcd = blockIdx.x & 7;
  const int64_t slot = blockIdx.x >> 3;
  const int64_t per_xcd = (work + 7) >> 3;
  if (slot >= per_xcd) return;
  const int64_t item = xcd * per_xcd + slot;
  if (item >= work) return;
  const int tile = g.tile_begin + (int)(item / g.n_slabs);
  const int slab = (int)(item - (int64_t)(tile - g.tile_begin) * g.n_slabs);
  const int grp = g.tiles[4 * tile], row0 = g.tiles[4 * tile + 1], rows = g.tiles[4 * tile + 2];
  const int nmb = (rows + 15) >> 4;
  const bool shared = grp == g.E;
  const int K = g.K, N = g.N;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, jq = lane >> 4;
  const int col0 = slab * (WAVES * NCB * 16) + wave * NCB * 16;

  // ---- A staging assignment: chunk c -> (row, 16-byte chunk) ----
  const bf16 *asrc[ACH_T];
  int adst[ACH_T];
#pragma unroll
  for (int i = 0; i < ACH_T; ++i) {
    const int c = tid + 256 * i;
    asrc[i] = nullptr;
    adst[i] = -1;
    if (c < nmb * 16 * CPR) {
      const int r = c / CPR, ch = c - r * CPR;
      adst[i] = r * BK + ((ch ^ (r & 7)) * 8);
      if (r < rows) {
        const int64_t src = g.a_rows ? g.a_rows[row0 + r] : (int64_t)(row0 + r);
        asrc[i] = g.A + src * K + ch * 8;
      }
    }
  }

  // ---- B pointers ----
  const uint8_t *bptr[NB][NCB];
  const uint8_t *sptr[NB][NCB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int64_t n = col0 + cb * 16 + r16;
      if constexpr (FP4) {
        const int64_t K2 = K / 2, K32 = K / 32;
        bptr[b][cb] = (const uint8_t *)g.B[b] + ((int64_t)grp * N + n) * K2 + jq * 16;
        sptr[b][cb] = g.S[b] + ((int64_t)grp * N + n) * K32 + jq;
      } else {
        const bf16 *base = shared ? g.SB[b] : (const bf16 *)g.B[b] + (int64_t)grp * N * K;
        bptr[b][cb] = (const uint8_t *)(base + n * K + jq * 8);
        sptr[b][cb] = nullptr;
      }
    }

  f32x4 acc[MB][NB][NCB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[m][b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 bq[PF][NB][NCB][NQ];
  uint32_t sq[PF][NB][NCB];
  u32x4 areg[ACH_T];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int nst = K / BK;

  auto load_a = [&](int st) {
#pragma unroll
    for (int i = 0; i < ACH_T; ++i)
      areg[i] = asrc[i] ? *(const u32x4 *)(asrc[i] + (int64_t)st * BK) : zero4;
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH_T; ++i)
      if (adst[i] >= 0) *(u32x4 *)(&As[buf][adst[i]]) = areg[i];
  };

#define MOE_LOAD_B(SLOT, ST)                                                          \
  {                                                                                   \
    _Pragma("unroll") for (int b = 0; b < NB; ++b)                                    \
    _Pragma("unroll") for (int cb = 0; cb < NCB; ++cb) {                              \
      if constexpr (FP4) {                                                            \
        bq[SLOT][b][cb][0] = *(const u32x4 *)(bptr[b][cb] + (int64_t)(ST) * (BK / 2)); \
        sq[SLOT][b][cb] = sptr[b][cb][(ST) * (BK / 32)];                              \
      } else {                                                                        \
        _Pragma("unroll") for (int q = 0; q < NQ; ++q)                                \
          bq[SLOT][b][cb][q] =                                                        \
              *(const u32x4 *)(bptr[b][cb] + ((int64_t)(ST) * BK + q * 32) * 2);      \
      }                                                                               \
    }                                                                                 \
  }

  // prologue
  load_a(0);
  store_a(0);
#pragma unroll
  for (int p = 0; p < PF - 1; ++p)
    if (p < nst) MOE_LOAD_B(p, p);
  __syncthreads();

  for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int st = s0 + p;
      if (st < nst) {
        const int buf = st & 1;
        if (st + 1 < nst) load_a(st + 1);
        if (st + PF - 1 < nst) MOE_LOAD_B((p + PF - 1) % PF, st + PF - 1);
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) {
          bf16x8 bf[NB][NCB];
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              if constexpr (FP4) {
                const unsigned word = bq[p][b][cb][0][sub];
                const float scale = __uint_as_float(sq[p][b][cb] << 23);
                const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
                const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
                const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
                const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
                bf[b][cb] = bf16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
              } else {
                bf[b][cb] = __builtin_bit_cast(bf16x8, bq[p][b][cb][sub]);
              }
            }
          // A chunk: bf16 keeps k = 32*sub + 8*jq; FP4 uses k = 32*jq + 8*sub so
          // that each lane's 32 weight codes share one scale.  Both operands
          // use the same k order, so the products are unchanged.
          const int ch = FP4 ? (4 * jq + sub) : (4 * sub + jq);
          const bf16 *abase = &As[buf][r16 * BK + ((ch ^ (r16 & 7)) * 8)];
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            if (m < nmb) {
              const bf16x8 a = *(const bf16x8 *)(abase + m * 16 * BK);
#pragma unroll
              for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                  acc[m][b][cb] =
                      __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bf[b][cb], acc[m][b][cb], 0, 0, 0);
            }
          }
        }
        if (st + 1 < nst) store_a(buf ^ 1);
        __syncthreads();
      }
    }
  }
#undef MOE_LOAD_B

  // ---- epilogue ----
  if constexpr (NB == 2) {
    const float L = g.limit;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < nmb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m * 16 + jq * 4 + i;
          if (row < rows) {
            bf16 *crow = g.C + (int64_t)(row0 + row) * N + col0 + r16;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              float gv = acc[m][0][cb][i], uv = acc[m][1][cb][i];
              if (L > 0.f) {
                gv = fminf(gv, L);
                uv = fminf(fmaxf(uv, -L), L);
              }
              const float h = gv / (1.f + __expf(-gv)) * uv;
              crow[cb * 16] = (bf16)h;
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < nmb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m * 16 + jq * 4 + i;
          if (row < rows) {
            const int64_t R = row0 + row;
            float wgt = 1.f;
            if (R < g.routed_rows) wgt = g.route_w[(int64_t)g.sorted_tok[R] * g.k + g.sorted_slot[R]];
            bf16 *crow = g.C + R * N + col0 + r16;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) crow[cb * 16] = (bf16)(acc[m][0][cb][i] * wgt);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 layers (small; correctness path): one thread per output element.
__global__ __launch_bounds__(256) void expert_up_f32(
    const float *x, const int32_t *sorted_tok, const int32_t *sorted_slot,
    const int32_t *route_idx, const int32_t *offsets, int E, int k, int64_t routed_rows,
    int64_t total_rows, int dim, int I, const float *Wg, const float *Wu, const float *SWg,
    const float *SWu, float L, float *H) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (n >= I || r >= total_rows) return;
  const float *wg, *wu;
  if (r < routed_rows) {
    if (r >= offsets[E]) return;
    const int e = route_idx[(int64_t)sorted_tok[r] * k + sorted_slot[r]];
    wg = Wg + ((int64_t)e * I + n) * dim;
    wu = Wu + ((int64_t)e * I + n) * dim;
  } else {
    wg = SWg + (int64_t)n * dim;
    wu = SWu + (int64_t)n * dim;
  }
  const float *xr = x + (int64_t)sorted_tok[r] * dim;
  float gv = 0.f, uv = 0.f;
  for (int i = 0; i < dim; ++i) {
    gv = fmaf(xr[i], wg[i], gv);
    uv = fmaf(xr[i], wu[i], uv);
  }
  if (L > 0.f) {
    gv = fminf(gv, L);
    uv = fminf(fmaxf(uv, -L), L);
  }
  H[r * I + n] = gv / (1.f + expf(-gv)) * uv;
}

__global__ __launch_bounds__(256) void expert_down_f32(
    const float *H, const int32_t *sorted_tok, const int32_t *sorted_slot,
    const int32_t *route_idx, const float *route_w, const int32_t *offsets, int E, int k,
    int64_t routed_rows, int64_t total_rows, int dim, int I, const float *Wd, const float *SWd,
    float *Y) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (n >= dim || r >= total_rows) return;
  const float *wd;
  float wgt = 1.f;
  if (r < routed_rows) {
    if (r >= offsets[E]) return;
    const int64_t pair = (int64_t)sorted_tok[r] * k + sorted_slot[r];
    const int e = route_idx[pair];
    wgt = route_w[pair];
    wd = Wd + ((int64_t)e * dim + n) * I;
  } else {
    wd = SWd + (int64_t)n * I;
  }
  const float *hr = H + r * I;
  float acc = 0.f;
  for (int i = 0; i < I; ++i) acc = fmaf(hr[i], wd[i], acc);
  Y[r * dim + n] = acc * wgt;
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j Y[inverse[t, j]] + Y[T*k + t], fp32 sum in slot order.
__global__ __launch_bounds__(256) void combine_bf16(const bf16 *Y, const int32_t *inverse,
                                                    int k, int dim, int64_t shared_base,
                                                    bf16 *y) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < dim; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = inverse[t * k + j];
      if (r >= 0) {
        const bf16x8 v = *(const bf16x8 *)(Y + (int64_t)r * dim + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += (float)v[i];
      }
    }
    if (shared_base >= 0) {
      const bf16x8 v = *(const bf16x8 *)(Y + (shared_base + t) * dim + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += (float)v[i];
    }
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)acc[i];
    *(bf16x8 *)(y + t * dim + c) = o;
  }
}

__global__ __launch_bounds__(256) void combine_f32(const float *Y, const int32_t *inverse, int k,
                                                   int dim, int64_t shared_base, float *y) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < dim; c += 256) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = inverse[t * k + j];
      if (r >= 0) acc += Y[(int64_t)r * dim + c];
    }
    if (shared_base >= 0) acc += Y[(shared_base + t) * dim + c];
    y[t * dim + c] = acc;
  }
}

// ---------------------------------------------------------------------------
// Host side.

static const int kTileMB[] = {1, 4, 8, 12, 16};

int choose_tile_rows(const moe_config &cfg, int64_t T) {
  if (cfg.act_dtype == MOE_DTYPE_F32) return 16;
  const double avg = (double)T * cfg.n_activated_experts / cfg.n_routed_experts;
  const double want = avg + 3.0 * sqrt(avg) + 4.0;
  for (int mb : kTileMB)
    if (16.0 * mb >= want) return 16 * mb;
  return 256;
}

template <int NB, int NCB, int MB, bool FP4, int PF>
static hipError_t run_gemm(const GemmArgs &a, int max_tiles, hipStream_t s) {
  int64_t blocks = (int64_t)max_tiles * a.n_slabs;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm<NB, NCB, MB, FP4, PF>), dim3((unsigned)blocks), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

template <int NB, int NCB, bool FP4, int PF>
static hipError_t run_gemm_mb(int mb, const GemmArgs &a, int max_tiles, hipStream_t s) {
  switch (mb) {
    case 1: return run_gemm<NB, NCB, 1, FP4, PF>(a, max_tiles, s);
    case 4: return run_gemm<NB, NCB, 4, FP4, PF>(a, max_tiles, s);
    case 8: return run_gemm<NB, NCB, 8, FP4, PF>(a, max_tiles, s);
    case 12: return run_gemm<NB, NCB, 12, FP4, PF>(a, max_tiles, s);
    case 16: return run_gemm<NB, NCB, 16, FP4, PF>(a, max_tiles, s);
    default: return hipErrorInvalidValue;
  }
}

// One grouped GEMM launch over a tile range.
static hipError_t gemm_launch(int nb, bool fp4, int mb, GemmArgs a, int max_tiles,
                              hipStream_t s) {
  const int ncb = (a.N % 128 == 0 && mb <= 1) ? 2 : 1;
  a.n_slabs = a.N / (4 * ncb * 16);
  if (fp4) {
    if (nb == 2) return run_gemm_mb<2, 1, true, 2>(mb, a, max_tiles, s);
    return run_gemm_mb<1, 1, true, 2>(mb, a, max_tiles, s);
  }
  if (ncb == 2) {
    if (nb == 2) return run_gemm_mb<2, 2, false, 4>(mb, a, max_tiles, s);
    return run_gemm_mb<1, 2, false, 4>(mb, a, max_tiles, s);
  }
  if (nb == 2) return run_gemm_mb<2, 1, false, 3>(mb, a, max_tiles, s);
  return run_gemm_mb<1, 1, false, 3>(mb, a, max_tiles, s);
}

static hipError_t mark(const ExpertPlan &p, int i, hipStream_t s) {
  return p.events ? hipEventRecord(p.events[i], s) : hipSuccess;
}

hipError_t launch_experts(const ExpertPlan &p, hipStream_t s) {
  const int64_t routed_rows = p.T * p.k;
  const int64_t total_rows = routed_rows + (p.has_shared ? p.T : 0);
  const moe_weights &w = *p.w;
  hipError_t err;
  if ((err = mark(p, MOE_STAGE_GEMM1, s)) != hipSuccess) return err;
  if (p.act_dtype == MOE_DTYPE_F32) {
    const dim3 g1((unsigned)((p.inter + 255) / 256), (unsigned)total_rows);
    hipLaunchKernelGGL(expert_up_f32, g1, dim3(256), 0, s, (const float *)p.x, p.sorted_tok,
                       p.sorted_slot, p.route_idx, p.offsets, p.E, p.k, routed_rows, total_rows,
                       p.dim, p.inter, (const float *)w.w_gate, (const float *)w.w_up,
                       (const float *)w.sh_gate, (const float *)w.sh_up, p.swiglu_limit,
                       (float *)p.h);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = mark(p, MOE_STAGE_GEMM2, s)) != hipSuccess) return err;
    const dim3 g2((unsigned)((p.dim + 255) / 256), (unsigned)total_rows);
    hipLaunchKernelGGL(expert_down_f32, g2, dim3(256), 0, s, (const float *)p.h, p.sorted_tok,
                       p.sorted_slot, p.route_idx, p.route_w, p.offsets, p.E, p.k, routed_rows,
                       total_rows, p.dim, p.inter, (const float *)w.w_down,
                       (const float *)w.sh_down, (float *)p.yrows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = mark(p, MOE_STAGE_COMBINE, s)) != hipSuccess) return err;
    hipLaunchKernelGGL(combine_f32, dim3((unsigned)p.T), dim3(256), 0, s,
                       (const float *)p.yrows, p.inverse, p.k, p.dim,
                       p.has_shared ? routed_rows : (int64_t)-1, (float *)p.y);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return mark(p, MOE_STAGE_COUNT, s);
  }

  const int mb = p.tile_rows / 16;
  const bool fp4 = p.expert_dtype == MOE_DTYPE_FP4_E2M1;
  GemmArgs a = {};
  a.E = p.E;
  a.tiles = p.tiles;
  a.tile_count = p.tile_count;
  a.k = p.k;
  a.routed_rows = routed_rows;
  a.sorted_tok = p.sorted_tok;
  a.sorted_slot = p.sorted_slot;
  a.route_w = p.route_w;

  // GEMM1: gate|up + SwiGLU -> H
  a.A = (const bf16 *)p.x;
  a.a_rows = p.sorted_tok;
  a.K = p.dim;
  a.N = p.inter;
  a.B[0] = w.w_gate; a.B[1] = w.w_up;
  a.S[0] = w.s_gate; a.S[1] = w.s_up;
  a.SB[0] = (const bf16 *)w.sh_gate; a.SB[1] = (const bf16 *)w.sh_up;
  a.C = (bf16 *)p.h;
  a.limit = p.swiglu_limit;
  if (fp4) {
    if (p.n_shared_tiles > 0) {
      GemmArgs sh = a;
      sh.tile_begin = 0; sh.tile_end = p.n_shared_tiles;
      if ((err = gemm_launch(2, false, mb, sh, p.n_shared_tiles, s)) != hipSuccess) return err;
    }
    a.tile_begin = p.n_shared_tiles; a.tile_end = -1;
    if ((err = gemm_launch(2, true, mb, a, p.max_tiles - p.n_shared_tiles, s)) != hipSuccess)
      return err;
  } else {
    a.tile_begin = 0; a.tile_end = -1;
    if ((err = gemm_launch(2, false, mb, a, p.max_tiles, s)) != hipSuccess) return err;
  }

  // GEMM2: down * gate value -> Y rows
  if ((err = mark(p, MOE_STAGE_GEMM2, s)) != hipSuccess) return err;
  a.A = (const bf16 *)p.h;
  a.a_rows = nullptr;
  a.K = p.inter;
  a.N = p.dim;
  a.B[0] = w.w_down; a.B[1] = nullptr;
  a.S[0] = w.s_down; a.S[1] = nullptr;
  a.SB[0] = (const bf16 *)w.sh_down; a.SB[1] = nullptr;
  a.C = (bf16 *)p.yrows;
  if (fp4) {
    if (p.n_shared_tiles > 0) {
      GemmArgs sh = a;
      sh.tile_begin = 0; sh.tile_end = p.n_shared_tiles;
      if ((err = gemm_launch(1, false, mb, sh, p.n_shared_tiles, s)) != hipSuccess) return err;
    }
    a.tile_begin = p.n_shared_tiles; a.tile_end = -1;
    if ((err = gemm_launch(1, true, mb, a, p.max_tiles - p.n_shared_tiles, s)) != hipSuccess)
      return err;
  } else {
    a.tile_begin = 0; a.tile_end = -1;
    if ((err = gemm_launch(1, false, mb, a, p.max_tiles, s)) != hipSuccess) return err;
  }

  if ((err = mark(p, MOE_STAGE_COMBINE, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(combine_bf16, dim3((unsigned)p.T), dim3(256), 0, s, (const bf16 *)p.yrows,
                     p.inverse, p.k, p.dim, p.has_shared ? routed_rows : (int64_t)-1,
                     (bf16 *)p.y);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return mark(p, MOE_STAGE_COUNT, s);
}

}  // namespace moe
