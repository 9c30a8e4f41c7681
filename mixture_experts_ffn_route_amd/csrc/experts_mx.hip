// Routed experts on MXFP8 activations for gfx950: the activation quantiser and
// the grouped GEMMs on v_mfma_scale_f32_16x16x128_f8f6f4.
//
// "From One Giant FFN to 384 Tiny Experts", Ch.11.6: the experts are stored
// as FP4 (E2M1) in OCP MXFP4 1x32 sub-blocks and computed in FP8 (E4M3).  On
// this GPU the scaled MFMA takes both operands in OCP MX form, so the FP4
// codes and their E8M0 scales go to the matrix core as stored, and the
// activations entering a routed expert GEMM are quantised to MXFP8 (E4M3
// elements, one E8M0 scale per 32 inputs).  One MFMA covers 16 rows x 16
// columns x 128 inputs.  Operand layout (lane l, r = l % 16, q = l / 16):
//   A (E4M3, 32 bytes): row r, inputs 16q .. 16q+15 and 64+16q .. 64+16q+15
//   B (E2M1, 16 bytes): column r, inputs 32q .. 32q+31 (low nibble first)
//   B (E4M3, 32 bytes): column r, inputs as A's
//   scales: lane l gives the E8M0 scale of its row (A) / column (B) for the
//           32-input block q
//   D: column r, rows 4q .. 4q+3 (as the 16x16x32 form)
//
// Two grouped-GEMM forms:
//   grouped_gemm_mx     decode tiles (one 16-row block), FP4 weights: the
//                       pipeline of the bf16 tile (experts.hip) with 128-input
//                       stages -- activation rows and their scale words
//                       copied global -> LDS and read by every wave, FP4 codes
//                       and scales in a register ring, the waves splitting the
//                       columns;
//   grouped_gemm_mx_rs  tiles of 4 and more row blocks, and every FP8-weight
//                       tile: the waves split the rows and the weights pass
//                       through LDS (gemm_tile_mx_rs below); FP4 weights as
//                       stored or FP8 weights re-dequantised from them
//                       (redequant.hip).
// The down GEMM's input, H in MXFP8, comes from the gate|up epilogues of
// both forms directly (store_swiglu_mxfp8), encoded from the fp32 SwiGLU
// values.

#include "gemm.h"

namespace moe {
namespace {

// One thread per 32-input block (rows are contiguous, so block i of the
// flattened array is row i / (K/32)): shared exponent floor(log2(amax)) - 8
// clamped to [-127, 127] (0 for an all-zero block), codes of v / 2^X by the
// hardware E4M3 conversion (v_cvt_pk_fp8_f32: round to nearest, ties to even)
// after clamping to +-448, which is the saturating OCP encoding.
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const bf16 *src, int64_t nblk,
                                                             uint8_t *codes, uint8_t *scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  const bf16x8 *p = (const bf16x8 *)(src + i * 32);
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 w = p[c];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[8 * c + j] = (float)w[j];
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  int X = 0;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);                         // amax = f * 2^ex, f in [0.5, 1)
    X = ex - 1 - 8;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
  }
  scales[i] = (uint8_t)(X + 127);
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float q[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) q[b] = fminf(fmaxf(ldexpf(v[4 * j + b], -X), -448.f), 448.f);
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
    w[j] = (uint32_t)word;
  }
  u32x4 *o = (u32x4 *)(codes + i * 32);
  o[0] = u32x4{w[0], w[1], w[2], w[3]};
  o[1] = u32x4{w[4], w[5], w[6], w[7]};
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// dma16 with the nontemporal cache policy (CPol NT), for the gate|up weight
// stream: V4.1-Flash MXFP8 GEMM1 1.60 -> 1.55 ms, and the combine after it
// 0.145 -> 0.136 ms; the down GEMM's weights measured slower that way.
__device__ __forceinline__ void dma16_nt(const void *gsrc, void *lds_block) {
  __builtin_amdgcn_global_load_lds((MOE_GLOBAL void *)gsrc, (MOE_LDS void *)lds_block, 16, 0, 2);
}

// Maximum over the 16 lanes of a DPP row, left on each of them: quad permutes
// (1,0,3,2) and (2,3,0,1), then the half-row and row mirrors -- VALU lane
// moves that need no LDS crossbar and no wait.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
  return v;
}

// SwiGLU output rows straight to MXFP8, as the quantiser would encode them
// (from the fp32 values, not their bf16 rounding).  acc holds MW row blocks
// (the first is row block mb0 of the tile) x SC 16-column blocks of gate and
// of up, in the 16x16 MFMA accumulator layout: lane (r16, q) has column
// col0 + 16cb + r16 of rows 4q .. 4q+3.  A 32-column block of a row is column
// blocks 2c and 2c+1 of the 16 lanes that share the row (a DPP row), so its
// amax is a 16-lane reduction; lane r16 keeps the scale of block r16 and the
// lanes of a row store the slab's scales at once.  Every lane takes part in
// the reductions (rows past the tile hold finite padding values and are not
// stored).
template <int MW, int SC>
__device__ __forceinline__ void store_swiglu_mxfp8(const GemmArgs &g, const f32x4 (&gate)[MW][SC],
                                                   const f32x4 (&up)[MW][SC], int mb0, int row0,
                                                   int rows, int col0, int N, int r16, int q) {
  static_assert(SC % 2 == 0 && SC <= 32, "whole MX blocks per slab");
  const float L = g.limit;
  const int64_t NS = N / 32;
#pragma unroll
  for (int m = 0; m < MW; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (mb0 + m) * 16 + q * 4 + i;
      const int64_t R = row0 + row;
      uint8_t *qrow = g.Cq + R * N + col0 + r16;
      int my_sc = 0;
#pragma unroll
      for (int c = 0; c < SC / 2; ++c) {
        const float v0 = swiglu_pair(gate[m][2 * c][i], up[m][2 * c][i], L);
        const float v1 = swiglu_pair(gate[m][2 * c + 1][i], up[m][2 * c + 1][i], L);
        const float amax = row16_max(fmaxf(fabsf(v0), fabsf(v1)));
        int X = 0;
        if (amax > 0.f) {
          int ex;
          frexpf(amax, &ex);                   // amax = f * 2^ex, f in [0.5, 1)
          X = ex - 1 - 8;
          X = X < -127 ? -127 : (X > 127 ? 127 : X);
        }
        if (r16 == c) my_sc = X + 127;
        const float q0 = fminf(fmaxf(ldexpf(v0, -X), -448.f), 448.f);
        const float q1 = fminf(fmaxf(ldexpf(v1, -X), -448.f), 448.f);
        const int word = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        if (row < rows) {
          qrow[32 * c] = (uint8_t)word;
          qrow[32 * c + 16] = (uint8_t)(word >> 8);
        }
      }
      if (row < rows && r16 < SC / 2) g.Csc[R * NS + col0 / 32 + r16] = (uint8_t)my_sc;
    }
}

// One decode tile on the scaled MFMA: MBE 16-row blocks, NB weight matrices,
// NCB 16-column blocks per wave and matrix.  SLOT = bytes per LDS ring slot
// (activation units, then the scale region).
template <int WAVES, int NB, int NCB, int MBE, int NS, int SLOT>
__device__ __forceinline__ void gemm_tile_mx(const GemmArgs &g, const TileCtx &t, uint8_t *Ls) {
  constexpr int BK = 128;                  // inputs per stage
  constexpr int UNIT = 1024;               // activation copy unit: 8 rows x 128 bytes
  constexpr int NFRAG = MBE * 2;
  constexpr int NFW = (NFRAG + WAVES - 1) / WAVES;
  constexpr int NSU = (MBE * 16 + 63) / 64; // scale copy units: 64 rows x 4 bytes
  constexpr int NSW = (NSU + WAVES - 1) / WAVES;
  constexpr int SCALE_OFF = NFW * WAVES * UNIT;
  constexpr int NBV = NB * NCB * 3;        // two 8-byte code loads + one scale byte
  constexpr int VM_PER_STAGE = NFW + NSW + NBV;
  constexpr int CH = MBE < 2 ? MBE : 2;    // row blocks per MFMA chunk (A operands are 8 VGPRs)
  static_assert(NS >= 2, "pipeline needs two stages");
  static_assert((NS - 2) * VM_PER_STAGE <= 63, "vmcnt holds 6 bits");
  static_assert(SCALE_OFF + NSW * WAVES * 256 <= SLOT, "ring slot too small");
  static_assert(MBE % CH == 0, "row blocks come in whole chunks");
  constexpr int ISSUE_PER_CHUNK = (VM_PER_STAGE + (MBE / CH) - 1) / (MBE / CH);

  const int lane = t.lane, wave = t.wave, r16 = lane & 15, q = lane >> 4;
  const int K = t.K, N = t.N, rows = t.rows, row0 = t.row0, col0 = t.col0;
  const int KS = K / 32;                   // scales per activation row

  float row_w[NB == 1 ? MBE : 1][4];
  if constexpr (NB == 1) {
#pragma unroll
    for (int m = 0; m < MBE; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int r = m * 16 + q * 4 + i;
        r = r < rows ? r : rows - 1;
        const int64_t R = row0 + r;
        row_w[m][i] = R < g.routed_rows ? g.sorted_w[R < g.routed_rows ? R : 0] : 1.f;
      }
  }

  // activation units (as the bf16 tile: lane l of unit (m, h) takes row
  // 16m + 8h + l/8, 16-byte chunk (l%8) ^ (l/8))
  const uint8_t *asrc[NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    const int f0 = wave + WAVES * i;
    const int f = f0 < NFRAG ? f0 : 0;
    int r = (f >> 1) * 16 + (f & 1) * 8 + (lane >> 3);
    r = r < rows ? r : rows - 1;
    const int64_t src = g.a_rows ? g.a_rows[row0 + r] : (int64_t)(row0 + r);
    asrc[i] = g.Aq + src * K + 16 * ((lane & 7) ^ (lane >> 3));
  }
  // scale units: lane l of unit u fetches the 4 scale bytes (one stage) of row 64u + l
  const uint8_t *ssrc[NSW];
#pragma unroll
  for (int i = 0; i < NSW; ++i) {
    const int u0 = wave + WAVES * i;
    const int u = u0 < NSU ? u0 : 0;
    int r = u * 64 + lane;
    r = r < rows ? r : rows - 1;
    const int64_t src = g.a_rows ? g.a_rows[row0 + r] : (int64_t)(row0 + r);
    ssrc[i] = g.Asc + src * KS;
  }
  // MFMA operand reads: row r16 (unit half r16/8, row-in-unit rr), chunks q
  // and 4 + q; scale byte of row r16, block q
  const int rr = r16 & 7;
  const int a_lo = (r16 >> 3) * UNIT + (rr * 8 + (q ^ rr)) * 16;
  const int a_hi = (r16 >> 3) * UNIT + (rr * 8 + ((4 + q) ^ rr)) * 16;
  const int a_sc = SCALE_OFF + r16 * 4 + q;

  // FP4 weights: column n = col0 + 16cb + r16, inputs 32q .. 32q+31 of the
  // stage.  Rows layout: bytes 16q.. of the stage's 64 (pieces +0, +8);
  // tiled: 64-input tile 2*stage + q/2, lane indices 2(q%2)*16 + r16 and +16
  // (pieces +0, +128).
  const bool tiled = g.tiled != 0;
  const int64_t bst = tiled ? 1024 : 64;
  const int64_t pst = tiled ? 128 : 8;
  const int64_t sst = tiled ? 64 : 4;
  const uint8_t *bptr[NB][NCB];
  const uint8_t *sptr[NB][NCB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int64_t n = col0 + cb * 16 + r16;
      const int64_t nb = n >> 4;
      const uint8_t *mat = (const uint8_t *)g.B[b] + (int64_t)t.grp * N * (K / 2);
      const uint8_t *smat = g.S[b] + (int64_t)t.grp * N * KS;
      if (tiled) {
        bptr[b][cb] = mat + (nb * (K / 64) + (q >> 1)) * 512 + ((2 * (q & 1)) * 16 + r16) * 8;
        sptr[b][cb] = smat + (nb * (K / 64) + (q >> 1)) * 32 + r16 * 2 + (q & 1);
      } else {
        bptr[b][cb] = mat + n * (K / 2) + 16 * q;
        sptr[b][cb] = smat + n * KS + q;
      }
    }

  f32x4 acc[MBE][NB][NCB];
#pragma unroll
  for (int m = 0; m < MBE; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[m][b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint2 fq[NS][NB][NCB][2];
  uint32_t sq[NS][NB][NCB];
  const int nst = K / BK;

  auto issue_op = [&](int SL, int ST, int qq) {
    uint8_t *slot = Ls + SL * SLOT;
    if (qq < NFW) {
      dma16(asrc[qq] + (int64_t)ST * BK, slot + (wave + WAVES * qq) * UNIT);
    } else if (qq < NFW + NSW) {
      const int i = qq - NFW;
      dma4(ssrc[i] + ST * 4, slot + SCALE_OFF + (wave + WAVES * i) * 256);
    } else {
      const int r = qq - NFW - NSW, bc = r / 3, w = r - bc * 3, b = bc / NCB, cb = bc - b * NCB;
      if (w < 2)
        fq[SL][b][cb][w] = *(const uint2 *)(bptr[b][cb] + ST * bst + w * pst);
      else
        sq[SL][b][cb] = sptr[b][cb][ST * sst];
    }
  };
  auto issue_stage = [&](int SL, int ST) {
#pragma unroll
    for (int qq = 0; qq < VM_PER_STAGE; ++qq) issue_op(SL, ST, qq);
  };

  const int last = nst - 1;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue_stage(p, p < last ? p : last);

  // one stage from ring slot p, refilling the slot stage st-1 used with
  // stage st+NS-1 (clamped) spread over the MFMA chunks; a scheduling barrier
  // after each chunk keeps the loads there
  auto compute_stage = [&](int p, int st) {
    const int nslot = (p + NS - 1) % NS;
    const int nx = st + NS - 1 < last ? st + NS - 1 : last;
    const uint8_t *abase = Ls + p * SLOT;
    i32x8 bv[NB][NCB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint2 c0 = fq[p][b][cb][0], c1 = fq[p][b][cb][1];
        bv[b][cb] = i32x8{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y, 0, 0, 0, 0};
      }
#pragma unroll
    for (int mc = 0; mc < MBE; mc += CH) {
      i32x8 av[CH];
      int sa[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int mo = (mc + j) * 2 * UNIT;
        const u32x4 lo = *(const u32x4 *)(abase + mo + a_lo);
        const u32x4 hi = *(const u32x4 *)(abase + mo + a_hi);
        av[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sa[j] = abase[a_sc + (mc + j) * 64];
      }
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            acc[mc + j][b][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                av[j], bv[b][cb], acc[mc + j][b][cb], 0, 4, 0, sa[j], 0,
                (int)sq[p][b][cb]);
      const int chunk = mc / CH;
#pragma unroll
      for (int j = 0; j < ISSUE_PER_CHUNK; ++j) {
        const int qq = chunk * ISSUE_PER_CHUNK + j;
        if (qq < VM_PER_STAGE) issue_op(nslot, nx, qq);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // whole groups of NS stages without a branch (the compiler then counts the
  // loads the MFMAs wait for exactly), then the last nst % NS with full waits
  const int nfull = nst - nst % NS;
  for (int s0 = 0; s0 < nfull; s0 += NS) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT((NS - 2) * VM_PER_STAGE));
      __builtin_amdgcn_s_barrier();
      compute_stage(p, s0 + p);
    }
  }
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) {
    if (nfull + p < nst) {
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
      __builtin_amdgcn_s_barrier();
      compute_stage(p, nfull + p);
    }
  }
  __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));

  // ---- epilogue (accumulator layout of the 16x16 MFMA forms) ----
  if constexpr (NB == 2) {
    if constexpr (NCB % 2 == 0) {
      if (g.Cq) {
        f32x4 gate[MBE][NCB], up[MBE][NCB];
#pragma unroll
        for (int m = 0; m < MBE; ++m)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            gate[m][cb] = acc[m][0][cb];
            up[m][cb] = acc[m][1][cb];
          }
        store_swiglu_mxfp8<MBE, NCB>(g, gate, up, 0, row0, rows, col0, N, r16, q);
        return;
      }
    }
    const float L = g.limit;
#pragma unroll
    for (int m = 0; m < MBE; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + q * 4 + i;
        if (row < rows) {
          bf16 *crow = g.C + (int64_t)(row0 + row) * N + col0 + r16;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            crow[cb * 16] = (bf16)swiglu_pair(acc[m][0][cb][i], acc[m][1][cb][i], L);
        }
      }
  } else {
#pragma unroll
    for (int m = 0; m < MBE; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + q * 4 + i;
        if (row < rows) {
          bf16 *crow = g.C + (int64_t)(row0 + row) * N + col0 + r16;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) crow[cb * 16] = (bf16)(acc[m][0][cb][i] * row_w[m][i]);
        }
      }
  }
}

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// LDS of the row-split kernel: NSA activation slots and NSB weight slots,
// each its own object so the compiler can tell copies into one slot from
// reads of another (and adds no waits between them).
struct MxRing {
  uint8_t *a[4];
  uint8_t *b[8];
  uint8_t *bs;    // FP8 weights: the slab's block scales, [matrix][block][stage]
};

// Most 128-input stages the FP8-weight form keeps block scales for (K <= 32768).
constexpr int kMxF8MaxStages = 256;

// 128-column FP8 weight blocks in a slab of SC 16-column blocks.
constexpr int mx_f8_blocks(int sc) { return sc > 8 ? sc / 8 : 1; }

// Row-split tile for tiles of 4 and more row blocks.  Each wave owns MW =
// MBE/WAVES row blocks and every column of the slab: SC 16-column blocks of
// each of the NB matrices.  Per stage of 128 inputs each wave copies its own
// activation rows into LDS (full 128-byte lines, 8 rows per copy, the 16-byte
// chunk of lane l at (l%8) ^ (l/8) so the reads are conflict-free) and reads
// them back once; the FP4 weight fragments (16 columns x 128 inputs, 1 KB)
// and the scales are copied once per workgroup and read by every wave.  So
// an activation byte crosses LDS once, not once per column wave.
//
// Two copy rings: activations (from L2) NSA stages deep, weights (streamed
// from HBM) NSB stages deep.  Each stage issues its activation copies first
// and its weight copies last: the in-order count then lets the wait for a
// stage's activations leave the far weight copies in flight.
//
// FP8 weights (F8, re-dequantised from FP4 by moe_redequant_fp8): a fragment
// is 2 KB stored in operand order -- lane (c, q) reads 16 bytes at
// (q*16 + c)*16 and 16 at 1024 + (q*16 + c)*16 -- and is copied as two 1 KB
// units; its scale is the E8M0 byte of its 128 x 128 block: a slab covers
// SC / 8 such blocks of each matrix (at least one: narrower slabs lie inside
// one), and their bytes for every stage of the tile are kept in LDS.
//
// LDS form of an FP4 weight fragment.  Tiled weights: the 16-byte chunk (t, g, p)
// of the stage (64-input tile t, 8-byte group g, column pair p) is stored at
// chunk t*32 + (g%2)*16 + (g/2)*8 + p, so the two 8-byte pieces a lane needs
// sit 256 bytes apart and 32 lanes of a read touch all 64 banks once.  Row
// weights: chunk (column r, 32-input part c) at chunk 16c + r, the lane's 16
// bytes contiguous.  Weight scales: the 64 bytes of the stage in the global
// order (tiled: [tile][column][block%2], rows: [column][block]).
template <int WAVES, int NB, int SC, int MBE, int NSA, int NSB, int A_MAX, bool F8>
__device__ __forceinline__ void gemm_tile_mx_rs(const GemmArgs &g, const TileCtx &t,
                                                const MxRing &ring) {
  constexpr int BK = 128;
  constexpr int MW = MBE / WAVES;                  // row blocks of one wave
  constexpr int NFR = NB * SC;                     // weight fragments per stage
  constexpr int FRAG = F8 ? 2048 : 1024;           // bytes per fragment in LDS
  constexpr int NBU = (NFR * (FRAG / 1024) + WAVES - 1) / WAVES;   // 1 KB copies per wave
  constexpr int NSG = F8 ? 0 : (NFR + 3) / 4;      // weight-scale copies (4 fragments each)
  constexpr int NSU = (NSG + WAVES - 1) / WAVES;   // per wave
  constexpr int AS_OFF = A_MAX * 2 * 1024;         // activation slot: units, then scales
  constexpr int S_OFF = NBU * WAVES * 1024;        // weight slot: fragments, then scales
  constexpr int VMA = 2 * MW + 1;                  // activation copies per stage
  constexpr int VMB = NBU + NSU;                   // weight copies per stage
  constexpr int VM = VMA + VMB;
  // copies issued after the last one a stage needs: its activations (first in
  // their issuing stage) when the weight ring is deeper, else its weights
  constexpr int WAIT = (NSB > NSA ? VMB : 0) + (NSA - 2) * VM;
  constexpr int GROUP = NSA * NSB / gcd_int(NSA, NSB);
  constexpr int ISSUE_PER_FRAG = (VM + NFR - 1) / NFR;
  static_assert(MBE % WAVES == 0 && MBE <= A_MAX, "row blocks split evenly over the waves");
  static_assert(MW * 16 <= 64, "one activation-scale copy per wave");
  static_assert(NSA >= 2 && NSA <= 4 && NSB >= NSA && NSB <= 8, "ring depths");
  static_assert(WAIT <= 63, "vmcnt holds 6 bits");

  const int lane = t.lane, wave = t.wave, r16 = lane & 15, q = lane >> 4;
  const int K = t.K, N = t.N, rows = t.rows, row0 = t.row0, col0 = t.col0;
  const int KS = K / 32;
  const int mb0 = wave * MW;
  const bool tiled = g.tiled != 0;

  // down GEMM: lane l holds the gate value of this wave's row l (a wave owns
  // at most 64 rows); the epilogue fetches each stored row's value by a lane
  // shuffle, so the main loop keeps one register for them.
  float my_w = 1.f;
  if constexpr (NB == 1) {
    const int r = mb0 * 16 + lane;
    const int64_t R = row0 + r;
    if (lane < MW * 16 && r < rows && R < g.routed_rows) my_w = g.sorted_w[R];
  }

  // activation copies of this wave: unit (m, h) = rows 16(mb0+m) + 8h .. +7
  const uint8_t *asrc[MW][2];
#pragma unroll
  for (int m = 0; m < MW; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int r = (mb0 + m) * 16 + h * 8 + (lane >> 3);
      r = r < rows ? r : rows - 1;
      const int64_t src = g.a_rows ? g.a_rows[row0 + r] : (int64_t)(row0 + r);
      asrc[m][h] = g.Aq + src * K + 16 * ((lane & 7) ^ (lane >> 3));
    }
  // activation-scale copy: lane l fetches the stage's 4 scale bytes of row
  // 16*mb0 + l (lanes past the wave's rows repeat its last row)
  const uint8_t *assrc;
  {
    int r = mb0 * 16 + (lane < MW * 16 ? lane : MW * 16 - 1);
    r = r < rows ? r : rows - 1;
    const int64_t src = g.a_rows ? g.a_rows[row0 + r] : (int64_t)(row0 + r);
    assrc = g.Asc + src * KS;
  }
  // weight copies: unit u = wave + WAVES*i is fragment (u / SC, u % SC)
  // (FP8: half u % 2 of fragment u / 2)
  const int64_t bst = F8 ? 2048 : (tiled ? 1024 : 64);
  const int64_t sst = tiled ? 64 : 4;
  const uint8_t *bsrc[NBU];
#pragma unroll
  for (int i = 0; i < NBU; ++i) {
    const int u0 = wave + WAVES * i;
    const int u = u0 < NFR * (FRAG / 1024) ? u0 : 0;
    const int f = F8 ? u >> 1 : u;
    const int b = f / SC, cb = f - b * SC;
    const int64_t nb = (col0 >> 4) + cb;
    if (F8) {
      const uint8_t *mat = (const uint8_t *)g.B[b] + (int64_t)t.grp * N * K;
      bsrc[i] = mat + nb * (K / 128) * 2048 + (u & 1) * 1024 + lane * 16;
      continue;
    }
    const uint8_t *mat = (const uint8_t *)g.B[b] + (int64_t)t.grp * N * (K / 2);
    if (tiled) {
      const int tt = lane >> 5, gg = ((lane >> 3) & 1) * 2 + ((lane >> 4) & 1), pp = lane & 7;
      bsrc[i] = mat + nb * (K / 64) * 512 + tt * 512 + gg * 128 + pp * 16;
    } else {
      bsrc[i] = mat + (nb * 16 + (lane & 15)) * (K / 2) + 16 * (lane >> 4);
    }
  }
  const uint8_t *ssrc[NSU > 0 ? NSU : 1];
#pragma unroll
  for (int i = 0; i < NSU; ++i) {
    const int j0 = wave + WAVES * i;
    const int j = j0 < NSG ? j0 : 0;
    const int f0 = j * 4 + (lane >> 4);
    const int f = f0 < NFR ? f0 : 0;
    const int b = f / SC, cb = f - b * SC;
    const int64_t nb = (col0 >> 4) + cb;
    const uint8_t *smat = g.S[b] + (int64_t)t.grp * N * KS;
    ssrc[i] = tiled ? smat + nb * (K / 64) * 32 + 4 * (lane & 15)
                    : smat + (nb * 16 + (lane & 15)) * KS;
  }
  // this lane's reads: activation chunks q and 4+q of row r16 of a row block,
  // its scale byte, a weight fragment's two 8-byte pieces and scale byte
  const int rr = r16 & 7;
  const int a_lo = (r16 >> 3) * 1024 + (rr * 8 + (q ^ rr)) * 16;
  const int a_hi = (r16 >> 3) * 1024 + (rr * 8 + ((4 + q) ^ rr)) * 16;
  const int a_sc = AS_OFF + wave * 256 + r16 * 4 + q;
  const int boff0 = F8 ? (q * 16 + r16) * 16
                 : tiled ? ((q >> 1) * 32 + (q & 1) * 8 + (r16 >> 1)) * 16 + (r16 & 1) * 8
                         : (q * 16 + r16) * 16;
  const int boff1 = boff0 + (F8 ? 1024 : tiled ? 256 : 8);
  const int soff = S_OFF + (tiled ? (q >> 1) * 32 + r16 * 2 + (q & 1) : r16 * 4 + q);

  f32x4 acc[MW][NB][SC];
#pragma unroll
  for (int m = 0; m < MW; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int cb = 0; cb < SC; ++cb) acc[m][b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nst = K / BK;
  const int last = nst - 1;
  constexpr int BPS = mx_f8_blocks(SC);           // FP8 weight blocks per slab and matrix
  static_assert(!F8 || SC % 8 == 0 || SC < 8, "a slab covers whole 128-column blocks");
  if constexpr (F8) {
    // block scales of this slab (BPS 128-row blocks of each matrix) for every stage
    const int br0 = col0 >> 7;
    for (int i = threadIdx.x; i < NB * BPS * nst; i += WAVES * 64) {
      const int bj = i / nst, st = i - bj * nst, b = bj / BPS, j = bj - b * BPS;
      ring.bs[i] = g.S[b][((int64_t)t.grp * (N / 128) + br0 + j) * nst + st];
    }
    __syncthreads();
  }
  // copy qq of a stage: activations of stage STA into slot SA (qq < VMA),
  // then weights of stage STB into slot SB
  auto issue_op = [&](int SA, int STA, int SB, int STB, int qq) {
    if (qq < 2 * MW) {
      const int m = qq >> 1, h = qq & 1;
      dma16(asrc[m][h] + (int64_t)STA * BK, ring.a[SA] + ((mb0 + m) * 2 + h) * 1024);
    } else if (qq == 2 * MW) {
      dma4(assrc + 4 * STA, ring.a[SA] + AS_OFF + wave * 256);
    } else if (qq < VMA + NBU) {
      const int i = qq - VMA;
      if constexpr (NB == 2)
        dma16_nt(bsrc[i] + STB * bst, ring.b[SB] + (wave + WAVES * i) * 1024);
      else
        dma16(bsrc[i] + STB * bst, ring.b[SB] + (wave + WAVES * i) * 1024);
    } else {
      const int i = qq - VMA - NBU;
      dma4(ssrc[i] + STB * sst, ring.b[SB] + S_OFF + (wave + WAVES * i) * 256);
    }
  };
  // prologue: virtual stages -(NSB-1) .. -1 issue what the steady state would
  // (weights of stage s+NSB-1, activations of stage s+NSA-1 once s >= 1-NSA)
#pragma unroll
  for (int v = 0; v < NSB - 1; ++v) {
    const int sb = v, sa = v - (NSB - NSA);
    const int stb = sb < last ? sb : last;
    if (sa >= 0) {
      const int sta = sa < last ? sa : last;
#pragma unroll
      for (int qq = 0; qq < VMA; ++qq) issue_op(sa % NSA, sta, 0, 0, qq);
    }
#pragma unroll
    for (int qq = VMA; qq < VM; ++qq) issue_op(0, 0, sb % NSB, stb, qq);
  }

  // stage with activations in slot pa and weights in slot pb; refills
  // activations of stage nxa into slot (pa+NSA-1)%NSA and weights of stage nxb
  // into slot (pb+NSB-1)%NSB, interleaved with the MFMAs
  auto compute_stage = [&](int st, int pa, int pb, int nxa, int nxb) {
    const int na = (pa + NSA - 1) % NSA, nb = (pb + NSB - 1) % NSB;
    const uint8_t *aslot = ring.a[pa];
    const uint8_t *bslot = ring.b[pb];
    i32x8 av[MW];
    int sa[MW];
#pragma unroll
    for (int m = 0; m < MW; ++m) {
      const uint8_t *u = aslot + (mb0 + m) * 2048;
      const u32x4 lo = *(const u32x4 *)(u + a_lo);
      const u32x4 hi = *(const u32x4 *)(u + a_hi);
      av[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      sa[m] = aslot[a_sc + m * 64];
    }
    // weight fragments are read one ahead of their MFMAs
    i32x8 bv[2];
    int sbv[2];
    int sblk[NB * BPS];
    if constexpr (F8) {
#pragma unroll
      for (int bj = 0; bj < NB * BPS; ++bj) sblk[bj] = ring.bs[bj * nst + st];
    }
    auto read_frag = [&](int f, int buf) {
      if constexpr (F8) {
        const u32x4 lo = *(const u32x4 *)(bslot + f * FRAG + boff0);
        const u32x4 hi = *(const u32x4 *)(bslot + f * FRAG + boff1);
        bv[buf] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sbv[buf] = sblk[(f / SC) * BPS + (f % SC) / (SC / BPS)];
      } else {
        const uint2 lo = *(const uint2 *)(bslot + f * FRAG + boff0);
        const uint2 hi = *(const uint2 *)(bslot + f * FRAG + boff1);
        bv[buf] = i32x8{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y, 0, 0, 0, 0};
        sbv[buf] = bslot[soff + f * 64];
      }
    };
    read_frag(0, 0);
#pragma unroll
    for (int f = 0; f < NFR; ++f) {
      if (f + 1 < NFR) read_frag(f + 1, (f + 1) & 1);
      const int b = f / SC, cb = f - b * SC;
#pragma unroll
      for (int m = 0; m < MW; ++m)
        acc[m][b][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av[m], bv[f & 1], acc[m][b][cb], 0, F8 ? 0 : 4, 0, sa[m], 0, sbv[f & 1]);
#pragma unroll
      for (int j = 0; j < ISSUE_PER_FRAG; ++j) {
        const int qq = f * ISSUE_PER_FRAG + j;
        if (qq < VM) issue_op(na, nxa, nb, nxb, qq);
      }
      // keep the copies spread: the scheduler otherwise sinks them below the
      // stage's MFMAs (V4.1-Flash MXFP8 gate|up 1.56 -> 1.46 ms, FP8-weight
      // gate|up 2.01 -> 1.74 ms once pinned)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // whole groups of GROUP stages (a multiple of both ring depths): no branch
  // inside, a fixed number of copies in flight (stages past the end re-copy
  // the last one)
  const int nfull = nst - nst % GROUP;
  for (int s0 = 0; s0 < nfull; s0 += GROUP) {
#pragma unroll
    for (int p = 0; p < GROUP; ++p) {
      const int st = s0 + p;
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT(WAIT));
      __builtin_amdgcn_s_barrier();
      compute_stage(st, p % NSA, p % NSB, st + NSA - 1 < last ? st + NSA - 1 : last,
                    st + NSB - 1 < last ? st + NSB - 1 : last);
    }
  }
  // the last nst % GROUP stages, with full waits (they still refill, since a
  // stage's copies are issued NSA-1 / NSB-1 stages ahead)
#pragma unroll
  for (int p = 0; p < GROUP - 1; ++p) {
    const int st = nfull + p;
    if (st < nst) {
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
      __builtin_amdgcn_s_barrier();
      compute_stage(st, p % NSA, p % NSB, st + NSA - 1 < last ? st + NSA - 1 : last,
                    st + NSB - 1 < last ? st + NSB - 1 : last);
    }
  }
  __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));

  if constexpr (NB == 2) {
    const float L = g.limit;
    auto swiglu = [&](float gv, float uv) { return swiglu_pair(gv, uv, L); };
    if (g.Cq) {
      f32x4 gate[MW][SC], up[MW][SC];
#pragma unroll
      for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int cb = 0; cb < SC; ++cb) {
          gate[m][cb] = acc[m][0][cb];
          up[m][cb] = acc[m][1][cb];
        }
      store_swiglu_mxfp8<MW, SC>(g, gate, up, mb0, row0, rows, col0, N, r16, q);
      return;
    }
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (mb0 + m) * 16 + q * 4 + i;
        if (row < rows) {
          bf16 *crow = g.C + (int64_t)(row0 + row) * N + col0 + r16;
#pragma unroll
          for (int cb = 0; cb < SC; ++cb)
            crow[cb * 16] = (bf16)swiglu(acc[m][0][cb][i], acc[m][1][cb][i]);
        }
      }
  } else {
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = __shfl(my_w, m * 16 + q * 4 + i);   // every lane takes part
        const int row = (mb0 + m) * 16 + q * 4 + i;
        if (row < rows) {
          bf16 *crow = g.C + (int64_t)(row0 + row) * N + col0 + r16;
#pragma unroll
          for (int cb = 0; cb < SC; ++cb) crow[cb * 16] = (bf16)(acc[m][0][cb][i] * w);
        }
      }
  }
}

template <int WAVES, int MB>
constexpr int gemm_mx_rs_aslot_bytes() { return MB * 2 * 1024 + WAVES * 256; }

template <int WAVES, int NB, int SC, bool F8>
constexpr int gemm_mx_rs_bslot_bytes() {
  constexpr int NFR = NB * SC;
  constexpr int NBU = (NFR * (F8 ? 2 : 1) + WAVES - 1) / WAVES;
  constexpr int NSU = F8 ? 0 : ((NFR + 3) / 4 + WAVES - 1) / WAVES;
  return NBU * WAVES * 1024 + NSU * WAVES * 256;
}

// Row-split kernel: the tile height is taken as the smallest multiple of
// WAVES row blocks (and of 4) that holds the tile's rows, up to MB.
template <int WAVES, int NB, int SC, int MB, int NSA, int NSB, int WPE, bool F8>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void grouped_gemm_mx_rs(const GemmArgs g) {
  constexpr int SA = gemm_mx_rs_aslot_bytes<WAVES, MB>();
  constexpr int SB = gemm_mx_rs_bslot_bytes<WAVES, NB, SC, F8>();
  constexpr int STEP = WAVES > 4 ? WAVES : 4;
  static_assert(MB % STEP == 0, "tile height in whole steps");
  __shared__ __attribute__((aligned(1024))) uint8_t A0[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t A1[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t A2[NSA > 2 ? SA : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t A3[NSA > 3 ? SA : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t B0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t B1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t B2[NSB > 2 ? SB : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t B3[NSB > 3 ? SB : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t B4[NSB > 4 ? SB : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t B5[NSB > 5 ? SB : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t B6[NSB > 6 ? SB : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t B7[NSB > 7 ? SB : 1];
  __shared__ uint8_t BS[F8 ? NB * mx_f8_blocks(SC) * kMxF8MaxStages : 1];
  const MxRing ring{{A0, A1, A2, A3}, {B0, B1, B2, B3, B4, B5, B6, B7}, BS};
  int tile, slab;
  if (!gemm_work_item(g, &tile, &slab)) return;
  TileCtx t = gemm_tile_ctx(g, tile, slab, 1, SC * 16);
  t.col0 = slab * (SC * 16);                // every wave covers the whole slab
  const int nmb = (t.rows + 15) >> 4;
  if (MB <= STEP || nmb <= STEP)
    gemm_tile_mx_rs<WAVES, NB, SC, STEP, NSA, NSB, MB, F8>(g, t, ring);
  else if (MB <= 2 * STEP || nmb <= 2 * STEP)
    gemm_tile_mx_rs<WAVES, NB, SC, (MB < 2 * STEP ? MB : 2 * STEP), NSA, NSB, MB, F8>(g, t, ring);
  else if (MB <= 3 * STEP || nmb <= 3 * STEP)
    gemm_tile_mx_rs<WAVES, NB, SC, (MB < 3 * STEP ? MB : 3 * STEP), NSA, NSB, MB, F8>(g, t, ring);
  else
    gemm_tile_mx_rs<WAVES, NB, SC, MB, NSA, NSB, MB, F8>(g, t, ring);
}

template <int WAVES, int NB, int SC, int MB, int NSA, int NSB, int WPE, bool F8 = false>
hipError_t run_gemm_mx_rs(GemmArgs a, int max_tiles, hipStream_t s) {
  if (a.N % (SC * 16) || (a.Cq && (NB != 2 || !a.Csc))) return hipErrorInvalidValue;
  a.n_slabs = a.N / (SC * 16);
  const int64_t blocks = gemm_grid_blocks(a, max_tiles);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_mx_rs<WAVES, NB, SC, MB, NSA, NSB, WPE, F8>),
                     dim3((unsigned)blocks), dim3(WAVES * 64), 0, s, a);
  return hipGetLastError();
}

template <int WAVES, int NB, int NCB, int MB, int NS>
constexpr int gemm_mx_slot_bytes() {
  constexpr int NFW = (MB * 2 + WAVES - 1) / WAVES;
  constexpr int NSW = ((MB * 16 + 63) / 64 + WAVES - 1) / WAVES;
  return NFW * WAVES * 1024 + NSW * WAVES * 256;
}

// Decode-tile kernel.  WPE: waves per SIMD it is compiled for (2: 256
// registers per wave; 1: 512).
template <int WAVES, int NB, int NCB, int MB, int NS, int WPE>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void grouped_gemm_mx(const GemmArgs g) {
  static_assert(MB < MCH, "tiles of 4+ row blocks run in grouped_gemm_mx_rs");
  constexpr int SLOT = gemm_mx_slot_bytes<WAVES, NB, NCB, MB, NS>();
  __shared__ __attribute__((aligned(1024))) uint8_t Ls[NS * SLOT];
  int tile, slab;
  if (!gemm_work_item(g, &tile, &slab)) return;
  const TileCtx t = gemm_tile_ctx(g, tile, slab, WAVES, NCB * 16);
  gemm_tile_mx<WAVES, NB, NCB, MB, NS, SLOT>(g, t, Ls);
}

template <int WAVES, int NB, int NCB, int MB, int NS, int WPE>
hipError_t run_gemm_mx(GemmArgs a, int max_tiles, hipStream_t s) {
  a.n_slabs = a.N / (WAVES * NCB * 16);
  const int64_t blocks = gemm_grid_blocks(a, max_tiles);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_mx<WAVES, NB, NCB, MB, NS, WPE>), dim3((unsigned)blocks),
                     dim3(WAVES * 64), 0, s, a);
  return hipGetLastError();
}

// FP4 decode tiles (one row block): 8 waves splitting the columns.  Tiles of
// 4+ row blocks: the row-split kernel, 4 waves with the whole register file.
// Every slab re-reads the tile's activations, so the slabs are as wide as the
// accumulators allow: for tiles of up to 12 row blocks 128 columns of gate and
// of up, or 256 down columns (half that when the width does not divide).
template <int NB, int MB>
hipError_t run_gemm_mx_mb(GemmArgs a, int max_tiles, hipStream_t s) {
  if (a.b_fp8) {
    // FP8 weights (2 KB fragments): tiles of up to 12 row blocks take 128 gate|up
    // or 256 down columns per slab with a 2-stage activation ring and a
    // 3-stage weight ring (146 KB of LDS); taller tiles, or widths that do
    // not divide, half that with 3 + 3 stages.  Decode tiles run as 4-block
    // tiles.
    constexpr int SC8 = NB == 2 ? 4 : 8;
    if (a.N % (SC8 * 16) != 0 || a.K / 128 > kMxF8MaxStages) return hipErrorInvalidValue;
    if constexpr (MB <= 12) {
      if (a.N % (2 * SC8 * 16) == 0)
        return run_gemm_mx_rs<4, NB, 2 * SC8, (MB < 4 ? 4 : MB), 2, 3, 1, true>(a, max_tiles, s);
    }
    return run_gemm_mx_rs<4, NB, SC8, (MB < 4 ? 4 : MB), 3, 3, 1, true>(a, max_tiles, s);
  }
  if constexpr (MB >= 4) {
    constexpr int NARROW = NB == 2 ? 4 : 8;
    constexpr int WIDE = MB <= 12 ? 2 * NARROW : NARROW;
    // 2-stage activation ring, 3-stage weight ring (V4.1-Flash MXFP8 layer:
    // 2.61 -> 2.48 ms against 3 + 3; 3 + 4 and 2 + 4 measured in between)
    if (a.N % (WIDE * 16) == 0) return run_gemm_mx_rs<4, NB, WIDE, MB, 2, 3, 1>(a, max_tiles, s);
    return run_gemm_mx_rs<4, NB, NARROW, MB, 3, 3, 1>(a, max_tiles, s);
  } else {
    // decode tiles; gate|up with an MXFP8 output: two 16-column blocks of
    // each matrix per wave, so that every 32-column MX block of a row lies in
    // one wave (N % 128 == 0 on MXFP8 layers)
    if (a.Cq) {
      if (NB != 2 || !a.Csc || a.N % 128 != 0) return hipErrorInvalidValue;
      if (a.N % 256 == 0) return run_gemm_mx<8, 2, 2, MB, 3, 2>(a, max_tiles, s);
      return run_gemm_mx<4, 2, 2, MB, 3, 2>(a, max_tiles, s);
    }
    if (NB == 1 && a.N % 256 == 0) return run_gemm_mx<8, 1, 2, MB, 3, 2>(a, max_tiles, s);
    if (a.N % 128 == 0) return run_gemm_mx<8, NB, 1, MB, 3, 2>(a, max_tiles, s);
    return run_gemm_mx<4, NB, 1, MB, 3, 1>(a, max_tiles, s);     // N % 64 == 0
  }
}

template <int NB>
hipError_t run_gemm_mx_any(int mb, GemmArgs a, int max_tiles, hipStream_t s) {
  switch (mb) {
    case 1: return run_gemm_mx_mb<NB, 1>(a, max_tiles, s);
    case 4: return run_gemm_mx_mb<NB, 4>(a, max_tiles, s);
    case 8: return run_gemm_mx_mb<NB, 8>(a, max_tiles, s);
    case 12: return run_gemm_mx_mb<NB, 12>(a, max_tiles, s);
    case 16: return run_gemm_mx_mb<NB, 16>(a, max_tiles, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_mx(int nb, int mb, GemmArgs a, int max_tiles, hipStream_t s) {
  return nb == 2 ? run_gemm_mx_any<2>(mb, a, max_tiles, s) : run_gemm_mx_any<1>(mb, a, max_tiles, s);
}

hipError_t launch_quantize_mxfp8(const bf16 *src, int64_t rows, int K, uint8_t *codes,
                                 uint8_t *scales, hipStream_t s) {
  const int64_t nblk = rows * (K / 32);
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0,
                     s, src, nblk, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
