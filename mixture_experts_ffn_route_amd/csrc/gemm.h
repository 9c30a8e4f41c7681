// Definitions shared by the grouped-GEMM translation units (experts.hip:
// bf16 operands on v_mfma_f32_16x16x32_bf16; experts_mx.hip: MXFP8
// activations x FP4 weights on v_mfma_scale_f32_16x16x128_f8f6f4).
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

struct GemmArgs {
  const bf16 *A;             // activation rows [*, K]
  const uint8_t *Aq;         // MX form: E4M3 activation rows [*, K]
  const uint8_t *Asc;        // MX form: E8M0 scales [*, K/32]
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
  const float *sorted_w;     // one-matrix form: gate value of each permuted row
  int tiled;                 // B, S, SB in the tiled layout (moe_pack_weights)
  float *Cf;                 // one-matrix form: fp32 output instead of C, or null
  int n_shared_tiles;        // leading tiles of the range that are shared-expert tiles
  int64_t dense_rows;        // tiles == null: one group of this many rows, cut
  int dense_tile_rows;       //   into tiles of dense_tile_rows rows
  int64_t routed_rows;       // T * k: rows at or above this belong to the shared expert
  int b_fp8;                 // MX form: B is E4M3 in the FP8 expert layout and S its
                             //   128 x 128 block scales [E, N/128, K/128]
  uint8_t *Cq;               // two-matrix MX form: the SwiGLU output in MXFP8 instead
  uint8_t *Csc;              //   of C -- E4M3 codes [*, N], E8M0 scales [*, N/32] -- or null
};

#define MOE_LDS __attribute__((address_space(3)))
#define MOE_GLOBAL __attribute__((address_space(1)))

// 16-byte asynchronous global -> LDS copy: lane l's 16 bytes land at
// lds_block + 16*l (lds_block must be wave-uniform).  Completion is tracked by
// vmcnt like any vector load.
__device__ __forceinline__ void dma16(const void *gsrc, void *lds_block) {
  __builtin_amdgcn_global_load_lds((MOE_GLOBAL void *)gsrc, (MOE_LDS void *)lds_block, 16, 0, 0);
}

// s_waitcnt immediate for vmcnt(n) (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima,
// i.e. not waited on).
#define MOE_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Row blocks are processed in chunks of MCH (2 where MCH does not divide the
// tile body's block count): every pipeline stage is then straight-line code
// in which the LDS reads of a chunk issue back to back and the MFMAs of one
// chunk overlap the reads of the next.  A tile runs the body for its block
// count rounded up to an even number (bodies of 4, 6, 8, ... blocks: measured
// 3-6 % faster on the FP4 and hash layers than multiples of 4, whose padding
// blocks cost MFMA issue slots there).  Padding blocks read real rows (the
// tile's last row) and are never stored.
constexpr int MCH = 4;

struct TileCtx {
  int grp, row0, rows, col0, lane, wave, K, N;
  bool shared;
  bool reread;               // other tiles stream the same weights (several tiles of
                             // one expert, the shared expert, or the dense form)
};

// 4-byte form: lane l's 4 bytes land at lds_block + 4*l.
__device__ __forceinline__ void dma4(const void *gsrc, void *lds_block) {
  __builtin_amdgcn_global_load_lds((MOE_GLOBAL void *)gsrc, (MOE_LDS void *)lds_block, 4, 0, 0);
}

// Work item of this workgroup.  Workgroups are dealt round-robin to the 8
// XCDs (blockIdx & 7).  Shared-expert tiles (every one a full, compute-heavy
// tile) go to the XCDs in turn, all slabs of a tile on one XCD; the routed
// items are then split into 8 contiguous runs, so an expert's slabs share one
// XCD's L2.  Returns false for a surplus workgroup.
__device__ __forceinline__ bool gemm_work_item(const GemmArgs &g, int *tile_out, int *slab_out) {
  const int tend = g.tile_end >= 0 ? g.tile_end : *g.tile_count;
  const int nsh = g.n_shared_tiles;
  const int xcd = blockIdx.x & 7;
  const int64_t slot = blockIdx.x >> 3;
  const int sh_cnt = nsh > xcd ? (nsh - xcd + 7) >> 3 : 0;
  const int64_t sh_items = (int64_t)sh_cnt * g.n_slabs;
  if (slot < sh_items) {
    const int i = (int)(slot / g.n_slabs);
    *tile_out = g.tile_begin + xcd + 8 * i;
    *slab_out = (int)(slot - (int64_t)i * g.n_slabs);
    return true;
  }
  const int64_t routed = (int64_t)(tend - g.tile_begin - nsh) * g.n_slabs;
  const int64_t r_per = (routed + 7) >> 3;
  const int64_t r = slot - sh_items;
  if (r >= r_per) return false;
  const int64_t item = xcd * r_per + r;
  if (item >= routed) return false;
  const int64_t rt = item / g.n_slabs;
  *tile_out = g.tile_begin + nsh + (int)rt;
  *slab_out = (int)(item - rt * g.n_slabs);
  return true;
}

// Tile context of a work item; each wave owns `wave_cols` output columns.
__device__ __forceinline__ TileCtx gemm_tile_ctx(const GemmArgs &g, int tile, int slab,
                                                 int waves, int wave_cols) {
  TileCtx t;
  if (g.tiles) {
    t.grp = g.tiles[4 * tile];
    t.row0 = g.tiles[4 * tile + 1];
    t.rows = g.tiles[4 * tile + 2];
    t.reread = g.tiles[4 * tile + 3] > 1;
  } else {
    t.reread = true;
    t.grp = 0;
    t.row0 = tile * g.dense_tile_rows;
    const int64_t left = g.dense_rows - t.row0;
    t.rows = left < g.dense_tile_rows ? (int)left : g.dense_tile_rows;
  }
  t.shared = t.grp == g.E;
  t.K = g.K;
  t.N = g.N;
  t.lane = threadIdx.x & 63;
  t.wave = threadIdx.x >> 6;
  t.col0 = slab * (waves * wave_cols) + t.wave * wave_cols;
  return t;
}

// Grid of a launch: per XCD its share of the shared tiles, then an eighth of
// the rest (a static upper bound; surplus workgroups exit).
inline int64_t gemm_grid_blocks(const GemmArgs &a, int max_tiles) {
  const int64_t per_xcd = (int64_t)((a.n_shared_tiles + 7) / 8) * a.n_slabs +
                          ((int64_t)(max_tiles - a.n_shared_tiles) * a.n_slabs + 7) / 8;
  return 8 * per_xcd;
}

// MX launches (experts_mx.hip): routed FP4 experts on MXFP8 activations.
// With a.Cq set (gate|up only) the output is the MXFP8 form of the SwiGLU
// rows 0 .. a.routed_rows-1 (a.C is not written).
hipError_t launch_gemm_mx(int nb, int mb, GemmArgs a, int max_tiles, hipStream_t s);
// E4M3 codes + E8M0 scales (OCP MX, one scale per 32 inputs) of rows x K.
hipError_t launch_quantize_mxfp8(const bf16 *src, int64_t rows, int K, uint8_t *codes,
                                 uint8_t *scales, hipStream_t s);

}  // namespace moe
