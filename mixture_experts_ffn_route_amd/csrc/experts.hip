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
// the routed weights are read once per forward -- straight into registers in
// the MFMA operand layout, through an NS-deep register ring.  The gathered
// activation rows travel global -> LDS through asynchronous copies
// (global_load_lds_dwordx4) that land directly in the MFMA A-operand layout,
// in an NS-deep LDS ring shared by the waves.  MFMA is
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  FP4 weights are loaded
// as 16 codes + one E8M0 scale per lane per 64-input stage and expanded to
// bf16 in registers with v_cvt_scalef32_pk_bf16_fp4.
//
// The workgroup -> work item map is XCD aware: consecutive workgroups land on
// different XCDs, so each XCD is given a contiguous range of items (all
// slabs of the same tiles), and the gathered rows of an expert stay in that
// XCD's L2 while its slabs stream.

#include "gemm.h"

namespace moe {

// One tile: MBE row blocks (compile time), NB weight matrices (2: gate|up
// with the SwiGLU epilogue, 1: down with the gate-value epilogue), NCB
// 16-column blocks per wave and matrix, FP4 or bf16 weights, NS-deep load
// pipeline.  SLOT = bf16 elements per LDS ring slot.
//
// Stage = BK inputs.  Per stage each wave issues (a) its share of the tile's
// A fragments as asynchronous global->LDS copies -- fragment (row block m,
// k-step s) is 64 lanes x 16 bytes, row 16m + (lane & 15) of the gathered
// activations, so the LDS block already has the MFMA A-operand layout and the
// readers take 16 consecutive bytes per lane without bank conflicts -- and
// (b) its own weight columns as 16-byte loads into a register ring
// (bf16 weights: nontemporal where no other work item reads the same weight
// fragment -- V3 decode GEMM1 2.15 -> 1.96 ms, hash layer GEMM1 0.203 ->
// 0.199 ms and GEMM2 0.124 -> 0.119 ms; taller tiles whose weights other
// tiles stream too -- an expert cut into several tiles, the shared expert,
// the dense form -- run a body of their own with plain loads, so that the
// re-reads can still hit the caches).  Stage st
// is consumed NS-1 stages after it was issued; one vmcnt wait and one barrier
// per stage.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// 8 FP4 weight bytes, loaded nontemporal: every weight fragment is read by one
// work item (V4.1-Flash FP4 layer 3.85 -> 3.78 ms, the combine after it
// 0.144 -> 0.132 ms, from less of the cache taken by weights).
__device__ __forceinline__ uint2 fp4_stream_load(const uint8_t *p) {
  const u32x2 v = __builtin_nontemporal_load((const u32x2 *)p);
  return uint2{v[0], v[1]};
}

template <int WAVES, int NB, int NCB, int MBE, bool FP4, int NS, int SLOT, bool SH = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, const TileCtx &t, bf16 *As) {
  constexpr int BK = 64;                   // inputs per stage
  constexpr int SUBS = BK / 32;            // MFMA k-steps per stage
  constexpr int FRAG = 512;                // bf16 per 16x32 A fragment (1 KB)
  constexpr int NFRAG = MBE * SUBS;        // A fragments per stage
  constexpr int NFW = (NFRAG + WAVES - 1) / WAVES;
  constexpr int NQ = SUBS;                 // bf16: 16-byte weight loads per (matrix, block) per stage
  // weight-side vector memory ops per stage: bf16 one 16-byte load per k-step;
  // FP4 one 8-byte load (16 codes) plus one scale byte
  constexpr int NBV = NB * NCB * (FP4 ? 2 : NQ);
  constexpr int VM_PER_STAGE = NFW + NBV;          // every wave issues exactly this many
  constexpr int CH = MBE < MCH ? MBE : (MBE % MCH == 0 ? MCH : 2);
  static_assert(NS >= 2, "pipeline needs two stages");
  static_assert((NS - 2) * VM_PER_STAGE <= 63, "vmcnt holds 6 bits");
  static_assert(NFW * WAVES * FRAG <= SLOT, "ring slot too small");
  static_assert(MBE % CH == 0, "row blocks come in whole chunks");
  // refill ops issued after each MFMA chunk (all of them land within the stage)
  constexpr int ISSUE_PER_CHUNK = (VM_PER_STAGE + SUBS * (MBE / CH) - 1) / (SUBS * (MBE / CH));

  const int lane = t.lane, wave = t.wave, r16 = lane & 15, jq = lane >> 4;
  const int K = t.K, N = t.N, rows = t.rows, row0 = t.row0, col0 = t.col0;

  // down GEMM: the gate values of the tile's rows, loaded up front (the latency
  // hides under the main loop) and spread over the wave, lane l holding rows
  // l, l + 64, ...; the epilogue fetches each stored row's value by a lane
  // shuffle.  NWR registers instead of one per stored row (4 MBE).
  constexpr int NWR = NB == 1 ? (16 * MBE + 63) / 64 : 1;
  float my_w[NWR];
#pragma unroll
  for (int j = 0; j < NWR; ++j) {
    const int r = 64 * j + lane;
    const int64_t R = row0 + r;
    my_w[j] = (NB == 1 && r < rows && R < g.routed_rows) ? g.sorted_w[R] : 1.f;
  }

  // ---- activation copies.  A stage holds, per 16-row block m, two 1 KB
  // copy units h = 0, 1 of 8 rows x 64 inputs (each row one full 128-byte
  // line).  Lane l of unit (m, h) fetches row 16m + 8h + l/8, 8-input chunk
  // (l%8) ^ (l/8) (^ h for FP4), which lands at byte 16*l of the unit; this wave's units
  // are f = wave + WAVES*i (units past NFRAG re-read unit 0 into slots nobody
  // reads, so every wave issues NFW). ----
  static_assert(SUBS == 2, "two copy units per row block and stage");
  const bf16 *asrc[NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    const int f0 = wave + WAVES * i;
    const int f = f0 < NFRAG ? f0 : 0;
    const int m = f >> 1, h = f & 1;
    int r = m * 16 + 8 * h + (lane >> 3);
    r = r < rows ? r : rows - 1;
    const int64_t src = g.a_rows ? g.a_rows[row0 + r] : (int64_t)(row0 + r);
    asrc[i] = g.A + src * K + 8 * ((lane & 7) ^ (lane >> 3) ^ (FP4 ? h : 0));
  }
  // MFMA operand of k-step `sub`: row r16, 8-input chunk c of the stage.
  // bf16 keeps k = 32 sub + 8 jq (c = 4 sub + jq); FP4 uses k = 16 jq + 8 sub
  // (c = 2 jq + sub) so that each lane's 16 weight codes of a stage lie in one
  // 32-input scale block.  A and B use the same order, so the products are
  // unchanged.  The chunks of a row sit at position chunk ^ row (^ the unit
  // half h for FP4), which keeps each half-wave's 16-byte reads on distinct
  // LDS banks: on this GPU those banks follow address bits 4..8 with bit 10
  // (the unit half) folded into bit 8, and with the FP4 order the plain
  // chunk ^ row placement made lanes 0-7 and 16-23 collide (2-way conflict,
  // half of the FP4 GEMMs' LDS cycles by the bank-conflict counter).
  int aoff[SUBS];
#pragma unroll
  for (int sub = 0; sub < SUBS; ++sub) {
    const int c = FP4 ? (2 * jq + sub) : (4 * sub + jq);
    const int rr = r16 & 7;
    aoff[sub] = (r16 >> 3) * FRAG + (rr * 8 + (c ^ rr ^ (FP4 ? (r16 >> 3) : 0))) * 8;
  }

  // ---- weight pointers: this lane's operand of stage 0, plus the byte
  // strides between stages (bst), between the two 32-input halves of a bf16
  // stage (qst) and between the scale bytes of two FP4 stages (sst).  Row
  // layout: the operand is 8 (bf16) or 16 (FP4) inputs of row n; tiled layout:
  // lane `lane` of the tile's contiguous 1 KB / 512 B block. ----
  const uint8_t *bptr[NB][NCB];
  const uint8_t *sptr[NB][NCB];
  const bool tiled = g.tiled != 0;
  const int64_t bst = FP4 ? (tiled ? 512 : BK / 2) : (tiled ? SUBS * 1024 : BK * 2);
  const int64_t qst = tiled ? 1024 : 64;
  const int64_t sst = tiled ? 32 : BK / 32;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int64_t n = col0 + cb * 16 + r16;
      const int64_t nb = (col0 + cb * 16) >> 4;    // column block of this 16-wide slice
      if constexpr (FP4) {
        const int64_t K2 = K / 2, K32 = K / 32;
        const uint8_t *mat = (const uint8_t *)g.B[b] + (int64_t)t.grp * N * K2;
        const uint8_t *smat = g.S[b] + (int64_t)t.grp * N * K32;
        if (tiled) {
          bptr[b][cb] = mat + nb * (K / 64) * 512 + lane * 8;
          sptr[b][cb] = smat + nb * (K / 64) * 32 + r16 * 2 + (jq >> 1);
        } else {
          bptr[b][cb] = mat + n * K2 + jq * 8;
          sptr[b][cb] = smat + n * K32 + (jq >> 1);
        }
      } else {
        const bf16 *base = t.shared ? g.SB[b] : (const bf16 *)g.B[b] + (int64_t)t.grp * N * K;
        bptr[b][cb] = tiled ? (const uint8_t *)base + nb * (K / 32) * 1024 + lane * 16
                            : (const uint8_t *)(base + n * K + jq * 8);
        sptr[b][cb] = nullptr;
      }
    }

  f32x4 acc[MBE][NB][NCB];
#pragma unroll
  for (int m = 0; m < MBE; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[m][b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 bq[NS][NB][NCB][FP4 ? 1 : NQ];   // bf16 weight fragments
  uint2 fq[NS][NB][NCB];                 // FP4 codes (16 per lane per stage)
  uint32_t sq[NS][NB][NCB];              // FP4 scale bytes
  const int nst = K / BK;

  // Issue the q-th vector memory op of stage ST into ring slot SL (ops
  // 0..NFW-1: activation copies; then the weight loads).  Called with
  // indices that are constants after unrolling, so the branches fold.
  auto issue_op = [&](int SL, int ST, int q) {
    if (q < NFW) {
      dma16(asrc[q] + (int64_t)ST * BK, As + SL * SLOT + (wave + WAVES * q) * FRAG);
    } else if constexpr (FP4) {
      const int r = q - NFW, bc = r >> 1, b = bc / NCB, cb = bc - b * NCB;
      if ((r & 1) == 0)
        fq[SL][b][cb] = fp4_stream_load(bptr[b][cb] + ST * bst);
      else
        sq[SL][b][cb] = sptr[b][cb][ST * sst];
    } else {
      const int r = q - NFW, bc = r / NQ, qq = r - bc * NQ, b = bc / NCB, cb = bc - b * NCB;
      const u32x4 *src = (const u32x4 *)(bptr[b][cb] + ST * bst + qq * qst);
      bq[SL][b][cb][qq] = (MBE == 1 || !SH) ? __builtin_nontemporal_load(src) : *src;
    }
  };
  auto issue_stage = [&](int SL, int ST) {
#pragma unroll
    for (int q = 0; q < VM_PER_STAGE; ++q) issue_op(SL, ST, q);
  };

  // prologue: stages 0 .. NS-2 (stage indices past the end re-read the
  // last stage: same addresses, so they hit in L2 and cost no HBM bytes)
  const int last = nst - 1;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue_stage(p, p < last ? p : last);

  // One pipeline stage: stage st from ring slot p; refills the slot freed by
  // stage st-1 with stage st+NS-1 (clamped to the last stage), spread over
  // the MFMA chunks, so a load that waits for queue space stalls the wave
  // while issued MFMAs keep the matrix unit busy.  A scheduling barrier after
  // each chunk keeps the loads there: the scheduler otherwise sinks them
  // below the stage's MFMAs (shorter live ranges), a stage less of prefetch.
  // (All refills right after the barrier measured slower: hash GEMM1
  // 0.20 -> 0.35 ms, FP4 GEMM1 1.96 -> 2.10 ms.)
  auto compute_stage = [&](int p, int st) {
    const int nslot = (p + NS - 1) % NS;
    const int nx = st + NS - 1 < last ? st + NS - 1 : last;
    const bf16 *abase = As + p * SLOT;
#pragma unroll
    for (int sub = 0; sub < SUBS; ++sub) {
      bf16x8 bf[NB][NCB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if constexpr (FP4) {
            const unsigned word = sub == 0 ? fq[p][b][cb].x : fq[p][b][cb].y;
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
#pragma unroll
      for (int mc = 0; mc < MBE; mc += CH) {
        bf16x8 a[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j)
          a[j] = *(const bf16x8 *)(abase + aoff[sub] + (mc + j) * 2 * FRAG);
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[mc + j][b][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  a[j], bf[b][cb], acc[mc + j][b][cb], 0, 0, 0);
        const int chunk = sub * (MBE / CH) + mc / CH;
#pragma unroll
        for (int j = 0; j < ISSUE_PER_CHUNK; ++j) {
          const int q = chunk * ISSUE_PER_CHUNK + j;
          if (q < VM_PER_STAGE) issue_op(nslot, nx, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Whole groups of NS stages: no branch inside, and every stage issues
  // exactly one stage of copies, so the number of vector memory ops between
  // a stage's issue and its use is the constant (NS-1) * VM_PER_STAGE and
  // every wait is a compile-time vmcnt.  The compiler also waits by itself
  // for the loads whose registers an MFMA reads; it can count those exactly
  // only when every path through the loop issues the same memory ops (a
  // `st < nst` branch around the compute made it wait for all outstanding
  // ops at the start of most stages, draining the ring).
  const int nfull = nst - nst % NS;
  for (int s0 = 0; s0 < nfull; s0 += NS) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      // stages st+1 .. st+NS-2 may stay in flight
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT((NS - 2) * VM_PER_STAGE));
      __builtin_amdgcn_s_barrier();     // every wave's copies for st landed; st-1 fully read
      compute_stage(p, s0 + p);
    }
  }
  // the last nst % NS stages, with full waits
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) {
    if (nfull + p < nst) {
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
      __builtin_amdgcn_s_barrier();
      compute_stage(p, nfull + p);
    }
  }
  // drain the trailing copies before the workgroup's LDS can be reused
  __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));

  // ---- epilogue ----
  // fp32 output (router logits on this kernel's dense form): direct stores
  if (NB == 1 && g.Cf) {
#pragma unroll
    for (int m = 0; m < MBE; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + jq * 4 + i;
        const float w = __shfl(my_w[m >> 2], row & 63);   // every lane takes part
        if (row < rows) {
          const int64_t o = (int64_t)(row0 + row) * N + col0 + r16;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) g.Cf[o + cb * 16] = acc[m][0][cb][i] * w;
        }
      }
    return;
  }
  // bf16 output, staged through the (now idle) LDS ring: every wave writes its
  // bf16 results into a row-major [rows][slab] tile, then the workgroup stores
  // whole rows with 16-byte stores, full cache lines, instead of a 2-byte
  // store per value in the accumulator layout (lane = one column of four
  // rows: 32-byte row segments).  Measured 1-4 % faster per GEMM (V4.1-Flash
  // FP4 layer 3.53 -> 3.42 ms, 2-gram hash layer 0.427 -> 0.409 ms).  Rows are
  // staged in chunks of RC that fit the ring; a 16-byte pad per staged row
  // spreads the four row groups of a write over distinct banks.
  constexpr int SW = WAVES * NCB * 16;               // slab columns
  constexpr int STRIDE = SW + 8;                     // bf16 per staged row
  constexpr int RC0 = NS * SLOT / STRIDE / 16 * 16;
  constexpr int RC = RC0 < MBE * 16 ? RC0 : MBE * 16;
  constexpr int NCHUNK = (MBE * 16 + RC - 1) / RC;
  constexpr int CPR = SW / 8;                        // 16-byte pieces per row
  constexpr int NT = WAVES * 64;
  constexpr int ITER = (RC * CPR + NT - 1) / NT;
  static_assert(RC >= 16 && RC % 16 == 0, "ring holds at least one row block");
  const int slab0 = col0 - wave * NCB * 16;
  const float L = g.limit;
  // every wave's copies have landed (each waited above) and every wave is
  // done reading the ring
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NCHUNK; ++c) {
#pragma unroll
    for (int m = c * RC / 16; m < (c + 1) * RC / 16 && m < MBE; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + jq * 4 + i;
        bf16 *srow = As + (row - c * RC) * STRIDE + wave * NCB * 16 + r16;
        if constexpr (NB == 2) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            srow[cb * 16] = (bf16)swiglu_pair(acc[m][0][cb][i], acc[m][1][cb][i], L);
        } else {
          // row / 64 = m / 4 for every lane; every lane takes part in the shuffle
          const float w = __shfl(my_w[m >> 2], row & 63);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) srow[cb * 16] = (bf16)(acc[m][0][cb][i] * w);
        }
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = it * NT + (int)threadIdx.x;
      const int rl = idx / CPR, pc = idx - rl * CPR;
      const int row = c * RC + rl;
      if (idx < RC * CPR && row < rows)
        *(u32x4 *)(g.C + (int64_t)(row0 + row) * N + slab0 + pc * 8) =
            *(const u32x4 *)(As + rl * STRIDE + pc * 8);
    }
    if (c + 1 < NCHUNK) __syncthreads();
  }
}

// The same tile on v_mfma_f32_32x32x16_bf16 (bf16 weights), for tiles of two
// or more row blocks.  One 32x32x16 instruction does the work of two
// 16x16x32 ones, and a stream of them keeps the matrix pipe 99 % busy where
// 16x16x32 reaches 57 % (MFMA-only probe, 8 waves per SIMD); each A operand
// read from LDS also feeds twice the flops.  The grouped GEMMs are not bound
// by the pipe, though: this form measured level with gemm_tile on most
// shapes, and gemm_launch uses it only where it was faster.  Operand layout
// (lane l, r = l % 32, h = l / 32): A row r, B column r, 8 inputs each
// (which 8 of a k-step's 16 is free as long as A and B agree); D 16 floats,
// column r, rows 8(e/4) + 4h + e%4 of the 32-row block.
//
// Here NCB counts 32-column blocks per wave and MBE 16-row blocks (even: the
// MFMA takes 32-row blocks).  The activation copies are those of gemm_tile
// (a 1 KB unit = 8 rows x 64 inputs, XOR-swizzled chunks); k-step s of a
// stage reads 16-byte chunk 2s + h of the 64-input row.  Weights: per lane,
// matrix, 32-column block and stage four 16-byte loads, k-step s from the
// 16 x 32 tile (column block r / 16, inputs 32(s/2) ..) at tile lane
// (r % 16) + 16(2(s%2) + h), i.e. inputs 16s + 8h .. of column r; the row
// layout gives the same inputs.  Nontemporal unless other tiles stream the
// same weights (SH), as in gemm_tile.
template <int WAVES, int NB, int NCB, int MBE, int NS, int SLOT, int LDSE, bool SH = false>
__device__ __forceinline__ void gemm_tile32(const GemmArgs &g, const TileCtx &t, bf16 *As) {
  constexpr int BK = 64;                   // inputs per stage
  constexpr int KS = BK / 16;              // MFMA k-steps per stage
  constexpr int FRAG = 512;                // bf16 per 1 KB copy unit
  static_assert(MBE % 2 == 0, "whole 32-row blocks");
  constexpr int M32 = MBE / 2;
  constexpr int NFRAG = MBE * 2;           // copy units per stage
  constexpr int NFW = (NFRAG + WAVES - 1) / WAVES;
  constexpr int NBV = NB * NCB * KS;       // weight loads per stage
  constexpr int VM_PER_STAGE = NFW + NBV;
  constexpr int CH = M32 % 4 == 0 ? 4 : (M32 % 2 == 0 ? 2 : 1);
  constexpr int NCHK = KS * (M32 / CH);    // MFMA chunks per stage
  constexpr int ISSUE_PER_CHUNK = (VM_PER_STAGE + NCHK - 1) / NCHK;
  static_assert(NS >= 2, "pipeline needs two stages");
  static_assert((NS - 2) * VM_PER_STAGE <= 63, "vmcnt holds 6 bits");
  static_assert(NFW * WAVES * FRAG <= SLOT, "ring slot too small");

  const int lane = t.lane, wave = t.wave, r32 = lane & 31, h = lane >> 5;
  const int K = t.K, N = t.N, rows = t.rows, row0 = t.row0, col0 = t.col0;

  constexpr int NWR = NB == 1 ? (16 * MBE + 63) / 64 : 1;
  float my_w[NWR];
#pragma unroll
  for (int j = 0; j < NWR; ++j) {
    const int r = 64 * j + lane;
    const int64_t R = row0 + r;
    my_w[j] = (NB == 1 && r < rows && R < g.routed_rows) ? g.sorted_w[R] : 1.f;
  }

  // activation copies: unit f = wave + WAVES*i holds rows 8f .. 8f+7, row
  // 8f + j at bytes 128j .. of the unit, its 16-byte chunk c at position
  // c ^ j ^ x(f), where x(f) = bit 1 of f (units 2, 3 of each 32-row block).
  // A k-step's read (lane = row r32 of a 32-row block, half h = chunk 2s + h)
  // then takes distinct LDS banks in each half-wave: on this GPU the banks of
  // a 16-byte read are set by address bits 4..8 with bit 10 folded into bit 8,
  // so units 0 and 2 (1 and 3), 2 KB apart, fall on the same banks unless
  // their chunks are permuted apart.  Without x(f) the reads take twice the
  // LDS cycles (bank-conflict counter: 44 % of the V3 down GEMM's LDS time).
  const bf16 *asrc[NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    const int f0 = wave + WAVES * i;
    const int f = f0 < NFRAG ? f0 : 0;
    int r = 8 * f + (lane >> 3);
    r = r < rows ? r : rows - 1;
    const int64_t src = g.a_rows ? g.a_rows[row0 + r] : (int64_t)(row0 + r);
    asrc[i] = g.A + src * K + 8 * ((lane & 7) ^ (lane >> 3) ^ ((f >> 1) & 1));
  }
  int aoff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int c = 2 * s + h;
    const int rr = r32 & 7;
    aoff[s] = (r32 >> 3) * FRAG + (rr * 8 + (c ^ rr ^ ((r32 >> 4) & 1))) * 8;
  }

  // weight pointers of stage 0 and the byte offsets of a stage (bst) and of
  // k-step q inside a stage (qoff)
  const uint8_t *bptr[NB][NCB];
  const bool tiled = g.tiled != 0;
  const int64_t bst = tiled ? 2048 : BK * 2;
  int qoff[KS];
#pragma unroll
  for (int q = 0; q < KS; ++q) qoff[q] = tiled ? (q >> 1) * 1024 + (q & 1) * 512 : 32 * q;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int64_t n = col0 + cb * 32 + r32;
      const int64_t nb = n >> 4;               // 16-column block of this lane's column
      const bf16 *base = t.shared ? g.SB[b] : (const bf16 *)g.B[b] + (int64_t)t.grp * N * K;
      bptr[b][cb] = tiled ? (const uint8_t *)base + nb * (K / 32) * 1024 + ((r32 & 15) + 16 * h) * 16
                          : (const uint8_t *)(base + n * K + h * 8);
    }

  f32x16 acc[M32][NB][NCB];
#pragma unroll
  for (int m = 0; m < M32; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][b][cb][e] = 0.f;

  u32x4 bq[NS][NB][NCB][KS];             // weight operands
  const int nst = K / BK;

  auto issue_op = [&](int SL, int ST, int q) {
    if (q < NFW) {
      dma16(asrc[q] + (int64_t)ST * BK, As + SL * SLOT + (wave + WAVES * q) * FRAG);
    } else {
      const int r = q - NFW, bc = r / KS, qq = r - bc * KS, b = bc / NCB, cb = bc - b * NCB;
      const u32x4 *src = (const u32x4 *)(bptr[b][cb] + ST * bst + qoff[qq]);
      bq[SL][b][cb][qq] = SH ? *src : __builtin_nontemporal_load(src);
    }
  };
  auto issue_stage = [&](int SL, int ST) {
#pragma unroll
    for (int q = 0; q < VM_PER_STAGE; ++q) issue_op(SL, ST, q);
  };

  const int last = nst - 1;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue_stage(p, p < last ? p : last);

  // one stage from ring slot p, refilling the slot of stage st-1 with stage
  // st+NS-1 between the MFMA chunks (as in gemm_tile).  The A operands of
  // each chunk are read from LDS while the previous chunk's MFMAs run: with
  // one wave per SIMD nothing else covers the LDS latency.
  auto compute_stage = [&](int p, int st) {
    const int nslot = (p + NS - 1) % NS;
    const int nx = st + NS - 1 < last ? st + NS - 1 : last;
    const bf16 *abase = As + p * SLOT;
    auto read_a = [&](int s, int mc, bf16x8 *a) {
#pragma unroll
      for (int j = 0; j < CH; ++j)
        a[j] = *(const bf16x8 *)(abase + aoff[s] + (mc + j) * 4 * FRAG);
    };
    bf16x8 a[2][CH];
    read_a(0, 0, a[0]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mc = 0; mc < M32; mc += CH) {
        const int chunk = s * (M32 / CH) + mc / CH;
        const int cur = chunk & 1;
        // next chunk's A operands (none after the stage's last chunk)
        if (chunk + 1 < NCHK) {
          const int s1 = mc + CH < M32 ? s : s + 1;
          const int mc1 = mc + CH < M32 ? mc + CH : 0;
          read_a(s1, mc1, a[cur ^ 1]);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[mc + j][b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  a[cur][j], __builtin_bit_cast(bf16x8, bq[p][b][cb][s]), acc[mc + j][b][cb],
                  0, 0, 0);
#pragma unroll
        for (int j = 0; j < ISSUE_PER_CHUNK; ++j) {
          const int q = chunk * ISSUE_PER_CHUNK + j;
          if (q < VM_PER_STAGE) issue_op(nslot, nx, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

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

  const float L = g.limit;
  // epilogue: bf16 rows staged through the ring as in gemm_tile (32-row
  // chunks; lane r32 writes column r32 of its block, the two lane halves
  // rows 4 apart, which the 16-byte row pad puts on distinct banks)
  constexpr int SW = WAVES * NCB * 32;
  constexpr int STRIDE = SW + 8;
  constexpr int RC0 = LDSE / STRIDE / 32 * 32;
  constexpr int RC = RC0 < MBE * 16 ? RC0 : MBE * 16;
  constexpr int NCHUNK = (MBE * 16 + RC - 1) / RC;
  constexpr int CPR = SW / 8;
  constexpr int NT = WAVES * 64;
  constexpr int ITER = (RC * CPR + NT - 1) / NT;
  static_assert(RC >= 32 && RC % 32 == 0, "ring holds at least one 32-row block");
  const int slab0 = col0 - wave * NCB * 32;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NCHUNK; ++c) {
#pragma unroll
    for (int m = c * RC / 32; m < (c + 1) * RC / 32 && m < M32; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        bf16 *srow = As + (row - c * RC) * STRIDE + wave * NCB * 32 + r32;
        if constexpr (NB == 2) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            srow[cb * 32] = (bf16)swiglu_pair(acc[m][0][cb][e], acc[m][1][cb][e], L);
        } else {
          // rows of block m lie in [32m, 32m + 32): row / 64 = m / 2 for every lane
          const float w = __shfl(my_w[m >> 1], row & 63);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) srow[cb * 32] = (bf16)(acc[m][0][cb][e] * w);
        }
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = it * NT + (int)threadIdx.x;
      const int rl = idx / CPR, pc = idx - rl * CPR;
      const int row = c * RC + rl;
      if (idx < RC * CPR && row < rows)
        *(u32x4 *)(g.C + (int64_t)(row0 + row) * N + slab0 + pc * 8) =
            *(const u32x4 *)(As + rl * STRIDE + pc * 8);
    }
    if (c + 1 < NCHUNK) __syncthreads();
  }
}

template <int WAVES, int NB, int NCB, int MB, bool FP4, int NS>
constexpr int gemm_slot_elems() {
  constexpr int SUBS = 2;
  return ((MB * SUBS + WAVES - 1) / WAVES) * WAVES * 512;
}

// Grouped GEMM kernel: one workgroup per (tile, slab) work item; MB is the
// tallest tile (in 16-row blocks) of this launch.
// Waves per SIMD the kernel is scheduled for: the tall tiles keep their
// accumulators in one wave per SIMD (the compiler then spends registers on
// latency hiding instead of chasing occupancy it cannot reach); the short
// decode tiles and 8-wave workgroups run two per SIMD.
template <int WAVES, int MB>
constexpr int gemm_waves_per_simd() { return (MB >= 8 && WAVES == 4) ? 1 : 2; }

template <int WAVES, int NB, int NCB, int MB, bool FP4, int NS>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(gemm_waves_per_simd<WAVES, MB>(),
                                   gemm_waves_per_simd<WAVES, MB>())))
void grouped_gemm(const GemmArgs g) {
  constexpr int SLOT = gemm_slot_elems<WAVES, NB, NCB, MB, FP4, NS>();
  __shared__ __attribute__((aligned(1024))) bf16 As[NS * SLOT];

  int tile, slab;
  if (!gemm_work_item(g, &tile, &slab)) return;
  const TileCtx t = gemm_tile_ctx(g, tile, slab, WAVES, NCB * 16);
  const int nmb = (t.rows + 15) >> 4;

  if constexpr (MB < MCH) {
    gemm_tile<WAVES, NB, NCB, MB, FP4, NS, SLOT>(g, t, As);
  } else if (!FP4 && (t.shared || t.reread)) {
    // tiles whose weights other tiles stream too (an expert of several tiles,
    // the shared expert, the dense form): plain weight loads (see above).
    // Such tiles are full height but for the last, which is often a short
    // remainder (an expert of 600 rows in 256-row tiles leaves 88, the
    // shared expert's 4096 rows in 192-row tiles leave 64): it takes a 4- or
    // 8-block body, not MB blocks of MFMAs on padding rows.
    const int n2 = (nmb + 1) / 2 * 2;
    if (MB > 4 && n2 <= 4)
      gemm_tile<WAVES, NB, NCB, (MB > 4 ? 4 : MB), FP4, NS, SLOT, true>(g, t, As);
    else if (MB > 8 && n2 <= 8)
      gemm_tile<WAVES, NB, NCB, (MB > 8 ? 8 : MB), FP4, NS, SLOT, true>(g, t, As);
    else
      gemm_tile<WAVES, NB, NCB, MB, FP4, NS, SLOT, true>(g, t, As);
  } else {
    const int n2 = (nmb + 1) / 2 * 2;
    if (n2 <= 4 || MB <= 4)
      gemm_tile<WAVES, NB, NCB, (MB < 4 ? MB : 4), FP4, NS, SLOT>(g, t, As);
    else if (n2 <= 6 || MB <= 6)
      gemm_tile<WAVES, NB, NCB, (MB < 6 ? MB : 6), FP4, NS, SLOT>(g, t, As);
    else if (n2 <= 8 || MB <= 8)
      gemm_tile<WAVES, NB, NCB, (MB < 8 ? MB : 8), FP4, NS, SLOT>(g, t, As);
    else if (n2 <= 10 || MB <= 10)
      gemm_tile<WAVES, NB, NCB, (MB < 10 ? MB : 10), FP4, NS, SLOT>(g, t, As);
    else if (n2 <= 12 || MB <= 12)
      gemm_tile<WAVES, NB, NCB, (MB < 12 ? MB : 12), FP4, NS, SLOT>(g, t, As);
    else if (n2 <= 14 || MB <= 14)
      gemm_tile<WAVES, NB, NCB, (MB < 14 ? MB : 14), FP4, NS, SLOT>(g, t, As);
    else
      gemm_tile<WAVES, NB, NCB, MB, FP4, NS, SLOT>(g, t, As);
  }
}

// The 32x32x16 grouped GEMM: as grouped_gemm, with tile bodies of 2, 4, 6,
// ... 16-row blocks.  Workgroups whose accumulators and weight ring take
// more than 192 of a lane's registers run one wave per SIMD (512 registers).
template <int WAVES, int NB, int NCB, int MB, int NS>
constexpr int gemm32_waves_per_simd() {
  return WAVES >= 8 ? 2 : ((MB / 2) * NB * NCB * 16 + NS * NB * NCB * 16 > 192 ? 1 : 2);
}

template <int WAVES, int NB, int NCB, int MB, int NS>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(gemm32_waves_per_simd<WAVES, NB, NCB, MB, NS>(),
                                   gemm32_waves_per_simd<WAVES, NB, NCB, MB, NS>())))
void grouped_gemm32(const GemmArgs g) {
  constexpr int SLOT = gemm_slot_elems<WAVES, NB, NCB, MB, false, NS>();
  // the copy ring, and at least 32 staged output rows for the epilogue
  constexpr int EPI = 32 * (WAVES * NCB * 32 + 8);
  constexpr int LDSE = NS * SLOT > EPI ? NS * SLOT : EPI;
  __shared__ __attribute__((aligned(1024))) bf16 As[LDSE];
  static_assert(MB % 2 == 0, "whole 32-row blocks");

  int tile, slab;
  if (!gemm_work_item(g, &tile, &slab)) return;
  const TileCtx t = gemm_tile_ctx(g, tile, slab, WAVES, NCB * 32);
  const int n2 = ((t.rows + 15) >> 4) + 1 & ~1;   // row blocks rounded up to even

  if (t.shared || t.reread) {
    // plain weight loads; a short last tile takes a short body (as above)
    if (MB > 4 && n2 <= 4)
      gemm_tile32<WAVES, NB, NCB, (MB > 4 ? 4 : MB), NS, SLOT, LDSE, true>(g, t, As);
    else if (MB > 8 && n2 <= 8)
      gemm_tile32<WAVES, NB, NCB, (MB > 8 ? 8 : MB), NS, SLOT, LDSE, true>(g, t, As);
    else
      gemm_tile32<WAVES, NB, NCB, MB, NS, SLOT, LDSE, true>(g, t, As);
  } else if (n2 <= 2 || MB <= 2) {
    gemm_tile32<WAVES, NB, NCB, 2, NS, SLOT, LDSE>(g, t, As);
  } else if (n2 <= 4 || MB <= 4) {
    gemm_tile32<WAVES, NB, NCB, (MB < 4 ? MB : 4), NS, SLOT, LDSE>(g, t, As);
  } else if (n2 <= 6 || MB <= 6) {
    gemm_tile32<WAVES, NB, NCB, (MB < 6 ? MB : 6), NS, SLOT, LDSE>(g, t, As);
  } else if (n2 <= 8 || MB <= 8) {
    gemm_tile32<WAVES, NB, NCB, (MB < 8 ? MB : 8), NS, SLOT, LDSE>(g, t, As);
  } else if (n2 <= 10 || MB <= 10) {
    gemm_tile32<WAVES, NB, NCB, (MB < 10 ? MB : 10), NS, SLOT, LDSE>(g, t, As);
  } else if (n2 <= 12 || MB <= 12) {
    gemm_tile32<WAVES, NB, NCB, (MB < 12 ? MB : 12), NS, SLOT, LDSE>(g, t, As);
  } else if (n2 <= 14 || MB <= 14) {
    gemm_tile32<WAVES, NB, NCB, (MB < 14 ? MB : 14), NS, SLOT, LDSE>(g, t, As);
  } else {
    gemm_tile32<WAVES, NB, NCB, MB, NS, SLOT, LDSE>(g, t, As);
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
// One workgroup per token with one lane per 8-column chunk (dim/8 lanes
// rounded up to whole waves, at most 1024; wider rows loop).  The token's k
// permuted rows (and its shared row) are looked up first; then every lane
// issues all k+1 16-byte loads of its chunk before adding them in slot order,
// shared row last (a dropped pair, inverse = -1, contributes nothing).
// Y is read once and y written once, so both go through nontemporal
// accesses (0.114 -> 0.102 ms at the V3 prefill shape).
template <int KMAX>
__global__ __launch_bounds__(1024) void combine_bf16(const bf16 *__restrict__ Y,
                                                     const int32_t *__restrict__ inverse,
                                                     int k, int dim, int64_t shared_base,
                                                     bf16 *__restrict__ y) {
  const int64_t t = blockIdx.x;
  int64_t row[KMAX + 1];
  bool use[KMAX + 1];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int r = j < k ? inverse[t * k + j] : -1;
    use[j] = r >= 0;
    row[j] = r >= 0 ? r : 0;
  }
  use[KMAX] = shared_base >= 0;
  row[KMAX] = shared_base >= 0 ? shared_base + t : 0;
  for (int c = threadIdx.x * 8; c < dim; c += blockDim.x * 8) {
    bf16x8 v[KMAX + 1];
#pragma unroll
    for (int j = 0; j <= KMAX; ++j)
      v[j] = __builtin_nontemporal_load((const bf16x8 *)(Y + row[j] * dim + c));
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j <= KMAX; ++j)
      if (use[j]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += (float)v[j][i];
      }
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)acc[i];
    __builtin_nontemporal_store(o, (bf16x8 *)(y + t * dim + c));
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
  // MXFP8 tiles stop at 12 row blocks: the row-split kernel then holds a
  // 128-column slab of each matrix in registers
  const int cap = cfg.act_quant == MOE_ACT_QUANT_MXFP8 ? 192 : 256;
  for (int mb : kTileMB)
    if (16.0 * mb >= want) return 16 * mb < cap ? 16 * mb : cap;
  return cap;
}

// Whether a configuration fits the hardware: the in-flight vector memory ops
// must fit vmcnt's 6 bits and the copy ring the 160 KB of LDS.
template <int WAVES, int NB, int NCB, int MB, bool FP4, int NS>
constexpr bool gemm_cfg_fits() {
  constexpr int SUBS = 2;
  constexpr int NFW = (MB * SUBS + WAVES - 1) / WAVES;
  constexpr int NBV = NB * NCB * 2;
  return (NS - 2) * (NFW + NBV) <= 63 && NS * NFW * WAVES * 1024 <= 160 * 1024;
}

template <int WAVES, int NB, int NCB, int MB, bool FP4, int NS>
static hipError_t run_gemm(const GemmArgs &a, int max_tiles, hipStream_t s) {
  if constexpr (!gemm_cfg_fits<WAVES, NB, NCB, MB, FP4, NS>()) {
    return hipErrorInvalidValue;
  } else {
  const int64_t blocks = gemm_grid_blocks(a, max_tiles);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm<WAVES, NB, NCB, MB, FP4, NS>), dim3((unsigned)blocks),
                     dim3(WAVES * 64), 0, s, a);
  return hipGetLastError();
  }
}

// Launch configuration: waves per workgroup, 16-column blocks per wave and
// matrix, pipeline depth.  Chosen per (matrix count, weight format, tile
// height) from sweeps on MI355X at the V3 prefill / decode, hash and
// V4.1-Flash shapes; the first entry whose column slab divides N is used.
struct GemmCfg { int waves, ncb, ns; };

// The 32x32x16 kernel (NCB in 32-column blocks): fits when the in-flight
// vector memory ops fit vmcnt and the copy ring the LDS.
template <int WAVES, int NB, int NCB, int MB, int NS>
constexpr bool gemm32_cfg_fits() {
  constexpr int NFW = (MB * 2 + WAVES - 1) / WAVES;
  constexpr int NBV = NB * NCB * 4;
  return MB % 2 == 0 && (NS - 2) * (NFW + NBV) <= 63 && NS * NFW * WAVES * 1024 <= 160 * 1024;
}

template <int WAVES, int NB, int NCB, int MB, int NS>
static hipError_t run_gemm32(const GemmArgs &a, int max_tiles, hipStream_t s) {
  if constexpr (!gemm32_cfg_fits<WAVES, NB, NCB, MB, NS>()) {
    return hipErrorInvalidValue;
  } else {
    const int64_t blocks = gemm_grid_blocks(a, max_tiles);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((grouped_gemm32<WAVES, NB, NCB, MB, NS>), dim3((unsigned)blocks),
                       dim3(WAVES * 64), 0, s, a);
    return hipGetLastError();
  }
}

template <int WAVES, int NB, int NCB, int NS>
static hipError_t run_gemm32_mb(int mb, const GemmArgs &a, int max_tiles, hipStream_t s) {
  switch (mb) {
    case 4: return run_gemm32<WAVES, NB, NCB, 4, NS>(a, max_tiles, s);
    case 8: return run_gemm32<WAVES, NB, NCB, 8, NS>(a, max_tiles, s);
    case 12: return run_gemm32<WAVES, NB, NCB, 12, NS>(a, max_tiles, s);
    default: return hipErrorInvalidValue;
  }
}

template <int WAVES, int NB, int NCB, bool FP4, int NS>
static hipError_t run_gemm_mb(int mb, const GemmArgs &a, int max_tiles, hipStream_t s) {
  switch (mb) {
    case 1: return run_gemm<WAVES, NB, NCB, 1, FP4, NS>(a, max_tiles, s);
    case 4: return run_gemm<WAVES, NB, NCB, 4, FP4, NS>(a, max_tiles, s);
    case 8: return run_gemm<WAVES, NB, NCB, 8, FP4, NS>(a, max_tiles, s);
    case 12: return run_gemm<WAVES, NB, NCB, 12, FP4, NS>(a, max_tiles, s);
    case 16: return run_gemm<WAVES, NB, NCB, 16, FP4, NS>(a, max_tiles, s);
    default: return hipErrorInvalidValue;
  }
}

// One grouped GEMM launch over a tile range.
static hipError_t gemm_launch(int nb, bool fp4, int mb, GemmArgs a, int max_tiles,
                              hipStream_t s) {
  const bool decode = mb == 1;
  // MOE_TRY: any tile height; MOE_TRY_DECODE: tiles of one row block only (the
  // decode configurations are built for that height alone)
#define MOE_TRY(W, NB_, NCB, FP4_, NS)                                          \
  if (a.N % ((W) * (NCB) * 16) == 0) {                                          \
    a.n_slabs = a.N / ((W) * (NCB) * 16);                                       \
    return run_gemm_mb<W, NB_, NCB, FP4_, NS>(mb, a, max_tiles, s);             \
  }
#define MOE_TRY_DECODE(W, NB_, NCB, FP4_, NS)                                   \
  if (a.N % ((W) * (NCB) * 16) == 0) {                                          \
    a.n_slabs = a.N / ((W) * (NCB) * 16);                                       \
    return run_gemm<W, NB_, NCB, 1, FP4_, NS>(a, max_tiles, s);                 \
  }
#define MOE_TRY32(W, NB_, NCB, NS)                                              \
  if (a.N % ((W) * (NCB) * 32) == 0) {                                          \
    a.n_slabs = a.N / ((W) * (NCB) * 32);                                       \
    return run_gemm32_mb<W, NB_, NCB, NS>(mb, a, max_tiles, s);                 \
  }
  // bf16 down GEMM on tiles of up to 192 rows: the 32x32x16 kernel (V3
  // prefill shape 1.65 -> 1.58 ms, same-box A/B).  Elsewhere it measured
  // level or slower than gemm_tile at the same slabs (hash and 2-gram
  // layers, FP4 down GEMM 3-7 % slower; V3 and FP4 gate|up within 1 %), and
  // so did 8-wave forms at two waves per SIMD (down GEMM one 32-column
  // block per wave; gate|up with the waves split between W_gate and W_up).
  if (!decode && a.Cf == nullptr && nb == 1 && !fp4 && mb <= 12) {
    MOE_TRY32(4, 1, 2, 3)
  }
  if (nb == 2) {
    if (fp4) {
      if (decode) { MOE_TRY_DECODE(4, 2, 2, true, 4) }
      else { MOE_TRY(8, 2, 1, true, 3) }
      MOE_TRY(4, 2, 1, true, 3)
    } else {
      if (decode) { MOE_TRY_DECODE(4, 2, 1, false, 3) }
      else if (mb >= 16) { MOE_TRY(8, 2, 1, false, 4) }
      else { MOE_TRY(8, 2, 1, false, 3) }
      MOE_TRY(4, 2, 1, false, 3)
    }
  } else {
    if (fp4) {
      if (decode) { MOE_TRY_DECODE(4, 1, 4, true, 4) }
      else { MOE_TRY(8, 1, 2, true, 3) }
      MOE_TRY(4, 1, 1, true, 3)
    } else {
      if (decode) { MOE_TRY_DECODE(4, 1, 2, false, 3) }
      else { MOE_TRY(8, 1, 2, false, 3) }
      MOE_TRY(4, 1, 1, false, 3)
    }
  }
#undef MOE_TRY
#undef MOE_TRY_DECODE
#undef MOE_TRY32
  return hipErrorInvalidValue;
}

hipError_t launch_dense_logits(const void *x, const void *w, int64_t T, int d, int E, float *z,
                               hipStream_t s) {
  if (E % 64 != 0 || d % 64 != 0) return hipErrorInvalidValue;
  GemmArgs a = {};
  a.A = (const bf16 *)x;
  a.K = d;
  a.N = E;
  a.B[0] = w;
  a.E = 1;                                   // group 0 is never the shared group
  a.Cf = z;
  a.dense_rows = T;
  a.dense_tile_rows = 64;
  a.tile_begin = 0;
  a.tile_end = (int)((T + 63) / 64);
  a.n_slabs = E / 64;
  return run_gemm<4, 1, 1, 4, false, 3>(a, a.tile_end, s);
}

static hipError_t mark(const ExpertPlan &p, int i, hipStream_t s) {
  return p.events ? hipEventRecord(p.events[i], s) : hipSuccess;
}

// The shared expert on the grouped kernel's dense form: its rows in order (no
// tile list), group 0 taken as the shared group (E = 0) and every row's gate
// value 1 (no row is below routed_rows = 0).
static GemmArgs shared_dense_args(const ExpertPlan &p, int tile_rows) {
  GemmArgs a = {};
  a.E = 0;
  a.routed_rows = 0;
  a.tiled = p.tiled ? 1 : 0;
  a.dense_rows = p.T;
  a.dense_tile_rows = tile_rows;
  a.tile_begin = 0;
  a.tile_end = (int)((p.T + tile_rows - 1) / tile_rows);
  return a;
}

hipError_t launch_shared_expert(const ExpertPlan &p, hipStream_t s, hipEvent_t xq_ready) {
  hipError_t err;
  const int64_t routed_rows = p.T * p.k;
  const moe_weights &w = *p.w;
  if (p.mx) {
    if ((err = launch_quantize_mxfp8((const bf16 *)p.x, p.T, p.dim, p.xq, p.xq_scales, s)) !=
        hipSuccess)
      return err;
    if ((err = hipEventRecord(xq_ready, s)) != hipSuccess) return err;
  }
  if (!p.has_shared) return hipSuccess;
  bf16 *hs = (bf16 *)p.h + routed_rows * p.inter;
  const int mb = p.tile_rows / 16;
  // gate|up + SwiGLU: the dense 32x32x16 kernel where the widths allow
  if (p.inter % 128 == 0 && p.dim % 128 == 0) {
    if ((err = launch_dense_swiglu(p.x, p.T, p.dim, p.inter, w.sh_gate, w.sh_up, p.tiled,
                                   p.swiglu_limit, hs, s)) != hipSuccess)
      return err;
  } else {
    GemmArgs a = shared_dense_args(p, p.tile_rows);
    a.A = (const bf16 *)p.x;
    a.K = p.dim;
    a.N = p.inter;
    a.SB[0] = (const bf16 *)w.sh_gate; a.SB[1] = (const bf16 *)w.sh_up;
    a.C = hs;
    a.limit = p.swiglu_limit;
    if ((err = gemm_launch(2, false, mb, a, a.tile_end, s)) != hipSuccess) return err;
  }
  // down projection on the grouped kernel (its tiles read less per MFMA here)
  GemmArgs a = shared_dense_args(p, p.tile_rows);
  a.A = hs;
  a.K = p.inter;
  a.N = p.dim;
  a.SB[0] = (const bf16 *)w.sh_down;
  a.C = (bf16 *)p.yrows + routed_rows * p.dim;
  return gemm_launch(1, false, mb, a, a.tile_end, s);
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
  // low-precision routed experts (FP4, or FP8 re-dequantised from FP4): the
  // shared expert runs as its own bf16 launch
  const bool fp4 = p.expert_dtype == MOE_DTYPE_FP4_E2M1 ||
                   p.expert_dtype == MOE_DTYPE_FP8_E4M3_B128;
  GemmArgs a = {};
  a.b_fp8 = p.expert_dtype == MOE_DTYPE_FP8_E4M3_B128 ? 1 : 0;
  a.E = p.E;
  a.tiles = p.tiles;
  a.tile_count = p.tile_count;
  a.routed_rows = routed_rows;
  a.sorted_w = p.sorted_w;
  a.tiled = p.tiled ? 1 : 0;

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
  // With a side stream the shared expert is already launched there and the
  // launches below cover the routed tiles only.  Otherwise the shared expert
  // of FP4 layers runs as launches of its own; its gate|up GEMM on the dense
  // 32x32x16 kernel where the widths allow (rows routed_rows .. of H).  Its
  // down GEMM stays on the grouped kernel, whose 192 x 256 tiles read less per
  // MFMA than the dense kernel's 128 x 128.
  const bool side = p.shared_done != nullptr;
  const bool dense_shared = p.inter % 128 == 0 && p.dim % 128 == 0;
  if (fp4 || side) {
    if (side) {
      if (p.mx && (err = hipStreamWaitEvent(s, p.xq_ready, 0)) != hipSuccess) return err;
    } else if (p.n_shared_tiles > 0 && dense_shared) {
      if ((err = launch_dense_swiglu(p.x, p.T, p.dim, p.inter, w.sh_gate, w.sh_up, p.tiled,
                                     p.swiglu_limit, (bf16 *)p.h + routed_rows * p.inter, s)) !=
          hipSuccess)
        return err;
    } else if (p.n_shared_tiles > 0) {
      GemmArgs sh = a;
      sh.tile_begin = 0; sh.tile_end = p.n_shared_tiles;
      if ((err = gemm_launch(2, false, mb, sh, p.n_shared_tiles, s)) != hipSuccess) return err;
    }
    a.tile_begin = p.n_shared_tiles; a.tile_end = -1;
    if (p.mx) {
      // routed experts on MXFP8 activations: quantise x, gather its rows
      if (!side && (err = launch_quantize_mxfp8((const bf16 *)p.x, p.T, p.dim, p.xq,
                                                p.xq_scales, s)) != hipSuccess)
        return err;
      // H's routed rows go straight to MXFP8 for the down GEMM
      a.Aq = p.xq;
      a.Asc = p.xq_scales;
      a.Cq = p.hq;
      a.Csc = p.hq_scales;
      if ((err = launch_gemm_mx(2, mb, a, p.max_tiles - p.n_shared_tiles, s)) != hipSuccess)
        return err;
      a.Cq = nullptr;
      a.Csc = nullptr;
    } else if ((err = gemm_launch(2, fp4, mb, a, p.max_tiles - p.n_shared_tiles, s)) !=
               hipSuccess) {
      return err;
    }
  } else {
    a.tile_begin = 0; a.tile_end = -1;
    a.n_shared_tiles = p.n_shared_tiles;
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
  if (fp4 || side) {
    if (!side && p.n_shared_tiles > 0) {
      GemmArgs sh = a;
      sh.tile_begin = 0; sh.tile_end = p.n_shared_tiles;
      if ((err = gemm_launch(1, false, mb, sh, p.n_shared_tiles, s)) != hipSuccess) return err;
    }
    a.tile_begin = p.n_shared_tiles; a.tile_end = -1;
    if (p.mx) {
      // the routed rows of H (the first T*k) in MXFP8, in permuted order
      a.Aq = p.hq;
      a.Asc = p.hq_scales;
      if ((err = launch_gemm_mx(1, mb, a, p.max_tiles - p.n_shared_tiles, s)) != hipSuccess)
        return err;
    } else if ((err = gemm_launch(1, fp4, mb, a, p.max_tiles - p.n_shared_tiles, s)) !=
               hipSuccess) {
      return err;
    }
  } else {
    a.tile_begin = 0; a.tile_end = -1;
    a.n_shared_tiles = p.n_shared_tiles;
    if ((err = gemm_launch(1, false, mb, a, p.max_tiles, s)) != hipSuccess) return err;
  }

  if ((err = mark(p, MOE_STAGE_COMBINE, s)) != hipSuccess) return err;
  if (side && (err = hipStreamWaitEvent(s, p.shared_done, 0)) != hipSuccess) return err;
  {
    const int64_t sb = p.has_shared ? routed_rows : (int64_t)-1;
    const int lanes = (p.dim / 8 + 63) / 64 * 64;
    const dim3 grid((unsigned)p.T), blk((unsigned)(lanes < 1024 ? lanes : 1024));
    const bf16 *Y = (const bf16 *)p.yrows;
    bf16 *yo = (bf16 *)p.y;
    if (p.k <= 2)
      hipLaunchKernelGGL(combine_bf16<2>, grid, blk, 0, s, Y, p.inverse, p.k, p.dim, sb, yo);
    else if (p.k <= 4)
      hipLaunchKernelGGL(combine_bf16<4>, grid, blk, 0, s, Y, p.inverse, p.k, p.dim, sb, yo);
    else if (p.k <= 8)
      hipLaunchKernelGGL(combine_bf16<8>, grid, blk, 0, s, Y, p.inverse, p.k, p.dim, sb, yo);
    else
      hipLaunchKernelGGL(combine_bf16<16>, grid, blk, 0, s, Y, p.inverse, p.k, p.dim, sb, yo);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return mark(p, MOE_STAGE_COUNT, s);
}

}  // namespace moe
