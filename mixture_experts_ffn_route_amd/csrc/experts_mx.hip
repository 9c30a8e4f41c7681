// FP4 experts on MXFP8 activations for gfx950: the activation quantiser and
// the grouped GEMM tile on v_mfma_scale_f32_16x16x128_f8f6f4.
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
//   scales: lane l gives the E8M0 scale of its row (A) / column (B) for the
//           32-input block q
//   D: column r, rows 4q .. 4q+3 (as the 16x16x32 form)
//
// The pipeline is the one of the bf16 tile (experts.hip): 128-input stages
// now, activation rows (one 128-byte line per row and stage) and their scale
// words copied global -> LDS, FP4 codes and scales into a register ring,
// static waits, refills spread over the MFMA chunks.

#include "gemm.h"

namespace moe {
namespace {

// Nearest E4M3 (OCP) code to v, ties to even mantissa, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 448.f)) {
    code = 0x7Eu;                              // 1.75 x 2^8
  } else if (a < 0.015625f) {                  // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.f);   // 8 -> 0x08 = 2^-6
  } else {
    const uint32_t f = __float_as_uint(a);
    uint32_t q = f >> 20;                      // fp32 exponent and top 3 mantissa bits
    const uint32_t rem = f & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    code = q - (120u << 3);                    // rebias 127 -> 7
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// One thread per 32-input block (rows are contiguous, so block i of the
// flattened array is row i / (K/32)): shared exponent floor(log2(amax)) - 8
// clamped to [-127, 127] (0 for an all-zero block), codes of v / 2^X.
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
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= e4m3_code(ldexpf(v[4 * j + b], -X)) << (8 * b);
    w[j] = word;
  }
  u32x4 *o = (u32x4 *)(codes + i * 32);
  o[0] = u32x4{w[0], w[1], w[2], w[3]};
  o[1] = u32x4{w[4], w[5], w[6], w[7]};
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One tile on the scaled MFMA: MBE 16-row blocks, NB weight matrices, NCB
// 16-column blocks per wave and matrix.  SLOT = bytes per LDS ring slot
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

  for (int s0 = 0; s0 < nst; s0 += NS) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      const int st = s0 + p;
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT((NS - 2) * VM_PER_STAGE));
      __builtin_amdgcn_s_barrier();
      const int nslot = (p + NS - 1) % NS;
      const int nx = st + NS - 1 < last ? st + NS - 1 : last;
      if (st >= nst) issue_stage(nslot, nx);
      if (st < nst) {
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
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));

  // ---- epilogue (accumulator layout of the 16x16 MFMA forms) ----
  if constexpr (NB == 2) {
    const float L = g.limit;
#pragma unroll
    for (int m = 0; m < MBE; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + q * 4 + i;
        if (row < rows) {
          bf16 *crow = g.C + (int64_t)(row0 + row) * N + col0 + r16;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            float gv = acc[m][0][cb][i], uv = acc[m][1][cb][i];
            if (L > 0.f) {
              gv = fminf(gv, L);
              uv = fminf(fmaxf(uv, -L), L);
            }
            crow[cb * 16] = (bf16)(gv / (1.f + __expf(-gv)) * uv);
          }
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

template <int WAVES, int NB, int NCB, int MB, int NS>
constexpr int gemm_mx_slot_bytes() {
  constexpr int NFW = (MB * 2 + WAVES - 1) / WAVES;
  constexpr int NSW = ((MB * 16 + 63) / 64 + WAVES - 1) / WAVES;
  return NFW * WAVES * 1024 + NSW * WAVES * 256;
}

// WPE: waves per SIMD the kernel is compiled for (2: 256 registers per wave;
// 1: 512, for the tall tiles whose accumulators would otherwise spill).
template <int WAVES, int NB, int NCB, int MB, int NS, int WPE>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void grouped_gemm_mx(const GemmArgs g) {
  constexpr int SLOT = gemm_mx_slot_bytes<WAVES, NB, NCB, MB, NS>();
  __shared__ __attribute__((aligned(1024))) uint8_t Ls[NS * SLOT];
  int tile, slab;
  if (!gemm_work_item(g, &tile, &slab)) return;
  const TileCtx t = gemm_tile_ctx(g, tile, slab, WAVES, NCB * 16);
  const int nmb = (t.rows + 15) >> 4;
  if constexpr (MB < MCH) {
    gemm_tile_mx<WAVES, NB, NCB, MB, NS, SLOT>(g, t, Ls);
  } else {
    const int nch = (nmb + MCH - 1) / MCH;
    if (nch <= 1 || MB < 2 * MCH)
      gemm_tile_mx<WAVES, NB, NCB, (MB < MCH ? MB : MCH), NS, SLOT>(g, t, Ls);
    else if (nch == 2 || MB < 3 * MCH)
      gemm_tile_mx<WAVES, NB, NCB, (MB < 2 * MCH ? MB : 2 * MCH), NS, SLOT>(g, t, Ls);
    else if (nch == 3 || MB < 4 * MCH)
      gemm_tile_mx<WAVES, NB, NCB, (MB < 3 * MCH ? MB : 3 * MCH), NS, SLOT>(g, t, Ls);
    else
      gemm_tile_mx<WAVES, NB, NCB, MB, NS, SLOT>(g, t, Ls);
  }
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

// Short tiles: 8 waves, two per SIMD; tiles of 12+ row blocks: 4 waves with
// the whole register file.  Column blocks per wave: 1 for gate|up, 2 for down
// when the width allows (else 1).
template <int NB, int MB>
hipError_t run_gemm_mx_mb(GemmArgs a, int max_tiles, hipStream_t s) {
  constexpr bool tall = MB >= 12;
  constexpr int W = tall ? 4 : 8;
  constexpr int WPE = tall ? 1 : 2;
  if (NB == 1 && a.N % (W * 32) == 0) return run_gemm_mx<W, 1, 2, MB, 3, WPE>(a, max_tiles, s);
  if (a.N % (W * 16) == 0) return run_gemm_mx<W, NB, 1, MB, 3, WPE>(a, max_tiles, s);
  return run_gemm_mx<4, NB, 1, MB, 3, 1>(a, max_tiles, s);     // N % 64 == 0
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
