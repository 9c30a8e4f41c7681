// Permutation of (token, slot) pairs by expert, for gfx950.
//
// Mirrors the dispatch loop of "DeepSeek-V3.2-Exp - Routing weights",
// excerpt "moe-forward": counts are a bincount of the [T, k] index table and
// an expert's rows are its pairs in row-major (token, slot) order.  Here the
// whole permutation is built on the device without a host round trip, by one
// workgroup of 16 wavefronts:
//   1. each wave histograms a contiguous chunk of pairs into its own LDS row;
//   2. a scan over waves (per expert) and over experts gives every wave the
//      first output row of each expert inside its chunk, plus counts/offsets
//      and the GEMM work list (one tile per tile_rows rows of an expert:
//      expert, first row, rows, the expert's tile count);
//   3. each wave walks its chunk 64 pairs at a time; lanes that hold the same
//      expert find each other with one ballot per expert-id bit, take
//      consecutive rows in lane order, and the last of them advances the
//      wave's running row for that expert.  Chunks are disjoint and in order,
//      so the scatter is stable and deterministic.
// Large batches inside moe_forward use the same steps spread over many
// workgroups (chunks of kChunk pairs, per-chunk histograms kept in the
// workspace): perm_hist_kernel, perm_colscan_kernel (one wave per expert
// scans that expert's chunk counts), perm_scan_kernel (one workgroup: the
// scan over experts and the tile list) and perm_scatter_kernel.  The
// permutation is unique, so both give the same result.

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kPermWaves = 16;
constexpr int kPermMinChunks = 16;   // below this many chunks one workgroup is faster
constexpr int kPermThreads = kPermWaves * 64;

struct PermuteArgs {
  const int32_t *indices;
  int64_t n;            // T * k
  int64_t T;
  int E, k, nbits;
  int32_t *counts, *offsets, *sorted_tok, *sorted_slot, *inverse;
  uint32_t *flags;
  int32_t *tiles, *tile_count, *shared_rows_tok;
  const float *route_w;
  float *sorted_w;
  int tile_rows, n_shared_tiles;
  int clear_flags;      // zero flags[0] before use (nothing earlier in the call set it)
};

// Block-wide exclusive scan of one int per thread (1024 threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kPermWaves; ++w) { const int c = scratch[w]; scratch[w] = run; run += c; }
    scratch[kPermWaves] = run;
  }
  __syncthreads();
  const int ex = scratch[wave] + inc - v;
  *total = scratch[kPermWaves];
  __syncthreads();
  return ex;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const PermuteArgs a) {
  extern __shared__ int lds[];
  const int E = a.E;
  int *hist = lds;                              // [kPermWaves][E]
  int *scratch = lds + kPermWaves * E;          // [kPermWaves + 1]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int i = tid; i < kPermWaves * E; i += kPermThreads) hist[i] = 0;
  if (a.clear_flags && a.flags && tid == 0) a.flags[0] = 0u;
  __syncthreads();

  const int64_t chunk = (((a.n + kPermWaves - 1) / kPermWaves) + 63) & ~(int64_t)63;
  const int64_t begin = (int64_t)w * chunk;
  const int64_t end = begin + chunk < a.n ? begin + chunk : a.n;

  // 1. per-wave histograms
  for (int64_t p = begin + lane; p < end; p += 64) {
    const int e = a.indices[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[w * E + e], 1);
  }
  __syncthreads();

  // 2. scans.  Experts are spread over the threads in rounds of 1024.
  int carry_rows = 0, carry_tiles = 0;
  for (int e0 = 0; e0 < E; e0 += kPermThreads) {
    const int e = e0 + tid;
    int total = 0;
    if (e < E) {
      for (int ww = 0; ww < kPermWaves; ++ww) {
        const int c = hist[ww * E + e];
        hist[ww * E + e] = total;
        total += c;
      }
    }
    const int ntile = (a.tiles && e < E) ? (total + a.tile_rows - 1) / a.tile_rows : 0;
    int sum_rows, sum_tiles;
    const int off = carry_rows + block_exclusive_scan(total, scratch, &sum_rows);
    const int toff = carry_tiles + block_exclusive_scan(ntile, scratch, &sum_tiles);
    if (e < E) {
      a.counts[e] = total;
      a.offsets[e] = off;
      for (int ww = 0; ww < kPermWaves; ++ww) hist[ww * E + e] += off;
      if (a.tiles) {
        for (int j = 0; j < ntile; ++j) {
          int32_t *td = a.tiles + 4 * (int64_t)(a.n_shared_tiles + toff + j);
          const int r0 = j * a.tile_rows;
          td[0] = e;
          td[1] = off + r0;
          td[2] = (total - r0) < a.tile_rows ? (total - r0) : a.tile_rows;
          td[3] = ntile;                 // tiles of this expert
        }
      }
    }
    carry_rows += sum_rows;
    carry_tiles += sum_tiles;
  }
  if (tid == 0) {
    a.offsets[E] = carry_rows;
    if (a.tiles) *a.tile_count = a.n_shared_tiles + carry_tiles;
  }
  if (a.tiles) {
    // shared expert: rows T*k .. T*k+T-1 are the tokens in order
    for (int j = tid; j < a.n_shared_tiles; j += kPermThreads) {
      int32_t *td = a.tiles + 4 * (int64_t)j;
      const int64_t r0 = (int64_t)j * a.tile_rows;
      td[0] = E;
      td[1] = (int)(a.n + r0);
      td[2] = (a.T - r0) < a.tile_rows ? (int)(a.T - r0) : a.tile_rows;
      td[3] = a.n_shared_tiles;
    }
    for (int64_t t = tid; t < a.T; t += kPermThreads) a.shared_rows_tok[t] = (int32_t)t;
  }
  __syncthreads();

  // 3. stable scatter
  for (int64_t base = begin; base < end; base += 64) {
    const int64_t p = base + lane;
    const bool valid = p < end;
    const int e = valid ? a.indices[p] : -1;
    const bool ok = valid && (unsigned)e < (unsigned)E;
    if (valid && !ok) {
      a.inverse[p] = -1;
      if (a.flags) atomicOr(a.flags, (uint32_t)MOE_FLAG_EXPERT_RANGE);
    }
    uint64_t same = __ballot(ok);
    for (int b = 0; b < a.nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    if (ok) {
      const uint64_t below = same & ((1ull << lane) - 1ull);
      const int rank = __popcll(below);
      const int cnt = __popcll(same);
      const int row0 = hist[w * E + e];
      const int dest = row0 + rank;
      const int64_t t = p / a.k;
      a.sorted_tok[dest] = (int32_t)t;
      a.sorted_slot[dest] = (int32_t)(p - t * a.k);
      a.inverse[p] = dest;
      if (a.sorted_w) a.sorted_w[dest] = a.route_w[p];
      if (rank == cnt - 1) hist[w * E + e] = row0 + cnt;
    }
  }
}

// ---------------------------------------------------------------------------
// Chunked permutation: one wavefront per chunk of kChunk consecutive pairs.

constexpr int kChunk = 256;

// 1. histogram of chunk c, stored transposed: chist[e * C + c].
__global__ __launch_bounds__(64) void perm_hist_kernel(const PermuteArgs a, int32_t *chist,
                                                       int C) {
  extern __shared__ int h[];                    // [E]
  const int E = a.E, lane = threadIdx.x, c = blockIdx.x;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  if (a.clear_flags && a.flags && c == 0 && lane == 0) a.flags[0] = 0u;
  __syncthreads();
  const int64_t begin = (int64_t)c * kChunk;
  const int64_t end = begin + kChunk < a.n ? begin + kChunk : a.n;
  for (int64_t p = begin + lane; p < end; p += 64) {
    const int e = a.indices[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) chist[(int64_t)e * C + c] = h[e];
}

// 2a. per expert, exclusive scan over chunks, one wave per expert (in place:
// chist becomes the expert-relative first row of each chunk); the expert's
// total goes to tot[e].  Every wave's loads of up to 256 chunk counts are in
// flight together; the experts' scans run side by side across the GPU (one
// workgroup doing them in turn took 35-95 us at 384 experts x 256 chunks).
__global__ __launch_bounds__(256) void perm_colscan_kernel(int E, int32_t *chist, int C,
                                                           int32_t *tot) {
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int32_t *col = chist + (int64_t)e * C;
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += 64 * U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u + lane;
      v[u] = c < C ? col[c] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int inc = v[u];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
      }
      const int c = c0 + 64 * u + lane;
      if (c < C) col[c] = carry + inc - v[u];
      carry += __shfl(inc, 63);
    }
  }
  if (lane == 0) tot[e] = carry;
}

// 2b. counts, offsets, the tile list and the shared-expert rows from the
// experts' totals, as in the one-workgroup kernel.
__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(const PermuteArgs a,
                                                                 const int32_t *tot_g) {
  extern __shared__ int tot[];                  // [E] pairs per expert, then scratch
  int *scratch = tot + a.E;                     // [kPermWaves + 1]
  const int E = a.E, tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) tot[e] = tot_g[e];
  __syncthreads();
  int carry_rows = 0, carry_tiles = 0;
  for (int e0 = 0; e0 < E; e0 += kPermThreads) {
    const int e = e0 + tid;
    const int total = e < E ? tot[e] : 0;
    const int ntile = (a.tiles && e < E) ? (total + a.tile_rows - 1) / a.tile_rows : 0;
    int sum_rows, sum_tiles;
    const int off = carry_rows + block_exclusive_scan(total, scratch, &sum_rows);
    const int toff = carry_tiles + block_exclusive_scan(ntile, scratch, &sum_tiles);
    if (e < E) {
      a.counts[e] = total;
      a.offsets[e] = off;
      if (a.tiles) {
        for (int j = 0; j < ntile; ++j) {
          int32_t *td = a.tiles + 4 * (int64_t)(a.n_shared_tiles + toff + j);
          const int r0 = j * a.tile_rows;
          td[0] = e;
          td[1] = off + r0;
          td[2] = (total - r0) < a.tile_rows ? (total - r0) : a.tile_rows;
          td[3] = ntile;                 // tiles of this expert
        }
      }
    }
    carry_rows += sum_rows;
    carry_tiles += sum_tiles;
  }
  if (tid == 0) {
    a.offsets[E] = carry_rows;
    if (a.tiles) *a.tile_count = a.n_shared_tiles + carry_tiles;
  }
  if (a.tiles) {
    for (int j = tid; j < a.n_shared_tiles; j += kPermThreads) {
      int32_t *td = a.tiles + 4 * (int64_t)j;
      const int64_t r0 = (int64_t)j * a.tile_rows;
      td[0] = E;
      td[1] = (int)(a.n + r0);
      td[2] = (a.T - r0) < a.tile_rows ? (int)(a.T - r0) : a.tile_rows;
      td[3] = a.n_shared_tiles;
    }
    for (int64_t t = tid; t < a.T; t += kPermThreads) a.shared_rows_tok[t] = (int32_t)t;
  }
}

// 3. stable scatter of chunk c: its first row for expert e is
// offsets[e] + chist[e * C + c]; lanes with equal experts rank by lane order.
__global__ __launch_bounds__(64) void perm_scatter_kernel(const PermuteArgs a,
                                                          const int32_t *chist, int C) {
  extern __shared__ int row[];                  // [E] next row per expert
  const int E = a.E, lane = threadIdx.x, c = blockIdx.x;
  for (int e = lane; e < E; e += 64) row[e] = a.offsets[e] + chist[(int64_t)e * C + c];
  __syncthreads();
  const int64_t begin = (int64_t)c * kChunk;
  const int64_t end = begin + kChunk < a.n ? begin + kChunk : a.n;
  for (int64_t base = begin; base < end; base += 64) {
    const int64_t p = base + lane;
    const bool valid = p < end;
    const int e = valid ? a.indices[p] : -1;
    const bool ok = valid && (unsigned)e < (unsigned)E;
    if (valid && !ok) {
      a.inverse[p] = -1;
      if (a.flags) atomicOr(a.flags, (uint32_t)MOE_FLAG_EXPERT_RANGE);
    }
    uint64_t same = __ballot(ok);
    for (int b = 0; b < a.nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    if (ok) {
      const uint64_t below = same & ((1ull << lane) - 1ull);
      const int rank = __popcll(below);
      const int cnt = __popcll(same);
      const int row0 = row[e];
      const int dest = row0 + rank;
      const int64_t t = p / a.k;
      a.sorted_tok[dest] = (int32_t)t;
      a.sorted_slot[dest] = (int32_t)(p - t * a.k);
      a.inverse[p] = dest;
      if (a.sorted_w) a.sorted_w[dest] = a.route_w[p];
      if (rank == cnt - 1) row[e] = row0 + cnt;
    }
    __syncthreads();
  }
}

int64_t permute_chunks(int64_t pairs) { return (pairs + kChunk - 1) / kChunk; }

hipError_t launch_permute(int E, int k, int64_t T, const int32_t *indices, int32_t *counts,
                          int32_t *offsets, int32_t *sorted_tok, int32_t *sorted_slot,
                          int32_t *inverse, uint32_t *flags, const TileSpec *tiles,
                          bool clear_flags, hipStream_t s, int32_t *chunk_hist) {
  PermuteArgs a;
  a.clear_flags = clear_flags ? 1 : 0;
  a.indices = indices;
  a.n = T * k;
  a.T = T;
  a.E = E;
  a.k = k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  a.nbits = nbits;
  a.counts = counts; a.offsets = offsets; a.sorted_tok = sorted_tok;
  a.sorted_slot = sorted_slot; a.inverse = inverse; a.flags = flags;
  a.tiles = tiles ? tiles->tiles : nullptr;
  a.tile_count = tiles ? tiles->tile_count : nullptr;
  a.shared_rows_tok = tiles ? tiles->shared_rows_tok : nullptr;
  a.tile_rows = tiles ? tiles->tile_rows : 1;
  a.n_shared_tiles = tiles ? tiles->n_shared_tiles : 0;
  a.route_w = tiles ? tiles->route_w : nullptr;
  a.sorted_w = tiles && tiles->route_w ? tiles->sorted_w : nullptr;
  const int64_t C = permute_chunks(a.n);
  if (chunk_hist && C > kPermMinChunks) {
    const size_t le = (size_t)E * sizeof(int);
    int32_t *tot = chunk_hist + C * E;
    hipLaunchKernelGGL(perm_hist_kernel, dim3((unsigned)C), dim3(64), le, s, a, chunk_hist, (int)C);
    hipLaunchKernelGGL(perm_colscan_kernel, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, s, E,
                       chunk_hist, (int)C, tot);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kPermThreads),
                       le + (kPermWaves + 1) * sizeof(int), s, a, (const int32_t *)tot);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)C), dim3(64), le, s, a, chunk_hist,
                       (int)C);
    return hipGetLastError();
  }
  const size_t lds = ((size_t)kPermWaves * E + kPermWaves + 1) * sizeof(int);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void *)permute_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, s, a);
  return hipGetLastError();
}

__global__ void clear_flags_kernel(uint32_t *flags) {
  if (threadIdx.x < 4) flags[threadIdx.x] = 0u;
}

hipError_t launch_clear_flags(uint32_t *flags, hipStream_t s) {
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(64), 0, s, flags);
  return hipGetLastError();
}

}  // namespace moe
