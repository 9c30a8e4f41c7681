// Host-side launch interface between the C ABI (moe_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Learned routing: score GEMM + affinity + bias + group limit + top-k.  With
// `logits` (route_logits_floats(cfg, T) floats of workspace) bf16 layers use
// the split router; without, one fused kernel keeps the logits in LDS.
hipError_t launch_route_learned(const moe_config &cfg, const void *x, const void *gate_w,
                                const float *bias, int64_t T, float *weights,
                                int32_t *indices, hipStream_t s, float *logits = nullptr);
size_t route_logits_floats(const moe_config &cfg, int64_t T);

// z[T, E] = x[T, d] . w[E, d]^T in fp32 on the grouped-GEMM kernel (one group,
// 64-row tiles, 64-expert slabs); bf16 operands, E % 64 == 0, d % 64 == 0.
hipError_t launch_dense_logits(const void *x, const void *w, int64_t T, int d, int E, float *z,
                               hipStream_t s);

// Dense bf16 GEMMs on the 32x32x16 MFMA (dense.hip); N % 128 == 0, K % 64 == 0.
//   swiglu:    H[M, N] = SwiGLU(A Bg^T, A Bu^T) (clamped at `limit` > 0), bf16
//   f32_parts: Cf[p, M, N] = A[:, Kp] B[:, Kp]^T for the k_parts splits Kp of K
// B matrices [N, K] in the row layout or (`tiled`) the moe_pack_weights one.
hipError_t launch_dense_swiglu(const void *A, int64_t M, int K, int N, const void *Bg,
                               const void *Bu, bool tiled, float limit, void *H, hipStream_t s);
hipError_t launch_dense_f32_parts(const void *A, int64_t M, int K, int N, const void *B,
                                  int k_parts, float *Cf, hipStream_t s);

// 2-gram hash routing: pairs [T, 2] (previous id, current id); primes
// [k] the k smallest primes above cfg.vocab_size.
hipError_t launch_route_ngram(const moe_config &cfg, const int32_t *pairs, const int64_t *primes,
                              int64_t T, float *weights, int32_t *indices, uint32_t *flags,
                              hipStream_t s);

// Sign update of the selection bias from the batch's expert counts, plus
// load statistics (stats may be null).
hipError_t launch_update_bias(const int32_t *counts, int E, int64_t T, int k, float gamma,
                              float *bias, double *stats, hipStream_t s);

// Hash routing: indices = tid2eid[token_id], weights = route_scale / k.
hipError_t launch_route_hash(const moe_config &cfg, const int32_t *token_ids,
                             const int32_t *tid2eid, int64_t T, float *weights,
                             int32_t *indices, uint32_t *flags, hipStream_t s);

// Work list for the grouped GEMMs, written by the permute kernel.
struct TileSpec {
  int32_t *tiles;        // [max_tiles, 4]: group, first row, rows, 0
  int32_t *tile_count;   // [1]
  int tile_rows;         // rows per tile (BM)
  int n_shared_tiles;    // shared-expert tiles, stored first
  int32_t *shared_rows_tok;  // sorted_tok + T*k: identity rows for the shared expert
  const float *route_w;      // [T, k] gate values, or null
  float *sorted_w;           // [T*k]  gate value of each permuted row, or null
};

// chunk_hist: null (one workgroup) or int32 [(permute_chunks(T*k) + 1) * E]
// of workspace (per-chunk histograms, then per-expert totals), which lets
// large batches use the many-workgroup kernels.
hipError_t launch_permute(int E, int k, int64_t T, const int32_t *indices, int32_t *counts,
                          int32_t *offsets, int32_t *sorted_tok, int32_t *sorted_slot,
                          int32_t *inverse, uint32_t *flags, const TileSpec *tiles,
                          bool clear_flags, hipStream_t s, int32_t *chunk_hist = nullptr);

// Chunks of the many-workgroup permutation for `pairs` (token, slot) pairs.
int64_t permute_chunks(int64_t pairs);

hipError_t launch_clear_flags(uint32_t *flags, hipStream_t s);

// Everything the expert GEMMs and the combine need for one forward call.
struct ExpertPlan {
  int64_t T;
  int k, E, dim, inter;
  bool has_shared;
  float swiglu_limit;
  int act_dtype, expert_dtype;
  bool tiled;            // expert matrices in MOE_LAYOUT_TILED
  bool mx;               // FP4 routed experts on MXFP8 activations
  uint8_t *xq, *xq_scales, *hq, *hq_scales;   // MXFP8 copies of x and of H's routed rows
  const void *x;
  const moe_weights *w;
  const float *route_w;
  const int32_t *route_idx, *offsets;
  const int32_t *sorted_tok, *sorted_slot, *inverse;
  const float *sorted_w;
  const int32_t *tiles, *tile_count;
  int max_tiles, tile_rows, n_shared_tiles;
  void *h, *yrows, *y;
  hipEvent_t *events;    // null, or [MOE_STAGE_COUNT + 1] stage timing events
  // Non-null when launch_shared_expert has put the shared expert (and, for
  // MXFP8, x's quantised copy) on a side stream: launch_experts then leaves
  // them out, waits for xq_ready before the routed up GEMM and for
  // shared_done before the combine.
  hipEvent_t shared_done, xq_ready;
};

// Rows per GEMM tile chosen for a layer of T tokens (depends on the
// expected rows per expert, T*k/E).
int choose_tile_rows(const moe_config &cfg, int64_t T);

hipError_t launch_experts(const ExpertPlan &p, hipStream_t s);

// The shared expert of a bf16-activation FP4 / FP8 expert layer on stream s: H rows
// [T k, T k + T) = SwiGLU_shared(x), Y rows [T k, T k + T) = H W_down^T (both
// only need x), after x's MXFP8 copy for MXFP8 layers (xq_ready recorded
// after it).  Needs nothing the routing or the permutation writes.
hipError_t launch_shared_expert(const ExpertPlan &p, hipStream_t s, hipEvent_t xq_ready);

// FP4 -> FP8 E4M3 in 128 x 128 blocks (moe_redequant_fp8).
hipError_t launch_redequant_fp8(const uint8_t *codes, const uint8_t *scales, int64_t n_mat, int N,
                                int K, uint8_t *out, uint8_t *bscale, uint8_t *lossy,
                                hipStream_t s);

// Rewrite `count` consecutive [N, K] expert matrices (bf16 or FP4 codes) or
// their E8M0 scales (scales = true) from the row layout into the tiled one.
hipError_t launch_pack_matrix(const void *src, void *dst, int64_t count, int64_t N, int64_t K,
                              int dtype, bool scales, hipStream_t s);

// Roofline probes (moe_probe_read / moe_probe_mfma).
hipError_t launch_probe_read(const void *buf, int64_t bytes, uint32_t *out, hipStream_t s);
hipError_t launch_probe_mfma(int iters, int shape, float *out, hipStream_t s);
int64_t probe_mfma_flops(int iters, int shape);

}  // namespace moe
