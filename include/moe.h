/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts feed-forward layer.
 *
 * The library computes the forward pass of a DeepSeek-style MoE FFN layer:
 *
 *   y[t] = cast( sum_j w[t,j] * FFN_{idx[t,j]}(x[t]) + FFN_shared(x[t]) )
 *   FFN(u) = W_down( SiLU(min(W_gate u, L)) * clamp(W_up u, -L, L) )
 *
 * Sources (pages, by title and section):
 *   - "DeepSeek-V3.2-Exp - Routing weights": excerpts "gate-init",
 *     "gate-forward" (learned gate) and "moe-forward" (dispatch loop).
 *   - "DeepSeek V4.1 - Add shared": the V4.1 MoE class (FP4 routed experts,
 *     swiglu_limit, shared expert added to every token, y cast to x's dtype).
 *   - "From One Giant FFN to 384 Tiny Experts": Ch.1 SwiGLU, Ch.4 routed +
 *     shared formula, Ch.6 selection-only bias, Ch.11.1 hash-routed layers,
 *     Ch.11.2 Sqrt(Softplus) affinity, Ch.11.4 SwiGLU clamp, Ch.11.6 FP4.
 *   - "How was DeepSeek V4's tid2eid derived?": eq. (1)-(2) and the greedy
 *     least-loaded table construction.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns
 *     every buffer; the library never allocates or frees device memory.
 *   - GPU work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising.  Outputs are
 *     valid once the stream reaches that point.
 *   - Arguments are validated on the host before any launch; invalid ones
 *     return MOE_ERR_INVALID_ARG (or MOE_ERR_UNSUPPORTED for valid-but-not-
 *     implemented shapes) and enqueue nothing.  A failed launch returns
 *     MOE_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Weight matrices are [out, in] row-major with the input (K) dimension
 *     contiguous, like nn.Linear: gate weight [E, dim]; routed W_gate and
 *     W_up [E, I, dim]; W_down [E, dim, I]; shared [I, dim], [I, dim], [dim, I].
 *     Routed and shared expert matrices (and FP4 scales) may instead be
 *     given in the tiled layout that moe_pack_weights writes
 *     (moe_config.weight_layout = MOE_LAYOUT_TILED); same sizes, same values.
 *   - bf16 is IEEE-style bfloat16 (upper half of an fp32); fp32 is IEEE.
 *   - FP4 routed experts (MOE_DTYPE_FP4_E2M1): E2M1 codes packed two per
 *     byte along the input dimension, element 2i in the low nibble; one
 *     E8M0 scale byte (value 2^(e-127)) per 32 consecutive input elements
 *     of each output row (OCP MXFP4, 1x32 sub-blocks).
 *   - All calls are thread-safe: the library holds no mutable global state.
 *     Calls that share a workspace must be ordered on one stream.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* bad pointer, size or config field            */
  MOE_ERR_UNSUPPORTED = -2,   /* valid config this build does not implement    */
  MOE_ERR_WORKSPACE = -3,     /* workspace missing, misaligned or too small    */
  MOE_ERR_HIP = -4            /* a HIP launch or runtime call failed           */
} moe_status;

typedef enum {                /* affinity s = f(z) of the logits z             */
  MOE_SCORE_SOFTMAX = 0,      /* softmax over the E routed experts             */
  MOE_SCORE_SIGMOID = 1,      /* 1 / (1 + exp(-z))                             */
  MOE_SCORE_SQRTSOFTPLUS = 2  /* sqrt(log(1 + exp(z)))                         */
} moe_score_func;

typedef enum {
  MOE_ROUTE_LEARNED = 0,      /* gate GEMM + affinity + bias + group top-k     */
  MOE_ROUTE_HASH = 1,         /* indices = tid2eid[token_id]                   */
  MOE_ROUTE_NGRAM_HASH = 2    /* 2-gram hash: token_ids holds [T, 2] pairs
                                 (previous id, current id); see moe_route     */
} moe_route_mode;

typedef enum {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  MOE_DTYPE_FP4_E2M1 = 2,     /* routed experts only; see conventions above    */
  MOE_DTYPE_FP8_E4M3_B128 = 3 /* routed experts only: E4M3 codes in the layout
                                 moe_redequant_fp8 writes, one E8M0 scale per
                                 128 x 128 block (moe_weights.s_gate/s_up/s_down
                                 point to the [E, out/128, in/128] scales);
                                 needs act_quant MXFP8 and weight_layout TILED */
} moe_dtype;

typedef enum {
  MOE_LAYOUT_ROWS = 0,        /* expert matrices [out, in] row-major           */
  MOE_LAYOUT_TILED = 1        /* expert matrices as written by moe_pack_weights */
} moe_weight_layout;

typedef enum {
  MOE_ACT_QUANT_NONE = 0,     /* routed experts see the bf16 activations       */
  MOE_ACT_QUANT_MXFP8 = 1     /* FP4 routed experts: the activations entering
                                 each routed GEMM (gathered x; SwiGLU output H)
                                 are quantised to OCP MXFP8 (E4M3 + one E8M0
                                 scale per 32 inputs, shared exponent
                                 floor(log2 amax) - 8, nearest value, ties to
                                 even, saturating at 448) and multiplied with
                                 the stored FP4 codes on the scaled MFMA; needs
                                 expert_dtype FP4_E2M1, act_dtype BF16,
                                 dim % 128 == 0, moe_inter_dim % 128 == 0.  The
                                 shared expert keeps bf16 activations.  The
                                 FP8 computation of FP4 experts: "From One
                                 Giant FFN to 384 Tiny Experts", Ch.11.6.      */
} moe_act_quant;

/* Layer configuration.  Field names follow the model arguments of the
 * "gate-init" excerpt and the V4.1 MoE class. */
typedef struct {
  int32_t dim;                 /* model width d                                  */
  int32_t n_routed_experts;    /* E (1..1024; learned routing: 1..512)           */
  int32_t n_activated_experts; /* k experts per token (1..16, k <= E)            */
  int32_t n_expert_groups;     /* G (1 = no groups); E % G == 0                  */
  int32_t n_limited_groups;    /* groups kept per token, 1..G                    */
  int32_t moe_inter_dim;       /* expert intermediate width I (also the shared) */
  int32_t n_shared_experts;    /* 0 or 1                                         */
  int32_t score_func;          /* moe_score_func                                 */
  float route_scale;           /* weights are multiplied by this                 */
  int32_t renormalize;         /* -1: renormalise iff score_func != softmax; 0/1 */
  float swiglu_limit;          /* L > 0 clamps; 0 = no clamp                     */
  int32_t route_mode;          /* moe_route_mode                                 */
  int64_t vocab_size;          /* hash routing: rows of tid2eid; 2-gram hash:
                                  the vocabulary size m (1 .. 2^31 - 1)          */
  int32_t act_dtype;           /* x, y, gate weight, shared expert: F32 or BF16  */
  int32_t expert_dtype;        /* routed experts: F32 (act F32), BF16 or
                                  FP4_E2M1 (act BF16)                            */
  int32_t weight_layout;       /* moe_weight_layout of the routed and shared
                                  expert matrices; TILED needs act_dtype BF16    */
  int32_t act_quant;           /* moe_act_quant for the routed FP4 experts       */
} moe_config;

/* Layer weights; unused members may be NULL. */
typedef struct {
  const void *gate_w;          /* [E, dim] act_dtype (learned routing)           */
  const float *gate_bias;      /* [E] fp32 selection bias, or NULL               */
  const void *w_gate;          /* [E, I, dim] (FP4: bytes [E, I, dim/2])         */
  const void *w_up;            /* [E, I, dim] (FP4: bytes [E, I, dim/2])         */
  const void *w_down;          /* [E, dim, I] (FP4: bytes [E, dim, I/2])         */
  const uint8_t *s_gate;       /* FP4 only: E8M0 [E, I, dim/32]                  */
  const uint8_t *s_up;         /* FP4 only: E8M0 [E, I, dim/32]                  */
  const uint8_t *s_down;       /* FP4 only: E8M0 [E, dim, I/32]                  */
  const void *sh_gate;         /* shared expert [I, dim] act_dtype               */
  const void *sh_up;           /* shared expert [I, dim] act_dtype               */
  const void *sh_down;         /* shared expert [dim, I] act_dtype               */
  const int32_t *tid2eid;      /* hash routing: [vocab_size, k] expert ids       */
} moe_weights;

/* Byte offsets of the sub-buffers moe_forward keeps in its workspace.
 * Every offset is 256-byte aligned; the workspace base must be too. */
typedef struct {
  size_t total_bytes;
  size_t route_weights;        /* float [T, k]   gate values                     */
  size_t route_indices;        /* int32 [T, k]   expert ids                      */
  size_t counts;               /* int32 [E]      pairs per expert                */
  size_t offsets;              /* int32 [E + 1]  exclusive scan of counts        */
  size_t sorted_tok;           /* int32 [T*k + T] token of each permuted row;
                                  rows T*k.. are the shared expert's (row-T*k)   */
  size_t sorted_slot;          /* int32 [T*k]    slot of each permuted row       */
  size_t sorted_weight;        /* float [T*k]    gate value of each permuted row */
  size_t inverse;              /* int32 [T, k]   permuted row of pair (t, j)     */
  size_t tiles;                /* int32 [max_tiles, 4] GEMM work list           */
  size_t tile_count;           /* int32 [1]      tiles written by the permute    */
  size_t flags;                /* uint32 [4]     device error flags (below)      */
  size_t route_logits;         /* float          partial gate logits (learned
                                  bf16 routing; 0 bytes otherwise)               */
  size_t perm_hist;            /* int32          per-chunk expert histograms and
                                  per-expert totals                          */
  size_t xq;                   /* uint8 [T, dim] MXFP8 codes of x (act_quant)   */
  size_t xq_scales;            /* uint8 [T, dim/32] their E8M0 scales            */
  size_t hq;                   /* uint8 [T*k, I] MXFP8 codes of H's routed rows  */
  size_t hq_scales;            /* uint8 [T*k, I/32]                              */
  size_t h;                    /* [T*k + T, I]   SwiGLU activations (bf16/f32);
                                  MXFP8 layers may leave the routed rows unwritten
                                  (the gate|up GEMM writes hq directly)          */
  size_t yrows;                /* [T*k + T, dim] weighted expert outputs         */
  int32_t max_tiles;
  int32_t tile_rows;           /* rows per GEMM tile chosen for this (cfg, T)    */
} moe_ws_layout;

/* Device error flag bits (flags[0]); a non-zero word means some output rows
 * were produced from substitute data as described. */
#define MOE_FLAG_TOKEN_ID_RANGE 1u  /* hash: a token id outside [0, vocab): the
                                       token used tid2eid row 0 with weight 0   */
#define MOE_FLAG_EXPERT_RANGE   2u  /* permute: an expert id outside [0, E):
                                       that pair was dropped (inverse = -1)     */

/* Human-readable name of a status code (static string). */
const char *moe_status_string(int status);

/* Host-only check of a configuration (no GPU needed).  Returns MOE_OK,
 * MOE_ERR_INVALID_ARG for inconsistent fields (E % G, k > E,
 * n_limited_groups > G, k > n_limited_groups * E / G, bad enums, ...) or
 * MOE_ERR_UNSUPPORTED for shapes this build does not implement (bf16/FP4
 * paths need dim % 64 == 0 and I % 64 == 0; group ranges whose size over
 * ceil(E/64) is not a power of two). */
int moe_validate_config(const moe_config *cfg);

/* Greedy hash-routing table ("How was DeepSeek V4's tid2eid derived?",
 * section "Mathematical formulation" and its reference implementation).
 * Tokens are taken by decreasing p (equal p: ascending id); each gets the k
 * experts of smallest current load (equal loads: ascending expert id), stored
 * in ascending (load, id) order, and each of those loads grows by p_i / k.
 *   p        (host) [m] token frequencies, any order, non-negative
 *   tid2eid  (host) [m, k] output, row = token id
 *   load     (host) [n] final normalised loads f, or NULL
 *   max_vio, min_vio (host) max(f) * n - 1 and min(f) * n - 1, or NULL
 * Pure host code, O(m * n); returns MOE_ERR_INVALID_ARG for m < 1, n < 1,
 * k < 1, k > n, NULL p/tid2eid or a negative/NaN p. */
int moe_build_tid2eid(const double *p, int64_t m, int32_t n, int32_t k,
                      int32_t *tid2eid, double *load,
                      double *max_vio, double *min_vio);

/* Rewrite the expert matrices into the tiled layout the grouped GEMMs
 * stream contiguously (a storage format only: the tiled matrices hold the same
 * values, and moe_forward gives bit-identical results with either layout).
 * Done once when the weights are loaded, not per forward call.
 *   src  expert matrices in MOE_LAYOUT_ROWS (cfg->weight_layout is ignored):
 *        w_gate, w_up, w_down, the FP4 scales and the shared matrices; NULL
 *        members are skipped.  gate_w, gate_bias and tid2eid are not touched.
 *   dst  caller-allocated buffers of the same byte sizes for every non-NULL
 *        src member (the pointers are written through; dst's struct itself is
 *        read-only), not overlapping src.
 * Layout, for a matrix [N, K] of one expert (K = input dim; N, K % 64 == 0):
 *   bf16: 16 x 32 tiles, tile (n/16, k/32) at element ((n/16)*(K/32) + k/32)*512;
 *         inside a tile, element (n, k) at (((k%32)/8)*16 + n%16)*8 + k%8 (one
 *         16-byte group per MFMA lane: 16 outputs x 8 consecutive inputs).
 *   FP4 codes (bytes [N, K/2]): 16 x 64-input tiles of 512 bytes, tile
 *         (n/16, kb/32) at byte ((n/16)*(K/64) + kb/32)*512 for byte column kb;
 *         inside, byte (n, kb) at (((kb%32)/8)*16 + n%16)*8 + kb%8.
 *   FP4 scales ([N, K/32]): 32-byte tiles, scale (n, j) at
 *         ((n/16)*(K/64) + j/2)*32 + (n%16)*2 + j%2.
 *   Experts follow each other as in the row layout (expert e at e*N*K elements).
 * Returns MOE_ERR_INVALID_ARG for a NULL cfg/src/dst, a NULL dst member whose
 * src member is set, or an fp32 layer; validation as moe_validate_config. */
int moe_pack_weights(const moe_config *cfg, const moe_weights *src,
                     const moe_weights *dst, void *stream);

/* FP4 -> FP8 re-dequantisation of expert weights ("From One Giant FFN to 384
 * Tiny Experts", Ch.11.6: FP4 weights in 1x32 sub-blocks dequantised to FP8
 * E4M3 in 128 x 128 blocks for computation, lossless while the sub-block
 * scale ratios stay within a bound).
 *   codes         n_mat consecutive FP4 matrices [N, K/2] bytes, row layout
 *                 (conventions above)
 *   scales        their E8M0 scales [N, K/32]
 *   fp8           out: E4M3 codes, n_mat x N x K bytes in the FP8 expert
 *                 layout: per matrix, 16-row block nb and 128-input stage st,
 *                 a 2 KB block at byte ((nb*(K/128) + st)*2048 whose byte
 *                 ((h*4 + q)*16 + c)*16 + i is the element of row 16nb + c,
 *                 input 128st + 64h + 16q + i
 *   block_scales  out: E8M0 [n_mat, N/128, K/128]: B = s_max - 6 floored at
 *                 0, s_max the largest scale among the block's 32-input
 *                 sub-blocks holding a nonzero code (127 if none)
 *   lossy         out: uint8 [n_mat, N/128, K/128], 1 where some element's
 *                 E4M3 code (the nearest value to e2m1 x 2^(s - B), ties to
 *                 even, saturating at 448) is not exactly its FP4 value --
 *                 exactly the blocks with a nonzero sub-block whose scale is
 *                 more than 2^14 below s_max -- else 0
 * Device pointers, enqueued on `stream` (hipStream_t or NULL).  N and K must
 * be positive multiples of 128 (MOE_ERR_UNSUPPORTED otherwise); NULL
 * pointers or n_mat < 0 give MOE_ERR_INVALID_ARG. */
int moe_redequant_fp8(const uint8_t *codes, const uint8_t *scales, int64_t n_mat, int32_t N,
                      int32_t K, uint8_t *fp8, uint8_t *block_scales, uint8_t *lossy,
                      void *stream);

/* Multi-start variant of moe_build_tid2eid (same page, "Reference
 * implementation": tokens taken in a random order instead of by decreasing
 * frequency; several runs; the table with the lowest max_vio is kept).
 *   orders      (host) [n_starts, m] int64: each row a permutation of
 *               0..m-1, the order one run takes the tokens in (the caller
 *               draws them, e.g. with its own seeded generator)
 *   best_start  (host) out: row of `orders` whose table is returned (equal
 *               max_vio keeps the earlier row), or NULL
 * Other arguments and tie rules as moe_build_tid2eid.  Returns
 * MOE_ERR_INVALID_ARG for n_starts < 1, a NULL `orders` or a row that is not
 * a permutation. */
int moe_build_tid2eid_multistart(const double *p, int64_t m, int32_t n, int32_t k,
                                 const int64_t *orders, int32_t n_starts, int32_t *tid2eid,
                                 double *load, double *max_vio, double *min_vio,
                                 int32_t *best_start);

/* Auxiliary-loss-free bias update ("From One Giant FFN to 384 Tiny Experts",
 * Ch.6 and 7.1), run once per training step after a forward pass:
 *   counts  [E] int32 pairs routed to each expert in the batch (the
 *           forward's workspace `counts`)
 *   T       tokens in the batch; the balanced level is T * k / E
 *   gamma   update speed (V3: 0.001)
 *   bias    [E] fp32 selection bias, updated in place: experts above the
 *           balanced level get bias - gamma, experts below it bias + gamma,
 *           experts exactly at it keep their bias (compared exactly as
 *           counts[e] * E against T * k; each step is one fp32 operation)
 *   stats   [4] double out, or NULL: mean load, population variance of the
 *           counts, max_vio = max(counts) * E / (T * k) - 1 and min_vio
 *           likewise (the balance measures of the tid2eid page and the
 *           load-variance table of the MaxText pull request "Load balancing
 *           changes for Deepseek v4")
 * Returns MOE_ERR_INVALID_ARG for a NULL cfg/counts/bias, T < 1 or a
 * non-finite gamma. */
int moe_update_bias(const moe_config *cfg, const int32_t *counts, int64_t T, float gamma,
                    float *bias, double *stats, void *stream);

/* Workspace needed by moe_forward for T tokens, and where each part lives.
 * Host-only; layout may be NULL.  Returns MOE_OK or a validation error. */
int moe_workspace_layout(const moe_config *cfg, int64_t T,
                         moe_ws_layout *layout);
size_t moe_workspace_size(const moe_config *cfg, int64_t T); /* 0 if invalid */

/* Routing ("gate-forward" excerpt; hash rule of Ch.11.1; the 2-gram hash
 * of "How was DeepSeek V4's tid2eid derived?", section "An extreme case").
 *   x         [T, dim] act_dtype (learned routing; may be NULL for hash)
 *   token_ids hash: [T] int32 token ids; 2-gram hash: [T, 2] int32 pairs
 *             (previous token id or -1 at a sequence start, current id);
 *             ignored for learned routing
 *   weights   [T, k] float out: gate values (hash: route_scale / k)
 *   indices   [T, k] int32 out: expert ids, in descending biased-score
 *             order; equal scores go to the lower expert id.  2-gram hash:
 *             expert j = (a * q_j + b) mod E for the pair (a, b), q_j the
 *             j-th smallest prime above vocab_size, a = vocab_size at a
 *             sequence start; the same expert may appear more than once.
 *             Ids outside [0, vocab_size) route like token 0 (2-gram: like
 *             the pair (vocab_size, 0)) with weight 0 and set
 *             MOE_FLAG_TOKEN_ID_RANGE in the forward's flags
 * Learned routing runs in one kernel: a workgroup owns 32 tokens and all E
 * experts, the score GEMM (bf16 MFMA, fp32 accumulation; fp32 FMAs for fp32
 * layers) leaves the logits in LDS, and the affinity, bias, group limit,
 * top-k and renormalisation run there; only weights and indices are written.
 * moe_forward, which has a workspace, routes with a split form instead (the
 * score GEMM split over the input dimension, its fp32 partial logits added
 * in order by the selection kernel): measured faster at every batch size,
 * see moe_forward.  Both forms select identically. */
int moe_route(const moe_config *cfg, const moe_weights *w, const void *x,
              const int32_t *token_ids, int64_t T,
              float *weights, int32_t *indices, void *stream);

/* Permutation by expert (the bincount / where loop of "moe-forward").
 *   indices     [T, k] int32 expert ids
 *   counts      [E]    out: pairs per expert
 *   offsets     [E+1]  out: exclusive scan, offsets[E] = pairs kept
 *   sorted_tok  [T*k]  out: token of each permuted row
 *   sorted_slot [T*k]  out: slot of each permuted row
 *   inverse     [T, k] out: permuted row of each pair (-1 if dropped)
 * Rows of one expert are in ascending (token, slot) order, so the result is
 * deterministic.  Ids outside [0, E) are dropped and flagged in `flags`
 * (uint32 [4], may be NULL; the caller zeroes it beforehand). */
int moe_permute(const moe_config *cfg, const int32_t *indices, int64_t T,
                int32_t *counts, int32_t *offsets, int32_t *sorted_tok,
                int32_t *sorted_slot, int32_t *inverse, uint32_t *flags,
                void *stream);

/* Full layer forward: route -> permute -> grouped GEMM1 (gate|up + SwiGLU,
 * clamp) -> grouped GEMM2 (down, times the gate value) -> combine with the
 * shared expert.  No host synchronisation inside.
 *   x   [T, dim] act_dtype;  token_ids [T] int32 (hash routing only)
 *   y   [T, dim] act_dtype out (may not alias x)
 *   ws  device workspace of at least moe_workspace_size(cfg, T) bytes,
 *       256-byte aligned; its sub-buffers (moe_ws_layout) hold the
 *       routing, permutation and intermediates of this call afterwards.
 * Learned bf16 routing inside the forward uses the split score GEMM: kp
 * partial [T, E] fp32 logit slices go to the workspace (route_logits) and the
 * selection kernel adds them in order.  That costs a round trip of
 * kp * T * E * 4 bytes (V3 prefill, T = 4096, E = 256, kp = 8: 33.6 MB each
 * way), but spreads the gate-weight stream over many workgroups: the route
 * stage takes 48 us there against 99 us for moe_route's one-kernel form
 * (23 against 90 us at T = 64), whose workgroups must each stream the whole
 * gate matrix.
 * Everything is enqueued on `stream`; nothing persists between calls.  The
 * call enqueues only kernels (and, in the variants below, event records and
 * waits): no host synchronisation, allocation or memset.  So it can be
 * captured in a HIP graph and replayed; a replay reads x, the weights and the
 * workspace at the addresses given at capture.
 * T == 0 is a no-op.  MOE_ERR_WORKSPACE if ws is NULL, misaligned or small. */
int moe_forward(const moe_config *cfg, const moe_weights *w, const void *x,
                const int32_t *token_ids, int64_t T, void *y,
                void *ws, size_t ws_bytes, void *stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the workspace is a fixed device array inside the library, one per GPU,
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) large and held until the process ends.
 * The caller still passes the inputs, the weights and y; arguments and
 * results are as moe_forward's.
 *   Returns MOE_ERR_WORKSPACE, before any launch, when moe_workspace_size(cfg,
 *   T) exceeds MOE_NOALLOC_SCRATCH_BYTES (V3 / V4.1-Flash shapes: decode
 *   batches of up to a few hundred tokens fit; large prefill batches do not),
 *   MOE_ERR_HIP if the array's device address cannot be obtained.
 * The call allocates nothing: the array's device address is taken once per
 * GPU (hipGetSymbolAddress, on the first call there).  Nothing in it needs to
 * start at zero (the kernels clear their flag words themselves).  Every call
 * on one GPU uses the same array and it keeps the last call's contents:
 * calls that overlap on one GPU (two streams, or two host threads without
 * ordering) race on it, so the caller orders them.  The workspace views of
 * moe_ws_layout are not exposed for this entry point. */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)
int moe_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                        const int32_t *token_ids, int64_t T, void *y, void *stream);

/* Stages of moe_forward in launch order (for moe_forward_profiled). */
#define MOE_STAGE_ROUTE 0     /* router kernel (or hash gather)                  */
#define MOE_STAGE_PERMUTE 1   /* permute kernel                                 */
#define MOE_STAGE_GEMM1 2     /* gate|up grouped GEMM + SwiGLU (routed + shared;
                                 routed only with a side stream, moe_forward_ex) */
#define MOE_STAGE_GEMM2 3     /* down grouped GEMM x gate value                  */
#define MOE_STAGE_COMBINE 4   /* gather-combine into y                          */
#define MOE_STAGE_COUNT 5

/* moe_forward that also records a timing event on `stream` before each stage
 * and after the last one, so the caller can time every kernel of the call.
 *   events (host) [MOE_STAGE_COUNT + 1] hipEvent_t handles created by the
 *   caller (hipEventCreate); event i precedes stage i, event COUNT follows
 *   the combine.  Results are identical to moe_forward's.  A failed
 *   hipEventRecord returns MOE_ERR_HIP. */
int moe_forward_profiled(const moe_config *cfg, const moe_weights *w, const void *x,
                         const int32_t *token_ids, int64_t T, void *y,
                         void *ws, size_t ws_bytes, void **events, void *stream);

/* moe_forward with optional stage events (as moe_forward_profiled; NULL: none)
 * and an optional second stream of the caller, `side_stream` (NULL: none;
 * not `stream` itself), on the same device.  For FP4 / FP8 expert layers with
 * bf16 activations the work that needs x alone -- the MXFP8 copy of x and the
 * shared expert -- is enqueued on side_stream, forked from `stream` at the
 * start of the call, so it runs while the latency-bound routing and
 * permutation run on `stream` (the shared expert's output is added to the
 * routed sum and depends on x alone, "DeepSeek V4.1 - Add shared", formula
 * of Delta_ffn; the shared experts' work placed in the routing's idle time,
 * "From One Giant FFN to 384 Tiny Experts", Ch.5.1); `stream` waits for x's copy before
 * the routed up GEMM and joins side_stream before the combine, so all work of
 * the call is ordered before whatever the caller enqueues on `stream` next,
 * and side_stream gets nothing the next call's fork does not order after
 * this call.  The fork and join events (three per host thread and device)
 * are created on a thread's first such call and kept until the process
 * ends; nothing else persists.  The stage events then time the routed launches
 * only.  Results are bit-identical to moe_forward's (the same kernels in the
 * same order per output).  Other layers ignore side_stream. */
int moe_forward_ex(const moe_config *cfg, const moe_weights *w, const void *x,
                   const int32_t *token_ids, int64_t T, void *y,
                   void *ws, size_t ws_bytes, void **events, void *stream,
                   void *side_stream);

/* Roofline probes: the achievable HBM read rate and bf16 / FP8 MFMA rates of
 * the GPU, measured with the instruction forms the layer kernels use (16-byte
 * nontemporal vector loads; v_mfma_f32_16x16x32_bf16, v_mfma_f32_32x32x16_bf16,
 * v_mfma_scale_f32_16x16x128_f8f6f4), for the caller to time on `stream` and
 * report next to the data-sheet peaks.  Neither touches the layer state.
 *   moe_probe_read: reads `bytes` (a multiple of 16) of `buf` (16-byte
 *     aligned); 1024 workgroups of 4 waves, each wave streaming its own
 *     contiguous share with 1 KB loads, 8 in flight.  out: uint32 [1024]
 *     device scratch, written only if the loaded words hash to one fixed
 *     value (so the loads cannot be dropped).
 *   moe_probe_mfma: 2048 workgroups x 4 waves, each wave `iters` rounds of 8
 *     independent bf16 MFMAs, 16x16x32 (shape 0) or 32x32x16 (shape 1), or
 *     of 16 independent scaled 16x16x128 MFMAs on E4M3 x E2M1 (shape 2, the
 *     MXFP8 x MXFP4 expert GEMMs) or E4M3 x E4M3 (shape 3).
 *     out: float [2048] device scratch, written likewise; *flops (host)
 *     receives the flops the launch performs.
 * Return MOE_ERR_INVALID_ARG for NULL/misaligned pointers, bytes < 16,
 * iters < 1 or another shape. */
int moe_probe_read(const void *buf, int64_t bytes, void *out, void *stream);
int moe_probe_mfma(int32_t iters, int32_t shape, void *out, double *flops, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
