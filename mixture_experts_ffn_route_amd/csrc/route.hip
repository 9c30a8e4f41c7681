// Routing kernels for gfx950.
//
// Learned gate ("DeepSeek-V3.2-Exp - Routing weights", excerpt "gate-forward";
// affinities from "From One Giant FFN to 384 Tiny Experts" Ch.4, Ch.7 and
// Ch.11.2; the selection-only bias of Ch.6): one workgroup owns a block of
// tokens and all E experts.  Phase 1 computes the fp32 logits z = x . W^T
// (bf16 operands on MFMA 16x16x32 with fp32 accumulation, or fp32 FMAs for
// fp32 layers) and parks them in LDS.  Phase 2 gives each token to one
// wavefront: lane l holds experts l*EPL .. l*EPL+EPL-1 in registers, applies
// the affinity and bias, reduces group top-2 sums with lane exchanges, ranks
// the groups, and runs k rounds of a wave-wide arg-max (ties to the lower
// expert id).  Only the k (index, weight) pairs per token reach HBM.
//
// Hash gate (Ch.11.1; "How was DeepSeek V4's tid2eid derived?"): a gather of
// tid2eid rows with uniform weights.

#include <climits>

#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace moe {

struct RouteArgs {
  const void *x;        // [T, d] bf16 or f32
  const void *w;        // [E, d] same dtype
  const float *bias;    // [E] or null
  int64_t T;
  int d, E, k, G, topk_groups, score_func, renorm;
  float route_scale;
  float *weights;       // [T, k]
  int32_t *indices;     // [T, k]
};

// ---------------------------------------------------------------------------
// Phase 2: selection for one token held by one wavefront.
// zrow: the token's E logits (LDS or global), given as `nparts` partial sums
// `pstride` floats apart that are added in order.  EPL experts per lane.
template <int EPL>
__device__ __forceinline__ void select_token(const RouteArgs &a, const float *zrow, int64_t t,
                                             int lane, int nparts = 1, int64_t pstride = 0) {
  float s[EPL], key[EPL];
  const int E = a.E;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane * EPL + j;
    s[j] = e < E ? zrow[e] : -INFINITY;
  }
  // parts added in order; each part's EPL loads are issued together
  for (int q = 1; q < nparts; ++q) {
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane * EPL + j;
      v[j] = e < E ? zrow[q * pstride + e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) s[j] += v[j];
  }
  // affinity
  if (a.score_func == MOE_SCORE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j) m = fmaxf(m, s[j]);
    m = wave_max(m);
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane * EPL + j;
      s[j] = (e < E) ? expf(s[j] - m) : 0.f;
      part += s[j];
    }
    const float inv = 1.f / wave_sum(part);
#pragma unroll
    for (int j = 0; j < EPL; ++j) s[j] *= inv;
  } else if (a.score_func == MOE_SCORE_SIGMOID) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) s[j] = 1.f / (1.f + expf(-s[j]));
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const float z = s[j];
      s[j] = sqrtf(fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))));
    }
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane * EPL + j;
    key[j] = (e < E) ? (a.bias ? s[j] + a.bias[e] : s[j]) : -INFINITY;
  }

  // group limit: lanes_per_group is a power of two (checked on the host)
  if (a.G > 1) {
    const int lpg = (E / a.G) / EPL;
    float a1 = -INFINITY, a2 = -INFINITY;   // largest and second largest key
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const float v = key[j];
      if (v > a1) { a2 = a1; a1 = v; } else if (v > a2) { a2 = v; }
    }
    // merge (a1, a2) pairs across the lpg lanes of the group
#define MOE_GROUP_MERGE(M)                                              \
    if (lpg > M) {                                                      \
      const float b1 = xor_lane<M>(a1), b2 = xor_lane<M>(a2);           \
      const float hi = fmaxf(a1, b1), lo = fminf(a1, b1);               \
      a2 = fmaxf(lo, fmaxf(a2, b2));                                    \
      a1 = hi;                                                          \
    }
    MOE_GROUP_MERGE(1) MOE_GROUP_MERGE(2) MOE_GROUP_MERGE(4)
    MOE_GROUP_MERGE(8) MOE_GROUP_MERGE(16) MOE_GROUP_MERGE(32)
#undef MOE_GROUP_MERGE
    const float gs = a.bias ? (a1 + a2) : a1;
    const int g = lane / lpg;
    int rank = 0;
    for (int gg = 0; gg < a.G; ++gg) {
      const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs), gg * lpg));
      rank += (v > gs) || (v == gs && gg < g);
    }
    if (g >= a.G || rank >= a.topk_groups) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) key[j] = -INFINITY;
    }
  }

  // top-k: k rounds of a wave-wide arg-max over (key desc, expert id asc)
  unsigned taken = 0;
  int my_idx = 0;
  float my_s = 0.f, ssum = 0.f;
  for (int r = 0; r < a.k; ++r) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {   // j ascending = expert id ascending: ties keep the lower id
      const int e = lane * EPL + j;
      const bool cand = !((taken >> j) & 1u) && e < E;
      if (cand && (be == 0x7fffffff || key[j] > bv)) { bv = key[j]; be = e; }
    }
#define MOE_ARGMAX_STEP(M)                                                   \
    {                                                                        \
      const float ov = xor_lane<M>(bv);                                      \
      const int oe = xor_lane<M>(be);                                        \
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }            \
    }
    MOE_ARGMAX_STEP(1) MOE_ARGMAX_STEP(2) MOE_ARGMAX_STEP(4)
    MOE_ARGMAX_STEP(8) MOE_ARGMAX_STEP(16) MOE_ARGMAX_STEP(32)
#undef MOE_ARGMAX_STEP
    const int owner = be / EPL;
    const int slot = be - owner * EPL;
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) if (j == slot) mine = s[j];
    if (lane == owner) taken |= 1u << slot;
    const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), owner));
    if (lane == r) { my_idx = be; my_s = sv; }
    ssum += sv;
  }
  if (lane < a.k) {
    float w = my_s;
    if (a.renorm) w = w / ssum;
    w *= a.route_scale;
    a.indices[t * a.k + lane] = my_idx;
    a.weights[t * a.k + lane] = w;
  }
}

// ---------------------------------------------------------------------------
// bf16 layers, fused: one workgroup (4 waves) owns 32 tokens and all E
// experts, so every logit of a token ends up in the workgroup's LDS and the
// selection runs on it there; only the k (index, weight) pairs per token
// reach HBM.
//
// Score GEMM z = x Wg^T on v_mfma_f32_32x32x16_bf16 (operand layout as in
// dense.hip: lane l, r = l % 32, h = l / 32 holds row / column r, inputs
// 8h .. 8h+7 of a 16-input step; the accumulator holds column r, rows
// 8(i/4) + 4h + i%4).  The input dimension runs in 64-input stages through
// an NS-deep LDS copy ring: per stage the 32 token rows (4 units) and the
// E_pad = 128 CPW gate rows (16 CPW units), each unit 8 rows x 128 bytes,
// copied global -> LDS by the DMA form of the 16-byte load (lane l takes row
// l/8, chunk (l%8) ^ (l/8), so every copied row is one full cache line and
// each 8-lane read phase hits distinct banks).  Wave w owns the CPW 32-expert
// column blocks w*CPW ..; every wave reads the shared token block.  Gate rows
// past E re-read row E-1 and token rows past T row T-1; their logits are
// dropped.  The ring slots are separate LDS objects and the steady-state
// loop has no branch, so the compiler adds no waits between a copy into one
// slot and a read of another; the waits are the explicit vmcnt counts.
//
// After the last stage the logits go to LDS ([32][E + 1] fp32, over the
// ring) and each wave runs select_token on 8 of the tokens.
template <int CPW, int NS>
constexpr int route_fused_slot_bytes() { return (4 + 16 * CPW) * 1024; }

template <int EPL, int CPW, int NS>
__global__ __launch_bounds__(256) void route_fused_bf16(const RouteArgs a) {
  constexpr int BT = 32;
  constexpr int XU = 4;                        // token units per stage
  constexpr int UNITS = XU + 16 * CPW;
  constexpr int VM = UNITS / 4;                // copies per wave and stage
  constexpr int SLOT = route_fused_slot_bytes<CPW, NS>();
  static_assert(NS >= 2 && NS <= 4 && (NS - 2) * VM <= 63, "ring depth");
  static_assert(SLOT >= BT * (64 * EPL + 1) * 4, "logit tile fits the first ring slot");
  __shared__ __attribute__((aligned(1024))) uint8_t S0[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t S1[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t S2[NS > 2 ? SLOT : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t S3[NS > 3 ? SLOT : 1];
  uint8_t *const ring[4] = {S0, S1, S2, S3};

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int E = a.E, d = a.d;
  const bf16 *x = (const bf16 *)a.x;
  const bf16 *w = (const bf16 *)a.w;

  // copy sources: unit u = wave + 4q; units 0..3 are token rows, the rest
  // gate rows 8(u - 4) ..
  const uint8_t *src[VM];
#pragma unroll
  for (int q = 0; q < VM; ++q) {
    const int u = wave + 4 * q;
    const int chunk = (lane & 7) ^ (lane >> 3);
    if (u < XU) {
      int64_t t = t0 + u * 8 + (lane >> 3);
      t = t < a.T ? t : a.T - 1;
      src[q] = (const uint8_t *)(x + t * d) + 16 * chunk;
    } else {
      int e = (u - XU) * 8 + (lane >> 3);
      e = e < E ? e : E - 1;
      src[q] = (const uint8_t *)(w + (int64_t)e * d) + 16 * chunk;
    }
  }
  const int r32 = lane & 31, h = lane >> 5, rr = lane & 7;
  int off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) off[s] = (r32 >> 3) * 1024 + (rr * 8 + ((2 * s + h) ^ rr)) * 16;

  typedef float f32x16 __attribute__((ext_vector_type(16)));
  f32x16 acc[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

  const int nst = d / 64;
  const int last = nst - 1;
  auto issue = [&](int SL, int ST, int q) {
    dma16(src[q] + (int64_t)ST * 128, ring[SL] + (wave + 4 * q) * 1024);
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
#pragma unroll
    for (int q = 0; q < VM; ++q) issue(p, p < last ? p : last, q);

  auto compute_stage = [&](int p, int nx) {
    const int nslot = (p + NS - 1) % NS;
    const uint8_t *base = ring[p];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 av = *(const bf16x8 *)(base + off[s]);
      bf16x8 bv[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        bv[j] = *(const bf16x8 *)(base + (XU + 4 * (wave * CPW + j)) * 1024 + off[s]);
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[j], acc[j], 0, 0, 0);
      // this k-step's share of the refill of the slot the previous stage used
#pragma unroll
      for (int q = s * ((VM + 3) / 4); q < (s + 1) * ((VM + 3) / 4) && q < VM; ++q)
        issue(nslot, nx, q);
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
  __syncthreads();                             // every wave is done with the ring

  // logits -> LDS [token][expert], over the first ring slot
  float *zl = (float *)S0;
  const int ldz = E + 1;
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int e = 32 * (wave * CPW + j) + r32;
    if (e < E) {
#pragma unroll
      for (int i = 0; i < 16; ++i) zl[(8 * (i >> 2) + 4 * h + (i & 3)) * ldz + e] = acc[j][i];
    }
  }
  __syncthreads();
  for (int tl = wave; tl < BT; tl += 4) {
    const int64_t t = t0 + tl;
    if (t < a.T) select_token<EPL>(a, zl + tl * ldz, t, lane);
  }
}

// ---------------------------------------------------------------------------
// Split router (moe_forward, which has a workspace for the logits).  The score
// GEMM is tiled over (16*MT tokens) x (64 experts) x (one of KS parts of the
// input dimension) so that even a decode batch spreads over many CUs; each of
// the 4 waves owns 16 experts and keeps NSR k-steps of operands in flight.
// Partial logits go to zpart[ks][t][e]; route_select_kernel adds the parts in
// order ks = 0, 1, ... and runs the same selection as the fused kernel.
template <int MT>
__global__ __launch_bounds__(256) void route_logits_bf16(const RouteArgs a, float *zpart, int KS) {
  constexpr int NSR = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * (16 * MT);
  const int ks = blockIdx.z;
  const int E = a.E, d = a.d;
  const int dk = d / KS;                        // a multiple of 32 (host picks KS)
  const int nsteps = dk / 32;
  const bf16 *x = (const bf16 *)a.x;
  const bf16 *w = (const bf16 *)a.w;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int ecol = (blockIdx.y * 4 + wave) * 16;   // first expert of this wave
  const bf16 *xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = t0 + m * 16 + r16;
    xrow[m] = x + (t < a.T ? t : a.T - 1) * (int64_t)d + ks * dk + kq;
  }
  const int ew = ecol + r16;
  const bf16 *wrow = w + (int64_t)(ew < E ? ew : E - 1) * d + ks * dk + kq;
  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 an[NSR][MT], bn[NSR];
  auto load = [&](int slot, int step) {
    const int off = step * 32;
#pragma unroll
    for (int m = 0; m < MT; ++m) an[slot][m] = *(const bf16x8 *)(xrow[m] + off);
    bn[slot] = *(const bf16x8 *)(wrow + off);
  };
  const int last = nsteps - 1;
#pragma unroll
  for (int p = 0; p < NSR - 1; ++p) load(p, p < last ? p : last);
  for (int s0 = 0; s0 < nsteps; s0 += NSR) {
#pragma unroll
    for (int p = 0; p < NSR; ++p) {
      const int st = s0 + p;
      const int nx = st + NSR - 1;
      load((p + NSR - 1) % NSR, nx < last ? nx : last);
      if (st < nsteps) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(an[p][m], bn[p], acc[m], 0, 0, 0);
      }
    }
  }
  if (ecol >= E) return;
  const int e = ecol + r16;
  float *zp = zpart + (int64_t)ks * a.T * E;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + m * 16 + (lane >> 4) * 4 + i;
      if (t < a.T && e < E) zp[t * E + e] = acc[m][i];
    }
}

template <int EPL>
__global__ __launch_bounds__(256) void route_select_kernel(const RouteArgs a, const float *zpart,
                                                           int KS) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < a.T) select_token<EPL>(a, zpart + t * a.E, t, lane, KS, a.T * (int64_t)a.E);
}

// Large batches with E % 64 == 0 compute the logits on a GEMM kernel: the
// dense 32x32x16 one split over the input dimension when E % 128 == 0, else
// the grouped-GEMM kernel as one group; small batches use route_logits_bf16
// split over the input dimension.
static bool use_dense_logits(int64_t T, int E) { return T >= 1024 && E % 64 == 0; }

// Splits of the input dimension for the 32x32x16 dense score GEMM (E % 128 ==
// 0): enough (row tile, expert tile, split) items to cover the GPU twice, each
// split at least 4 stages of 64 inputs; 0 when the dense GEMM does not apply.
static int dense32_parts(int64_t T, int E, int d) {
  if (E % 128 != 0 || d % 64 != 0) return 0;
  const int64_t items = ((T + 127) / 128) * (E / 128);
  int kp = 1;
  while (kp < 8 && items * kp < 512 && d / 64 >= 8 * kp) kp *= 2;
  return kp;
}

// Split-router shape for T tokens: row blocks per workgroup and input parts.
static void split_shape(int64_t T, int E, int d, int *mt, int *ks) {
  *mt = T >= 1024 ? 4 : 1;
  const int64_t blocks = ((T + 16 * *mt - 1) / (16 * *mt)) * ((E + 63) / 64);
  int k = 1;
  while (k < 8 && blocks * k * 2 <= 512 && d % (32 * k * 2) == 0) k *= 2;
  *ks = k;
}

size_t route_logits_floats(const moe_config &cfg, int64_t T) {
  if (cfg.route_mode != MOE_ROUTE_LEARNED || cfg.act_dtype != MOE_DTYPE_BF16) return 0;
  if (use_dense_logits(T, cfg.n_routed_experts)) {
    const int kp = dense32_parts(T, cfg.n_routed_experts, cfg.dim);
    return (size_t)(kp > 0 ? kp : 1) * T * cfg.n_routed_experts;
  }
  int mt, ks;
  split_shape(T, cfg.n_routed_experts, cfg.dim, &mt, &ks);
  return (size_t)ks * T * cfg.n_routed_experts;
}

// fp32 layers: logits by FMA (small layers; correctness path).
template <int EPL>
__global__ __launch_bounds__(256) void route_learned_f32(const RouteArgs a) {
  constexpr int BT = 16;
  extern __shared__ float zl[];                 // [BT][E + 1]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int E = a.E, d = a.d, ldz = E + 1;
  const float *x = (const float *)a.x;
  const float *w = (const float *)a.w;
  for (int p = threadIdx.x; p < BT * E; p += 256) {
    const int tl = p / E, e = p - tl * E;
    const int64_t t = t0 + tl;
    float z = 0.f;
    if (t < a.T) {
      const float *xr = x + t * d;
      const float *wr = w + (int64_t)e * d;
      for (int kk = 0; kk < d; ++kk) z = fmaf(xr[kk], wr[kk], z);
    }
    zl[tl * ldz + e] = z;
  }
  __syncthreads();
  for (int tl = wave; tl < BT; tl += 4) {
    const int64_t t = t0 + tl;
    if (t < a.T) select_token<EPL>(a, zl + tl * ldz, t, lane);
  }
}

__global__ __launch_bounds__(256) void route_hash(const int32_t *token_ids, const int32_t *tid2eid,
                                                  int64_t T, int k, int64_t vocab, float wval,
                                                  float *weights, int32_t *indices,
                                                  uint32_t *flags) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= T * k) return;
  const int64_t t = p / k;
  const int j = (int)(p - t * k);
  const int64_t id = token_ids[t];
  const bool ok = id >= 0 && id < vocab;
  indices[p] = tid2eid[(ok ? id : 0) * k + j];
  weights[p] = ok ? wval : 0.f;
  if (!ok && flags) atomicOr(flags, (uint32_t)MOE_FLAG_TOKEN_ID_RANGE);
}

// 2-gram hash ("How was DeepSeek V4's tid2eid derived?", section "An extreme
// case"): one thread per (token, slot); expert = (a * q_j + b) mod E in
// 64-bit integers.
struct NgramPrimes { int64_t q[16]; };

__global__ __launch_bounds__(256) void route_ngram(const int32_t *pairs, NgramPrimes primes,
                                                   int64_t T, int k, int E, int64_t vocab,
                                                   float wval, float *weights, int32_t *indices,
                                                   uint32_t *flags) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= T * k) return;
  const int64_t t = p / k;
  const int j = (int)(p - t * k);
  const int64_t prev = pairs[2 * t], cur = pairs[2 * t + 1];
  const bool ok = prev >= -1 && prev < vocab && cur >= 0 && cur < vocab;
  const int64_t a = ok ? (prev < 0 ? vocab : prev) : vocab;
  const int64_t b = ok ? cur : 0;
  indices[p] = (int32_t)((a * primes.q[j] + b) % E);
  weights[p] = ok ? wval : 0.f;
  if (!ok && flags) atomicOr(flags, (uint32_t)MOE_FLAG_TOKEN_ID_RANGE);
}

hipError_t launch_route_ngram(const moe_config &cfg, const int32_t *pairs, const int64_t *primes,
                              int64_t T, float *weights, int32_t *indices, uint32_t *flags,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int k = cfg.n_activated_experts;
  NgramPrimes q = {};
  for (int j = 0; j < k; ++j) q.q[j] = primes[j];
  const int64_t n = T * k;
  hipLaunchKernelGGL(route_ngram, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, pairs, q,
                     T, k, cfg.n_routed_experts, cfg.vocab_size, cfg.route_scale / (float)k,
                     weights, indices, flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bias update ("From One Giant FFN to 384 Tiny Experts", Ch.6): one
// workgroup; experts strided over the threads; the statistics reduce in a
// fixed order (per-wave shuffles, then wave 0 over the waves).
__global__ __launch_bounds__(1024) void update_bias_kernel(const int32_t *counts, int E, int64_t T,
                                                           int k, float gamma, float *bias,
                                                           double *stats) {
  __shared__ double ssq[16];
  __shared__ int smax[16], smin[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t total = T * k;
  const double mean = (double)total / E;
  double sq = 0.0;
  int mx = INT_MIN, mn = INT_MAX;
  for (int e = tid; e < E; e += 1024) {
    const int c = counts[e];
    const int64_t lhs = (int64_t)c * E;
    if (lhs > total) bias[e] = bias[e] - gamma;
    else if (lhs < total) bias[e] = bias[e] + gamma;
    const double dv = (double)c - mean;
    sq += dv * dv;
    mx = c > mx ? c : mx;
    mn = c < mn ? c : mn;
  }
  if (!stats) return;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sq += __shfl_xor(sq, off);
    const int omx = __shfl_xor(mx, off), omn = __shfl_xor(mn, off);
    mx = omx > mx ? omx : mx;
    mn = omn < mn ? omn : mn;
  }
  if (lane == 0) { ssq[w] = sq; smax[w] = mx; smin[w] = mn; }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    int gmx = INT_MIN, gmn = INT_MAX;
    for (int i = 0; i < 16; ++i) {
      s += ssq[i];
      gmx = smax[i] > gmx ? smax[i] : gmx;
      gmn = smin[i] < gmn ? smin[i] : gmn;
    }
    stats[0] = mean;
    stats[1] = s / E;
    stats[2] = (double)((int64_t)gmx * E) / (double)total - 1.0;
    stats[3] = (double)((int64_t)gmn * E) / (double)total - 1.0;
  }
}

hipError_t launch_update_bias(const int32_t *counts, int E, int64_t T, int k, float gamma,
                              float *bias, double *stats, hipStream_t s) {
  hipLaunchKernelGGL(update_bias_kernel, dim3(1), dim3(1024), 0, s, counts, E, T, k, gamma, bias,
                     stats);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The fused bf16 router's configuration for E experts: CPW = ceil(E / 128)
// 32-expert blocks per wave; a 3-stage ring where it fits the 160 KB of LDS
// (E <= 384), else 2 stages.
template <int EPL>
static hipError_t launch_fused_epl(const RouteArgs &a, hipStream_t s) {
  constexpr int CPW = (EPL + 1) / 2;
  constexpr int NS = CPW <= 3 ? 3 : 2;
  static_assert(NS * route_fused_slot_bytes<CPW, NS>() <= 160 * 1024, "LDS");
  const dim3 grid((unsigned)((a.T + 31) / 32));
  hipLaunchKernelGGL((route_fused_bf16<EPL, CPW, NS>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int EPL>
static hipError_t launch_learned_epl(const RouteArgs &a, int act_dtype, hipStream_t s) {
  if (act_dtype == MOE_DTYPE_BF16) return launch_fused_epl<EPL>(a, s);
  const size_t lds = (size_t)16 * (a.E + 1) * sizeof(float);
  const dim3 grid((unsigned)((a.T + 15) / 16));
  hipLaunchKernelGGL((route_learned_f32<EPL>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int EPL>
static hipError_t launch_split_epl(const RouteArgs &a, float *zpart, hipStream_t s) {
  if (use_dense_logits(a.T, a.E)) {
    // experts in multiples of 128: the 32x32x16 GEMM, the input dimension
    // split into kp parts that the selection kernel adds in order
    const int kp = dense32_parts(a.T, a.E, a.d);
    const hipError_t e = kp > 0 ? launch_dense_f32_parts(a.x, a.T, a.d, a.E, a.w, kp, zpart, s)
                                : launch_dense_logits(a.x, a.w, a.T, a.d, a.E, zpart, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_select_kernel<EPL>, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0,
                       s, a, (const float *)zpart, kp > 0 ? kp : 1);
    return hipGetLastError();
  }
  int mt, ks;
  split_shape(a.T, a.E, a.d, &mt, &ks);
  const dim3 grid((unsigned)((a.T + 16 * mt - 1) / (16 * mt)), (unsigned)((a.E + 63) / 64),
                  (unsigned)ks);
  if (mt == 4)
    hipLaunchKernelGGL(route_logits_bf16<4>, grid, dim3(256), 0, s, a, zpart, ks);
  else
    hipLaunchKernelGGL(route_logits_bf16<1>, grid, dim3(256), 0, s, a, zpart, ks);
  hipLaunchKernelGGL(route_select_kernel<EPL>, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s,
                     a, (const float *)zpart, ks);
  return hipGetLastError();
}

hipError_t launch_route_learned(const moe_config &cfg, const void *x, const void *gate_w,
                                const float *bias, int64_t T, float *weights,
                                int32_t *indices, hipStream_t s, float *logits) {
  if (T == 0) return hipSuccess;
  RouteArgs a;
  a.x = x; a.w = gate_w; a.bias = bias; a.T = T;
  a.d = cfg.dim; a.E = cfg.n_routed_experts; a.k = cfg.n_activated_experts;
  a.G = cfg.n_expert_groups; a.topk_groups = cfg.n_limited_groups;
  a.score_func = cfg.score_func;
  a.renorm = cfg.renormalize < 0 ? (cfg.score_func != MOE_SCORE_SOFTMAX) : (cfg.renormalize != 0);
  a.route_scale = cfg.route_scale;
  a.weights = weights; a.indices = indices;
  const int epl = (a.E + 63) / 64;
  if (logits && cfg.act_dtype == MOE_DTYPE_BF16) {
    switch (epl) {
      case 1: return launch_split_epl<1>(a, logits, s);
      case 2: return launch_split_epl<2>(a, logits, s);
      case 3: return launch_split_epl<3>(a, logits, s);
      case 4: return launch_split_epl<4>(a, logits, s);
      case 5: return launch_split_epl<5>(a, logits, s);
      case 6: return launch_split_epl<6>(a, logits, s);
      case 7: return launch_split_epl<7>(a, logits, s);
      case 8: return launch_split_epl<8>(a, logits, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epl) {
    case 1: return launch_learned_epl<1>(a, cfg.act_dtype, s);
    case 2: return launch_learned_epl<2>(a, cfg.act_dtype, s);
    case 3: return launch_learned_epl<3>(a, cfg.act_dtype, s);
    case 4: return launch_learned_epl<4>(a, cfg.act_dtype, s);
    case 5: return launch_learned_epl<5>(a, cfg.act_dtype, s);
    case 6: return launch_learned_epl<6>(a, cfg.act_dtype, s);
    case 7: return launch_learned_epl<7>(a, cfg.act_dtype, s);
    case 8: return launch_learned_epl<8>(a, cfg.act_dtype, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_route_hash(const moe_config &cfg, const int32_t *token_ids,
                             const int32_t *tid2eid, int64_t T, float *weights,
                             int32_t *indices, uint32_t *flags, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int k = cfg.n_activated_experts;
  const int64_t n = T * k;
  const float wval = cfg.route_scale / (float)k;
  hipLaunchKernelGGL(route_hash, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, token_ids,
                     tid2eid, T, k, cfg.vocab_size, wval, weights, indices, flags);
  return hipGetLastError();
}

}  // namespace moe
