// C ABI of the MoE layer library: validation, workspace layout, the host
// tid2eid builder and the launch sequence of a forward pass.  See moe.h for
// the contract of each entry point.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <numeric>
#include <vector>

#include "internal.h"
#include "moe.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int validate(const moe_config *c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  const int E = c->n_routed_experts, k = c->n_activated_experts, G = c->n_expert_groups;
  if (c->dim < 1 || E < 1 || k < 1 || c->moe_inter_dim < 1) return MOE_ERR_INVALID_ARG;
  if (k > E) return MOE_ERR_INVALID_ARG;
  if (G < 1 || E % G != 0) return MOE_ERR_INVALID_ARG;
  if (c->n_limited_groups < 1 || c->n_limited_groups > G) return MOE_ERR_INVALID_ARG;
  if (G > 1 && (int64_t)k > (int64_t)c->n_limited_groups * (E / G)) return MOE_ERR_INVALID_ARG;
  if (c->score_func < MOE_SCORE_SOFTMAX || c->score_func > MOE_SCORE_SQRTSOFTPLUS)
    return MOE_ERR_INVALID_ARG;
  if (c->route_mode != MOE_ROUTE_LEARNED && c->route_mode != MOE_ROUTE_HASH &&
      c->route_mode != MOE_ROUTE_NGRAM_HASH)
    return MOE_ERR_INVALID_ARG;
  if (c->renormalize < -1 || c->renormalize > 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->route_scale)) return MOE_ERR_INVALID_ARG;
  if (!(c->swiglu_limit >= 0.f) || std::isinf(c->swiglu_limit)) return MOE_ERR_INVALID_ARG;
  if (c->n_shared_experts < 0) return MOE_ERR_INVALID_ARG;
  if (c->n_shared_experts > 1) return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_DTYPE_F32) {
    if (c->expert_dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARG;
  } else if (c->act_dtype == MOE_DTYPE_BF16) {
    if (c->expert_dtype != MOE_DTYPE_BF16 && c->expert_dtype != MOE_DTYPE_FP4_E2M1 &&
        c->expert_dtype != MOE_DTYPE_FP8_E4M3_B128)
      return MOE_ERR_INVALID_ARG;
    if (c->dim % 64 != 0 || c->moe_inter_dim % 64 != 0) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  if (c->weight_layout != MOE_LAYOUT_ROWS && c->weight_layout != MOE_LAYOUT_TILED)
    return MOE_ERR_INVALID_ARG;
  if (c->weight_layout == MOE_LAYOUT_TILED && c->act_dtype != MOE_DTYPE_BF16)
    return MOE_ERR_UNSUPPORTED;
  if (c->act_quant != MOE_ACT_QUANT_NONE && c->act_quant != MOE_ACT_QUANT_MXFP8)
    return MOE_ERR_INVALID_ARG;
  if (c->act_quant == MOE_ACT_QUANT_MXFP8) {
    if (c->expert_dtype != MOE_DTYPE_FP4_E2M1 && c->expert_dtype != MOE_DTYPE_FP8_E4M3_B128)
      return MOE_ERR_INVALID_ARG;
    if (c->dim % 128 != 0 || c->moe_inter_dim % 128 != 0) return MOE_ERR_UNSUPPORTED;
  }
  // FP8 (re-dequantised) experts exist only in their own layout and run only
  // on MXFP8 activations
  if (c->expert_dtype == MOE_DTYPE_FP8_E4M3_B128) {
    if (c->act_quant != MOE_ACT_QUANT_MXFP8 || c->weight_layout != MOE_LAYOUT_TILED)
      return MOE_ERR_INVALID_ARG;
    if (c->dim > 32768 || c->moe_inter_dim > 32768) return MOE_ERR_UNSUPPORTED;
  }
  if (k > 16 || E > 1024) return MOE_ERR_UNSUPPORTED;
  if (c->route_mode == MOE_ROUTE_HASH) {
    if (c->vocab_size < 1) return MOE_ERR_INVALID_ARG;
  } else if (c->route_mode == MOE_ROUTE_NGRAM_HASH) {
    if (c->vocab_size < 1 || c->vocab_size > INT32_MAX) return MOE_ERR_INVALID_ARG;
  } else {
    if (E > 512) return MOE_ERR_UNSUPPORTED;
    if (G > 1) {
      const int epl = (E + 63) / 64;
      const int gs = E / G;
      if (G > 64 || gs % epl != 0 || !is_pow2(gs / epl)) return MOE_ERR_UNSUPPORTED;
    }
  }
  return MOE_OK;
}

int make_layout(const moe_config *c, int64_t T, moe_ws_layout *out) {
  const int st = validate(c);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  const int64_t k = c->n_activated_experts, E = c->n_routed_experts;
  const int64_t shared = c->n_shared_experts;
  const int64_t rows = T * k + T * shared;
  if (T * (k + 1) > INT32_MAX - 1) return MOE_ERR_UNSUPPORTED;
  const int bm = moe::choose_tile_rows(*c, T);
  const int64_t n_sh = shared ? (T + bm - 1) / bm : 0;
  const int64_t max_tiles = n_sh + (T * k + bm - 1) / bm + std::min<int64_t>(E, T * k);
  const size_t es = c->act_dtype == MOE_DTYPE_F32 ? 4 : 2;
  moe_ws_layout l;
  std::memset(&l, 0, sizeof(l));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.route_weights = take(sizeof(float) * T * k);
  l.route_indices = take(sizeof(int32_t) * T * k);
  l.counts = take(sizeof(int32_t) * E);
  l.offsets = take(sizeof(int32_t) * (E + 1));
  l.sorted_tok = take(sizeof(int32_t) * (T * k + T));
  l.sorted_slot = take(sizeof(int32_t) * T * k);
  l.sorted_weight = take(sizeof(float) * T * k);
  l.inverse = take(sizeof(int32_t) * T * k);
  l.tiles = take(sizeof(int32_t) * 4 * max_tiles);
  l.tile_count = take(sizeof(int32_t));
  l.flags = take(sizeof(uint32_t) * 4);
  l.route_logits = take(sizeof(float) * moe::route_logits_floats(*c, T));
  l.perm_hist = take(sizeof(int32_t) * (moe::permute_chunks(T * k) + 1) * E);
  const bool mx = c->act_quant == MOE_ACT_QUANT_MXFP8;
  l.xq = take(mx ? (size_t)T * c->dim : 0);
  l.xq_scales = take(mx ? (size_t)T * c->dim / 32 : 0);
  l.hq = take(mx ? (size_t)T * k * c->moe_inter_dim : 0);
  l.hq_scales = take(mx ? (size_t)T * k * c->moe_inter_dim / 32 : 0);
  l.h = take(es * rows * c->moe_inter_dim);
  l.yrows = take(es * rows * c->dim);
  l.total_bytes = off;
  l.max_tiles = (int32_t)max_tiles;
  l.tile_rows = bm;
  if (out) *out = l;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Events that fork a caller's side stream from its main stream and join it
// back: three per host thread and device.  A thread takes a triple for a
// device on its first call with a side stream there and keeps it while it
// lives; when the thread ends, its triples go back to a process-wide pool for
// the next thread that needs one (no HIP call at thread or process exit), so
// the number of events is bounded by the threads alive at once, not by the
// threads ever created.  A thread enqueues its calls one after another, and a
// wait takes the record made just before it, so the next call may record the
// same events again; no other thread uses them while they are taken.
struct SideEvents {
  hipEvent_t fork = nullptr, join = nullptr, xq_ready = nullptr;
  int device = -1;
};
constexpr int kMaxDevices = 64;

std::mutex &side_pool_mutex() {
  static std::mutex *m = new std::mutex;       // never destroyed: used at thread exit
  return *m;
}
std::vector<SideEvents> &side_pool() {
  static std::vector<SideEvents> *v = new std::vector<SideEvents>;
  return *v;
}

struct ThreadSideEvents {
  SideEvents per_device[kMaxDevices];
  ~ThreadSideEvents() {
    std::lock_guard<std::mutex> lock(side_pool_mutex());
    for (const SideEvents &ev : per_device)
      if (ev.device >= 0) side_pool().push_back(ev);
  }
};

hipError_t side_events(SideEvents **out) {
  thread_local ThreadSideEvents mine;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideEvents &ev = mine.per_device[dev];
  if (ev.device < 0) {
    {
      std::lock_guard<std::mutex> lock(side_pool_mutex());
      std::vector<SideEvents> &pool = side_pool();
      for (size_t i = 0; i < pool.size(); ++i)
        if (pool[i].device == dev) {
          ev = pool[i];
          pool.erase(pool.begin() + (std::ptrdiff_t)i);
          break;
        }
    }
    if (ev.device < 0) {
      SideEvents n;
      for (hipEvent_t *p : {&n.fork, &n.join, &n.xq_ready}) {
        if ((e = hipEventCreateWithFlags(p, hipEventDisableTiming)) != hipSuccess) {
          for (hipEvent_t q : {n.fork, n.join, n.xq_ready})
            if (q) (void)hipEventDestroy(q);
          return e;
        }
      }
      n.device = dev;
      ev = n;
    }
  }
  *out = &ev;
  return hipSuccess;
}

// The k smallest primes above m (trial division; m < 2^31, k <= 16).
void primes_above(int64_t m, int k, int64_t *out) {
  int have = 0;
  for (int64_t q = m + 1; have < k; ++q) {
    bool prime = q >= 2;
    for (int64_t d = 2; prime && d * d <= q; ++d)
      if (q % d == 0) prime = false;
    if (prime) out[have++] = q;
  }
}

// The greedy least-loaded rule over tokens in `order` (tid2eid page,
// "Reference implementation"); writes table rows and returns the loads.
void greedy_in_order(const double *p, const int64_t *order, int64_t m, int32_t n, int32_t k,
                     int32_t *tid2eid, std::vector<double> &f) {
  f.assign(n, 0.0);
  std::vector<int32_t> pick(k);
  for (int64_t oi = 0; oi < m; ++oi) {
    const int64_t i = order[oi];
    // k smallest (load, id) pairs, kept sorted ascending by insertion
    int have = 0;
    for (int32_t j = 0; j < n; ++j) {
      const double fj = f[j];
      if (have == k && !(fj < f[pick[k - 1]])) continue;   // ids ascend: equal load loses
      int pos = have < k ? have : k - 1;
      while (pos > 0 && fj < f[pick[pos - 1]]) {
        pick[pos] = pick[pos - 1];
        --pos;
      }
      pick[pos] = j;
      if (have < k) ++have;
    }
    const double share = p[i] / (double)k;
    for (int q = 0; q < k; ++q) {
      f[pick[q]] += share;
      tid2eid[i * k + q] = pick[q];
    }
  }
}

// Device memory of moe_forward_noalloc: one array per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: its address on each device comes from hipGetSymbolAddress,
// taken once per device (with that device current) on the first call there,
// and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex &scratch_mutex() {
  static std::mutex *m = new std::mutex;
  return *m;
}

hipError_t scratch_address(void **out) {
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex());
  if (!addr[dev]) {
    void *p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

void max_min(const std::vector<double> &f, double *mx, double *mn) {
  *mx = f[0];
  *mn = f[0];
  for (size_t j = 1; j < f.size(); ++j) {
    *mx = std::max(*mx, f[j]);
    *mn = std::min(*mn, f[j]);
  }
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int moe_validate_config(const moe_config *cfg) { return validate(cfg); }

int moe_build_tid2eid(const double *p, int64_t m, int32_t n, int32_t k, int32_t *tid2eid,
                      double *load, double *max_vio, double *min_vio) {
  if (!p || !tid2eid || m < 1 || n < 1 || k < 1 || k > n) return MOE_ERR_INVALID_ARG;
  for (int64_t i = 0; i < m; ++i)
    if (!(p[i] >= 0.0) || std::isinf(p[i])) return MOE_ERR_INVALID_ARG;
  // tokens by decreasing frequency, equal frequencies by ascending id
  std::vector<int64_t> order(m);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [p](int64_t a, int64_t b) { return p[a] > p[b]; });
  std::vector<double> f;
  greedy_in_order(p, order.data(), m, n, k, tid2eid, f);
  double mx, mn;
  max_min(f, &mx, &mn);
  if (load) std::copy(f.begin(), f.end(), load);
  if (max_vio) *max_vio = mx * n - 1.0;
  if (min_vio) *min_vio = mn * n - 1.0;
  return MOE_OK;
}

int moe_workspace_layout(const moe_config *cfg, int64_t T, moe_ws_layout *layout) {
  return make_layout(cfg, T, layout);
}

size_t moe_workspace_size(const moe_config *cfg, int64_t T) {
  moe_ws_layout l;
  return make_layout(cfg, T, &l) == MOE_OK ? l.total_bytes : 0;
}

int moe_build_tid2eid_multistart(const double *p, int64_t m, int32_t n, int32_t k,
                                 const int64_t *orders, int32_t n_starts, int32_t *tid2eid,
                                 double *load, double *max_vio, double *min_vio,
                                 int32_t *best_start) {
  if (!p || !tid2eid || !orders || m < 1 || n < 1 || k < 1 || k > n || n_starts < 1)
    return MOE_ERR_INVALID_ARG;
  for (int64_t i = 0; i < m; ++i)
    if (!(p[i] >= 0.0) || std::isinf(p[i])) return MOE_ERR_INVALID_ARG;
  std::vector<char> seen(m);
  for (int32_t s = 0; s < n_starts; ++s) {
    std::fill(seen.begin(), seen.end(), 0);
    for (int64_t i = 0; i < m; ++i) {
      const int64_t v = orders[s * m + i];
      if (v < 0 || v >= m || seen[v]) return MOE_ERR_INVALID_ARG;
      seen[v] = 1;
    }
  }
  std::vector<int32_t> table((size_t)m * k);
  std::vector<double> f, best_f;
  double best_mx = 0.0;
  int32_t best = -1;
  for (int32_t s = 0; s < n_starts; ++s) {
    greedy_in_order(p, orders + s * m, m, n, k, table.data(), f);
    double mx, mn;
    max_min(f, &mx, &mn);
    const double vio = mx * n - 1.0;
    if (best < 0 || vio < best_mx) {
      best = s;
      best_mx = vio;
      best_f = f;
      std::copy(table.begin(), table.end(), tid2eid);
    }
  }
  double mx, mn;
  max_min(best_f, &mx, &mn);
  if (load) std::copy(best_f.begin(), best_f.end(), load);
  if (max_vio) *max_vio = mx * n - 1.0;
  if (min_vio) *min_vio = mn * n - 1.0;
  if (best_start) *best_start = best;
  return MOE_OK;
}

int moe_update_bias(const moe_config *cfg, const int32_t *counts, int64_t T, float gamma,
                    float *bias, double *stats, void *stream) {
  const int st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!counts || !bias || T < 1 || !std::isfinite(gamma)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_update_bias(counts, cfg->n_routed_experts, T,
                                            cfg->n_activated_experts, gamma, bias, stats,
                                            (hipStream_t)stream));
}

int moe_route(const moe_config *cfg, const moe_weights *w, const void *x,
              const int32_t *token_ids, int64_t T, float *weights, int32_t *indices,
              void *stream) {
  int st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!w || T < 0 || (T > 0 && (!weights || !indices))) return MOE_ERR_INVALID_ARG;
  if (T * cfg->n_activated_experts > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (cfg->route_mode == MOE_ROUTE_HASH) {
    if (!token_ids || !w->tid2eid) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_route_hash(*cfg, token_ids, w->tid2eid, T, weights, indices,
                                             nullptr, s));
  }
  if (cfg->route_mode == MOE_ROUTE_NGRAM_HASH) {
    if (!token_ids) return MOE_ERR_INVALID_ARG;
    int64_t q[16];
    primes_above(cfg->vocab_size, cfg->n_activated_experts, q);
    return hip_status(moe::launch_route_ngram(*cfg, token_ids, q, T, weights, indices, nullptr, s));
  }
  if (!x || !w->gate_w) return MOE_ERR_INVALID_ARG;
  return hip_status(
      moe::launch_route_learned(*cfg, x, w->gate_w, w->gate_bias, T, weights, indices, s));
}

int moe_permute(const moe_config *cfg, const int32_t *indices, int64_t T, int32_t *counts,
                int32_t *offsets, int32_t *sorted_tok, int32_t *sorted_slot, int32_t *inverse,
                uint32_t *flags, void *stream) {
  int st = validate(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!indices || !sorted_tok || !sorted_slot || !inverse)) return MOE_ERR_INVALID_ARG;
  if (T * cfg->n_activated_experts > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_permute(cfg->n_routed_experts, cfg->n_activated_experts, T,
                                        indices, counts, offsets, sorted_tok, sorted_slot,
                                        inverse, flags, nullptr, false, (hipStream_t)stream));
}

static int forward_impl(const moe_config *cfg, const moe_weights *w, const void *x,
                        const int32_t *token_ids, int64_t T, void *y, void *ws, size_t ws_bytes,
                        hipEvent_t *events, void *stream, void *side_stream) {
  moe_ws_layout L;
  int st = make_layout(cfg, T, &L);
  if (st != MOE_OK) return st;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !y || x == y) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
  if ((cfg->expert_dtype == MOE_DTYPE_FP4_E2M1 || cfg->expert_dtype == MOE_DTYPE_FP8_E4M3_B128) &&
      (!w->s_gate || !w->s_up || !w->s_down))
    return MOE_ERR_INVALID_ARG;
  if (cfg->n_shared_experts == 1 && (!w->sh_gate || !w->sh_up || !w->sh_down))
    return MOE_ERR_INVALID_ARG;
  if (cfg->route_mode == MOE_ROUTE_HASH) {
    if (!token_ids || !w->tid2eid) return MOE_ERR_INVALID_ARG;
  } else if (cfg->route_mode == MOE_ROUTE_NGRAM_HASH) {
    if (!token_ids) return MOE_ERR_INVALID_ARG;
  } else if (!w->gate_w) {
    return MOE_ERR_INVALID_ARG;
  }
  if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < L.total_bytes) return MOE_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)ws;
  float *route_w = (float *)(base + L.route_weights);
  int32_t *route_idx = (int32_t *)(base + L.route_indices);
  int32_t *counts = (int32_t *)(base + L.counts);
  int32_t *offsets = (int32_t *)(base + L.offsets);
  int32_t *sorted_tok = (int32_t *)(base + L.sorted_tok);
  int32_t *sorted_slot = (int32_t *)(base + L.sorted_slot);
  float *sorted_w = (float *)(base + L.sorted_weight);
  int32_t *inverse = (int32_t *)(base + L.inverse);
  int32_t *tiles = (int32_t *)(base + L.tiles);
  int32_t *tile_count = (int32_t *)(base + L.tile_count);
  uint32_t *flags = (uint32_t *)(base + L.flags);
  float *logits = (float *)(base + L.route_logits);
  int32_t *perm_hist = (int32_t *)(base + L.perm_hist);
  const int k = cfg->n_activated_experts;
  const bool hash = cfg->route_mode != MOE_ROUTE_LEARNED;

  const int n_shared_tiles =
      cfg->n_shared_experts ? (int)((T + L.tile_rows - 1) / L.tile_rows) : 0;
  moe::ExpertPlan p;
  p.T = T;
  p.k = k;
  p.E = cfg->n_routed_experts;
  p.dim = cfg->dim;
  p.inter = cfg->moe_inter_dim;
  p.has_shared = cfg->n_shared_experts == 1;
  p.swiglu_limit = cfg->swiglu_limit;
  p.act_dtype = cfg->act_dtype;
  p.expert_dtype = cfg->expert_dtype;
  p.tiled = cfg->weight_layout == MOE_LAYOUT_TILED;
  p.mx = cfg->act_quant == MOE_ACT_QUANT_MXFP8;
  p.xq = (uint8_t *)(base + L.xq);
  p.xq_scales = (uint8_t *)(base + L.xq_scales);
  p.hq = (uint8_t *)(base + L.hq);
  p.hq_scales = (uint8_t *)(base + L.hq_scales);
  p.x = x;
  p.w = w;
  p.route_w = route_w;
  p.route_idx = route_idx;
  p.offsets = offsets;
  p.sorted_tok = sorted_tok;
  p.sorted_slot = sorted_slot;
  p.sorted_w = sorted_w;
  p.inverse = inverse;
  p.tiles = tiles;
  p.tile_count = tile_count;
  p.max_tiles = L.max_tiles;
  p.tile_rows = L.tile_rows;
  p.n_shared_tiles = n_shared_tiles;
  p.h = base + L.h;
  p.yrows = base + L.yrows;
  p.y = y;
  p.events = events;
  p.shared_done = nullptr;
  p.xq_ready = nullptr;

  // With a side stream, FP4 / FP8 expert layers put the shared expert (bf16,
  // launches of its own) and the MXFP8 copy of x, which need x alone, on it:
  // forked from s here, so they run while the routing and the permutation
  // (latency-bound, most CUs idle) run on s; s waits for x's copy before the
  // routed up GEMM and joins the side stream before the combine.  bf16 expert
  // layers keep the shared tiles inside the grouped launches, where they
  // share the CUs with the HBM-bound routed tiles (on a side stream the
  // shared dense GEMM held every CU and delayed the routing: 2 % slower at
  // the V3 prefill shape), and ignore the side stream.
  hipError_t e;
  const bool low_precision = cfg->expert_dtype == MOE_DTYPE_FP4_E2M1 ||
                             cfg->expert_dtype == MOE_DTYPE_FP8_E4M3_B128;
  // Once the side stream is forked, every return joins it back into s first
  // (the join recorded again after whatever reached the side stream), so no
  // side work is left unordered against the caller's next work on s, also
  // when a launch fails.
  hipStream_t s2 = nullptr;
  SideEvents *side = nullptr;
  auto finish = [&](int status) {
    if (side) {
      (void)hipEventRecord(side->join, s2);
      (void)hipStreamWaitEvent(s, side->join, 0);
    }
    return status;
  };
  if (side_stream && cfg->act_dtype == MOE_DTYPE_BF16 && low_precision &&
      (p.has_shared || p.mx)) {
    s2 = (hipStream_t)side_stream;
    SideEvents *ev = nullptr;
    if (side_events(&ev) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventRecord(ev->fork, s) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamWaitEvent(s2, ev->fork, 0) != hipSuccess) return MOE_ERR_HIP;
    side = ev;
    if (moe::launch_shared_expert(p, s2, side->xq_ready) != hipSuccess ||
        hipEventRecord(side->join, s2) != hipSuccess)
      return finish(MOE_ERR_HIP);
    p.shared_done = side->join;
    p.xq_ready = p.mx ? side->xq_ready : nullptr;
  }

  if (events && hipEventRecord(events[MOE_STAGE_ROUTE], s) != hipSuccess)
    return finish(MOE_ERR_HIP);
  if (hash) {
    if ((e = moe::launch_clear_flags(flags, s)) != hipSuccess) return finish(MOE_ERR_HIP);
    if (cfg->route_mode == MOE_ROUTE_NGRAM_HASH) {
      int64_t q[16];
      primes_above(cfg->vocab_size, k, q);
      e = moe::launch_route_ngram(*cfg, token_ids, q, T, route_w, route_idx, flags, s);
    } else {
      e = moe::launch_route_hash(*cfg, token_ids, w->tid2eid, T, route_w, route_idx, flags, s);
    }
  } else {
    e = moe::launch_route_learned(*cfg, x, w->gate_w, w->gate_bias, T, route_w, route_idx, s,
                                  moe::route_logits_floats(*cfg, T) ? logits : nullptr);
  }
  if (e != hipSuccess) return finish(MOE_ERR_HIP);

  moe::TileSpec ts;
  ts.tiles = tiles;
  ts.tile_count = tile_count;
  ts.tile_rows = L.tile_rows;
  ts.n_shared_tiles = n_shared_tiles;
  ts.shared_rows_tok = sorted_tok + T * k;
  ts.route_w = route_w;
  ts.sorted_w = sorted_w;
  if (events && hipEventRecord(events[MOE_STAGE_PERMUTE], s) != hipSuccess)
    return finish(MOE_ERR_HIP);
  e = moe::launch_permute(cfg->n_routed_experts, k, T, route_idx, counts, offsets, sorted_tok,
                          sorted_slot, inverse, flags, &ts, /*clear_flags=*/!hash, s, perm_hist);
  if (e != hipSuccess) return finish(MOE_ERR_HIP);
  if (moe::launch_experts(p, s) != hipSuccess) return finish(MOE_ERR_HIP);
  return MOE_OK;
}

int moe_pack_weights(const moe_config *cfg, const moe_weights *src, const moe_weights *dst,
                     void *stream) {
  if (!cfg || !src || !dst) return MOE_ERR_INVALID_ARG;
  moe_config c = *cfg;
  c.weight_layout = MOE_LAYOUT_ROWS;
  const int st = validate(&c);
  if (st != MOE_OK) return st;
  if (c.act_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  const int64_t E = c.n_routed_experts, d = c.dim, I = c.moe_inter_dim;
  const int ed = c.expert_dtype;
  struct Job { const void *s; const void *d; int64_t count, N, K; int dtype; bool scales; };
  const Job jobs[] = {
      {src->w_gate, dst->w_gate, E, I, d, ed, false},
      {src->w_up, dst->w_up, E, I, d, ed, false},
      {src->w_down, dst->w_down, E, d, I, ed, false},
      {ed == MOE_DTYPE_FP4_E2M1 ? src->s_gate : nullptr, dst->s_gate, E, I, d, ed, true},
      {ed == MOE_DTYPE_FP4_E2M1 ? src->s_up : nullptr, dst->s_up, E, I, d, ed, true},
      {ed == MOE_DTYPE_FP4_E2M1 ? src->s_down : nullptr, dst->s_down, E, d, I, ed, true},
      {src->sh_gate, dst->sh_gate, 1, I, d, MOE_DTYPE_BF16, false},
      {src->sh_up, dst->sh_up, 1, I, d, MOE_DTYPE_BF16, false},
      {src->sh_down, dst->sh_down, 1, d, I, MOE_DTYPE_BF16, false},
  };
  for (const Job &j : jobs)
    if (j.s && (!j.d || j.d == j.s)) return MOE_ERR_INVALID_ARG;
  for (const Job &j : jobs) {
    if (!j.s) continue;
    const hipError_t e = moe::launch_pack_matrix(j.s, const_cast<void *>(j.d), j.count, j.N,
                                                 j.K, j.dtype, j.scales, (hipStream_t)stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

int moe_redequant_fp8(const uint8_t *codes, const uint8_t *scales, int64_t n_mat, int32_t N,
                      int32_t K, uint8_t *fp8, uint8_t *block_scales, uint8_t *lossy,
                      void *stream) {
  if (n_mat < 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (N % 128 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (n_mat == 0) return MOE_OK;
  if (!codes || !scales || !fp8 || !block_scales || !lossy) return MOE_ERR_INVALID_ARG;
  if (n_mat * (N / 128) * (int64_t)(K / 128) > (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_redequant_fp8(codes, scales, n_mat, N, K, fp8, block_scales, lossy,
                                              (hipStream_t)stream));
}

int moe_forward(const moe_config *cfg, const moe_weights *w, const void *x,
                const int32_t *token_ids, int64_t T, void *y, void *ws, size_t ws_bytes,
                void *stream) {
  return forward_impl(cfg, w, x, token_ids, T, y, ws, ws_bytes, nullptr, stream, nullptr);
}

int moe_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                        const int32_t *token_ids, int64_t T, void *y, void *stream) {
  moe_ws_layout L;
  const int st = make_layout(cfg, T, &L);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (L.total_bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
  return forward_impl(cfg, w, x, token_ids, T, y, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, nullptr,
                      stream, nullptr);
}

int moe_forward_profiled(const moe_config *cfg, const moe_weights *w, const void *x,
                         const int32_t *token_ids, int64_t T, void *y, void *ws,
                         size_t ws_bytes, void **events, void *stream) {
  if (!events) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i <= MOE_STAGE_COUNT; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, w, x, token_ids, T, y, ws, ws_bytes, (hipEvent_t *)events, stream,
                      nullptr);
}

int moe_forward_ex(const moe_config *cfg, const moe_weights *w, const void *x,
                   const int32_t *token_ids, int64_t T, void *y, void *ws, size_t ws_bytes,
                   void **events, void *stream, void *side_stream) {
  if (events)
    for (int i = 0; i <= MOE_STAGE_COUNT; ++i)
      if (!events[i]) return MOE_ERR_INVALID_ARG;
  if (side_stream && side_stream == stream) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, w, x, token_ids, T, y, ws, ws_bytes, (hipEvent_t *)events, stream,
                      side_stream);
}

int moe_probe_read(const void *buf, int64_t bytes, void *out, void *stream) {
  if (!buf || !out || bytes < 16 || bytes % 16 || ((uintptr_t)buf % 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_probe_read(buf, bytes, (uint32_t *)out, (hipStream_t)stream));
}

int moe_probe_mfma(int32_t iters, int32_t shape, void *out, double *flops, void *stream) {
  if (!out || iters < 1 || shape < 0 || shape > 3) return MOE_ERR_INVALID_ARG;
  if (flops) *flops = (double)moe::probe_mfma_flops(iters, shape);
  return hip_status(moe::launch_probe_mfma(iters, shape, (float *)out, (hipStream_t)stream));
}

}  // extern "C"
