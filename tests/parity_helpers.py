"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same synthetic inputs, compare."""

import itertools

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp4": 5e-2}     # max relative error of y
WEIGHT_RTOL = 1e-5                                  # routing weights
TIE_RTOL = 1e-6                                     # near-tie exemption


def f64(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def cpu_np(t):
    return t.detach().cpu().numpy()


def expert_fetcher(layer, cfg, fp8=False):
    """expert(e) -> float64 (w_gate, w_up, w_down), decoded by the oracle for FP4
    (fp8: the oracle's FP8 re-dequantisation of the FP4 matrices)."""
    def get(e):
        if fp8:
            out = []
            for n, s in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")):
                c, b, _ = oracle.fp4_to_fp8_blocks(cpu_np(layer[n][e]), cpu_np(layer[s][e]))
                out.append(oracle.fp8_blocks_decode(c, b))
            return tuple(out)
        if cfg.expert_dtype == "fp4":
            return (oracle.fp4_decode(cpu_np(layer["w_gate"][e]), cpu_np(layer["s_gate"][e])),
                    oracle.fp4_decode(cpu_np(layer["w_up"][e]), cpu_np(layer["s_up"][e])),
                    oracle.fp4_decode(cpu_np(layer["w_down"][e]), cpu_np(layer["s_down"][e])))
        return f64(layer["w_gate"][e]), f64(layer["w_up"][e]), f64(layer["w_down"][e])
    return get


class PrefetchedExperts:
    """expert(e) for the oracle's layer loop over a known list of experts
    (ascending ids, the order the oracle asks for them): the float64 weights
    of the next few experts are prepared in worker threads while the current
    one is used.  fp8: the oracle's FP4 -> FP8 re-dequantisation (a Python loop
    over 128 x 128 blocks) runs in spawned worker processes, which import only
    the oracle (no torch, no GPU); the decode stays here.  Prints a line every `report` experts."""

    def __init__(self, layer, cfg, experts, fp8=False, threads=8, procs=16, ahead=12,
                 report=64, label=""):
        from concurrent.futures import ProcessPoolExecutor, ThreadPoolExecutor
        self.layer, self.cfg, self.fp8 = layer, cfg, fp8
        self.order = [int(e) for e in experts]
        self.threads = ThreadPoolExecutor(threads)
        self.procs = None
        if fp8:
            import multiprocessing
            self.procs = ProcessPoolExecutor(procs, mp_context=multiprocessing.get_context("spawn"))
        self.plain = expert_fetcher(layer, cfg)
        self.pending = {}
        self.next = 0
        self.ahead = ahead
        self.done = 0
        self.report = report
        self.label = label
        for _ in range(ahead):
            self._submit()

    def _submit(self):
        if self.next < len(self.order):
            e = self.order[self.next]
            self.next += 1
            self.pending[e] = self.threads.submit(self._get, e)

    def _get(self, e):
        if not self.fp8:
            return self.plain(e)
        futs = [self.procs.submit(oracle.fp4_to_fp8_blocks, cpu_np(self.layer[n][e]),
                                  cpu_np(self.layer[s][e]))
                for n, s in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down"))]
        return tuple(oracle.fp8_blocks_decode(*f.result()[:2]) for f in futs)

    def __call__(self, e):
        e = int(e)
        fut = self.pending.pop(e, None)
        out = fut.result() if fut is not None else self._get(e)
        self._submit()
        self.done += 1
        if self.report and self.done % self.report == 0:
            print(f"[oracle]{' ' + self.label if self.label else ''}: {self.done} of "
                  f"{len(self.order)} experts", flush=True)
        return out

    def close(self):
        self.threads.shutdown(wait=True, cancel_futures=True)
        if self.procs is not None:
            self.procs.shutdown(wait=True, cancel_futures=True)


def shared_weights(layer, cfg):
    if not cfg.n_shared_experts:
        return None
    return f64(layer["sh_gate"]), f64(layer["sh_up"]), f64(layer["sh_down"])


def oracle_route(cfg, layer, tid2eid_oracle=None, rows=None):
    """Oracle routing of all tokens (or of `rows`)."""
    if cfg.route_mode == "hash":
        ids = cpu_np(layer["token_ids"]).astype(np.int64)
        if rows is not None:
            ids = ids[rows]
        w, idx = oracle.hash_gate(ids, tid2eid_oracle, cfg.route_scale)
        return w, idx, None
    if cfg.route_mode == "ngram":
        pairs = cpu_np(layer["token_ids"]).astype(np.int64)
        if rows is not None:
            pairs = pairs[rows]
        w, idx = oracle.ngram_hash_gate(pairs[:, 0], pairs[:, 1], cfg.vocab_size,
                                        cfg.n_routed_experts, cfg.n_activated_experts,
                                        cfg.route_scale)
        return w, idx, None
    x = f64(layer["x"]) if rows is None else f64(layer["x"][torch.as_tensor(rows)])
    bias = None if layer["gate_bias"] is None else cpu_np(layer["gate_bias"])
    return oracle.learned_gate(
        x, f64(layer["gate_w"]), bias, score_func=cfg.score_func, n_groups=cfg.n_expert_groups,
        topk_groups=cfg.n_limited_groups, topk=cfg.n_activated_experts,
        route_scale=cfg.route_scale, renormalize=cfg.renormalize)


def _close(a, b):
    """a and b within the 1e-6 relative tie band (elementwise)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b) <= TIE_RTOL * np.maximum(np.abs(a), np.abs(b))


def _kept_group_candidates(cfg, gscores):
    """Every set of kept groups the 1e-6 band allows for one token: the groups
    whose score is clearly above the g-th largest are always kept, the rest of
    the g are any choice among the groups whose score ties the g-th one."""
    G, g = cfg.n_expert_groups, cfg.n_limited_groups
    if G <= 1 or g >= G:
        return [np.arange(max(G, 1))]
    gs = np.asarray(gscores, dtype=np.float64)
    gth = np.sort(gs)[::-1][g - 1]
    band = _close(gs, gth)
    sure = np.nonzero((gs > gth) & ~band)[0]
    tied = np.nonzero(band)[0]
    need = g - sure.size
    return [np.concatenate([sure, np.asarray(c, dtype=np.int64)])
            for c in itertools.combinations(tied, need)]


def _valid_topk(cfg, keys, sel, kept_groups):
    """sel (GPU ids in slot order) is a top-k of the fp32 selection keys with
    all groups outside kept_groups masked: every selected expert is in a kept
    group, no eligible unselected key exceeds a selected one by more than the
    tie band, and the slot order descends in key up to the band."""
    E = keys.shape[0]
    per = E // max(cfg.n_expert_groups, 1)
    eligible = np.zeros(E, dtype=bool)
    for grp in kept_groups:
        eligible[grp * per:(grp + 1) * per] = True
    if not eligible[sel].all():
        return False
    ks = keys[sel].astype(np.float64)
    rest = np.ones(E, dtype=bool)
    rest[sel] = False
    rest &= eligible
    if rest.any():
        top_rest = keys[rest].astype(np.float64).max()
        low = ks.min()
        if top_rest > low and not _close(top_rest, low):
            return False
    for j in range(ks.size - 1):
        if ks[j] < ks[j + 1] and not _close(ks[j], ks[j + 1]):
            return False
    return True


class RoutingCheck:
    """Outcome of check_routing: the GPU's indices (validated), the oracle's
    weights at those indices, and the tokens whose indices differ from the
    oracle's own choice (every one of them validated inside the tie band)."""

    def __init__(self, idx, ref_w, differ):
        self.idx = idx
        self.ref_w = ref_w
        self.differ = differ


def check_routing(cfg, gpu_w, gpu_idx, ora_w, ora_idx, aux, label=""):
    """GPU routing against the oracle's.

    Indices: equal to the oracle's for every token, except that learned
    routing may differ where the pages leave the choice open, inside a 1e-6
    relative tie band (on the oracle's fp32 keys): the k-th / (k+1)-th
    keys, the g-th / (g+1)-th group scores, or the slot order of two selected
    experts.  Every differing token is validated rather than skipped: k
    distinct ids in [0, E); all of them in a set of kept groups that the band
    allows; no unselected eligible key above a selected one beyond the band
    (so the set equals the oracle's up to swaps inside the band); slot order
    descending up to the band.  At most 1 % of the tokens may differ.

    Weights: for every token, against the oracle's affinity at the GPU's
    indices (renormalised over them unless softmax, times route_scale), to
    WEIGHT_RTOL relative, or for learned routing to 16 fp32 ulps of the
    token's largest |logit| where that is larger (the logits are fp32 sums, a
    few ulps of max|z| off, and a weight's relative error is the absolute
    error of its logits, up to 4x through a softmax and the renormalisation).

    Returns a RoutingCheck; its (idx, ref_w) are the routing the oracle layer
    is then evaluated on for every token."""
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    ora_idx = np.asarray(ora_idx, dtype=np.int64)
    T, k = ora_idx.shape
    E = cfg.n_routed_experts
    assert gpu_idx.shape == (T, k)
    assert np.all((gpu_idx >= 0) & (gpu_idx < E)), "expert id out of range"
    differ = np.any(gpu_idx != ora_idx, axis=1)
    ref_w = np.array(ora_w, dtype=np.float64, copy=True)
    bad = np.nonzero(differ)[0]
    if bad.size:
        assert aux is not None, (
            f"{bad.size} tokens routed differently by a table or hash rule, e.g. token "
            f"{bad[0]}: gpu {gpu_idx[bad[0]]} oracle {ora_idx[bad[0]]}")
        assert bad.size <= max(2, 0.01 * T), f"too many tokens in the tie band: {bad.size}"
        renorm = (cfg.score_func != "softmax") if cfg.renormalize < 0 else bool(cfg.renormalize)
        for t in bad:
            sel = gpu_idx[t]
            assert np.unique(sel).size == k, f"token {t}: repeated expert {sel}"
            keys = np.asarray(aux["keys"][t], dtype=np.float32)
            ok = any(_valid_topk(cfg, keys, sel, kg)
                     for kg in _kept_group_candidates(cfg, aux["group_scores"][t]))
            assert ok, (f"token {t}: gpu {sel} is not a top-{k} of the oracle keys within the "
                        f"1e-6 band (oracle {ora_idx[t]}; keys gpu "
                        f"{keys[sel]} oracle {keys[ora_idx[t]]})")
            s = np.asarray(aux["scores"][t], dtype=np.float64)[sel]
            if renorm:
                s = s / s.sum()
            ref_w[t] = s * cfg.route_scale
    gw = np.asarray(gpu_w, dtype=np.float64)
    rtol = np.full(T, WEIGHT_RTOL)
    if aux is not None and "logits" in aux:
        zmax = np.max(np.abs(np.asarray(aux["logits"], dtype=np.float64)), axis=1)
        rtol = np.maximum(rtol, 16.0 * 2.0 ** -24 * zmax)
    err = np.abs(gw - ref_w)
    lim = rtol[:, None] * np.abs(ref_w) + 1e-7
    assert np.all(err <= lim), (
        f"routing weight off by {np.max(err / lim):.2f} x its tolerance "
        f"(token {np.argmax(np.max(err / lim, axis=1))})")
    print(f"[routing]{' ' + label if label else ''}: {bad.size} of {T} tokens differ from the "
          f"oracle inside the 1e-6 tie band, all {bad.size} validated; weights of all "
          f"{T} tokens checked", flush=True)
    return RoutingCheck(gpu_idx, ref_w, differ)


def check_permutation_exact(idx, E, counts, offsets, sorted_tok, sorted_slot, inverse):
    """The permutation of the (validated) routing idx equals the oracle's
    permutation of the same indices, bit for bit."""
    T, k = idx.shape
    oc, oo, ost, oss, oinv = oracle.permute(idx, E)
    np.testing.assert_array_equal(counts, oc)
    np.testing.assert_array_equal(offsets, oo)
    np.testing.assert_array_equal(np.asarray(sorted_tok)[:T * k], ost)
    np.testing.assert_array_equal(np.asarray(sorted_slot)[:T * k], oss)
    np.testing.assert_array_equal(np.asarray(inverse).reshape(T, k), oinv)


def oracle_forward(cfg, x, weights, indices, layer, fp8=False, prefetch=False, label=""):
    """The oracle layer for cfg: bf16 activations, or MXFP8 activations on the
    routed FP4 experts (fp8: on their FP8 re-dequantisation).  prefetch: the
    experts' float64 weights are prepared ahead in workers (large layers)."""
    f = oracle.layer_forward_mx if cfg.act_quant == "mxfp8" else oracle.layer_forward
    if not prefetch:
        return f(x, weights, indices, expert_fetcher(layer, cfg, fp8), shared_weights(layer, cfg),
                 cfg.swiglu_limit)
    get = PrefetchedExperts(layer, cfg, np.unique(np.asarray(indices)), fp8=fp8, label=label)
    try:
        return f(x, weights, indices, get, shared_weights(layer, cfg), cfg.swiglu_limit)
    finally:
        get.close()


def check_layer_output(cfg, y_gpu, y_ref, label=""):
    """Layer output bars: max|y - y_ref| / max|y_ref| over the tensor within the
    dtype's bar, and every token's row within twice the bar against its own
    largest reference value (so one bad token is not hidden by a large
    neighbour)."""
    tol = TOL[cfg.expert_dtype if cfg.expert_dtype == "fp4" else cfg.act_dtype]
    err = max_rel_err(y_gpu, y_ref)
    denom = np.max(np.abs(y_ref), axis=1)
    row_err = np.max(np.abs(y_gpu - y_ref), axis=1) / np.where(denom > 0, denom, 1.0)
    worst = int(np.argmax(row_err)) if row_err.size else 0
    print(f"[output]{' ' + label if label else ''}: {y_ref.shape[0]} tokens, max rel err "
          f"{err:.3e} (bar {tol}), worst token {worst} at {row_err[worst] if row_err.size else 0:.3e}",
          flush=True)
    assert err <= tol
    assert np.all(row_err <= 2 * tol), f"token {worst}: {row_err[worst]:.3e}"


def run_weights(wl, cfg, layer, B):
    """(config, layer) the GPU runs for a workload: the FP8 re-dequantisation
    of an FP4 layer when the workload asks for it (no block may be lossy for
    the synthetic weights), else the layer as given."""
    if not wl.fp8_weights:
        return cfg, layer
    cfg8, layer8, lossy = B.redequant_layer(cfg, layer)
    assert lossy == 0
    return cfg8, layer8


def max_rel_err(y, ref):
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / denom) if denom > 0 else float(np.max(np.abs(y)))


def check_permutation_valid(indices, E, counts, offsets, sorted_tok, sorted_slot, inverse):
    """Properties that pin a permutation by expert whatever the routing."""
    indices = np.asarray(indices, dtype=np.int64)
    T, k = indices.shape
    np.testing.assert_array_equal(counts, np.bincount(indices.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets[:-1], np.concatenate([[0], np.cumsum(counts)[:-1]]))
    assert offsets[-1] == T * k
    sorted_tok = np.asarray(sorted_tok[:T * k], dtype=np.int64)
    sorted_slot = np.asarray(sorted_slot[:T * k], dtype=np.int64)
    # every row holds a pair of its segment's expert, tokens ascending (stable)
    experts_of_rows = indices[sorted_tok, sorted_slot]
    seg = np.repeat(np.arange(E), counts)
    np.testing.assert_array_equal(experts_of_rows, seg)
    key = sorted_tok * k + sorted_slot
    for e in range(E):
        s = key[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(s) > 0)
    inverse = np.asarray(inverse, dtype=np.int64).reshape(T, k)
    np.testing.assert_array_equal(sorted_tok[inverse.ravel()], np.repeat(np.arange(T), k))
    np.testing.assert_array_equal(sorted_slot[inverse.ravel()], np.tile(np.arange(k), T))
