"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same synthetic inputs, compare."""

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


def near_tie_tokens(cfg, aux):
    """Tokens whose routing is not unique at the north-star's 1e-6 relative
    tolerance: among the top k+1 fp32 keys (after the group mask) two
    neighbours are that close, or the kept/dropped group scores are."""
    if aux is None:
        return np.zeros(0, dtype=bool)
    keys = aux["masked_keys"].astype(np.float64)
    T = keys.shape[0]
    k = cfg.n_activated_experts
    tie = np.zeros(T, dtype=bool)
    for t in range(T):
        row = np.sort(keys[t])[::-1][:k + 1]
        row = row[np.isfinite(row)]
        gaps = np.abs(np.diff(row))
        scale = np.maximum(np.abs(row[:-1]), np.abs(row[1:]))
        if np.any(gaps <= TIE_RTOL * scale):
            tie[t] = True
    if cfg.n_expert_groups > 1:
        gs = np.sort(aux["group_scores"].astype(np.float64), axis=1)[:, ::-1]
        g = cfg.n_limited_groups
        if g < cfg.n_expert_groups:
            a, b = gs[:, g - 1], gs[:, g]
            tie |= np.abs(a - b) <= TIE_RTOL * np.maximum(np.abs(a), np.abs(b))
    return tie


def compare_routing(cfg, gpu_w, gpu_idx, ora_w, ora_idx, aux):
    """Bit-exact indices except near-tie tokens; weights to WEIGHT_RTOL
    relative (learned routing: to 16 ulps of the token's largest |logit| where
    that is larger).
    Returns the boolean mask of tokens whose routing differs (all exempt)."""
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    differ = np.any(gpu_idx != ora_idx, axis=1)
    if differ.any():
        tie = near_tie_tokens(cfg, aux)
        bad = np.nonzero(differ & ~tie)[0]
        assert bad.size == 0, (
            f"{bad.size} tokens routed differently without a near tie, e.g. token {bad[0]}: "
            f"gpu {gpu_idx[bad[0]]} oracle {ora_idx[bad[0]]}")
        assert differ.sum() <= max(2, 0.01 * differ.size), f"too many near-tie tokens: {differ.sum()}"
    same = ~differ
    gw = np.asarray(gpu_w, dtype=np.float64)[same]
    ow = np.asarray(ora_w, dtype=np.float64)[same]
    rtol = np.full(gw.shape[0], WEIGHT_RTOL)
    if aux is not None and "logits" in aux:
        # learned routing: the GPU's logits are fp32 sums, a few ulps of the
        # token's largest |z| off, and a weight's relative error is the
        # absolute error of its logits (up to 4x through a softmax and the
        # renormalisation): 16 ulps of max |z|, floored at WEIGHT_RTOL
        zmax = np.max(np.abs(np.asarray(aux["logits"], dtype=np.float64)), axis=1)[same]
        rtol = np.maximum(rtol, 16.0 * 2.0 ** -24 * zmax)
    err = np.abs(gw - ow)
    lim = rtol[:, None] * np.abs(ow) + 1e-7
    assert np.all(err <= lim), (
        f"routing weight off by {np.max(err / lim):.2f} x its tolerance "
        f"(token {np.argmax(np.max(err / lim, axis=1))} of the compared ones)")
    return differ


def oracle_forward(cfg, x, weights, indices, layer, fp8=False):
    """The oracle layer for cfg: bf16 activations, or MXFP8 activations on the
    routed FP4 experts (fp8: on their FP8 re-dequantisation)."""
    f = oracle.layer_forward_mx if cfg.act_quant == "mxfp8" else oracle.layer_forward
    return f(x, weights, indices, expert_fetcher(layer, cfg, fp8), shared_weights(layer, cfg),
             cfg.swiglu_limit)


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
