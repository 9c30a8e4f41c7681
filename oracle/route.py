"""Oracle: token -> expert routing (learned gate and hash gate).

Test infrastructure only (see the package docstring).

Learned gate, following "DeepSeek-V3.2-Exp - Routing weights", excerpt
"gate-forward", with the affinity choices of "From One Giant FFN to 384 Tiny
Experts" (Ch.4 softmax form, Ch.7 sigmoid, Ch.11.2 Sqrt(Softplus)) and the
selection-only bias of Ch.6:

  1. z = x . W^T, the fp32 linear of the page computed here exactly in fp64;
  2. s = affinity(z): softmax over experts, sigmoid, or sqrt(softplus);
  3. selection key b = s + bias (bias only perturbs the top-k cut);
  4. with groups: experts are split into n_groups contiguous ranges; a
     group's score is the sum of its two largest keys (the largest key when
     there is no bias); all but the topk_groups best groups are masked to -inf;
  5. the topk largest keys give the expert indices, in descending key order;
  6. weights = unbiased s at those indices, renormalised over the selected
     experts unless the affinity is softmax, then multiplied by route_scale.

Readings where the pages leave a step open:
  * the page adds the fp32 bias to fp32 scores and takes the cut on those
    fp32 values; the oracle does the same: the fp64 affinity is rounded once
    to fp32, the bias is added in fp32 and the group top-2 sums are fp32
    additions, so the integer decisions are taken in the page's precision;
  * torch.topk leaves equal keys unordered; here equal keys go to the lower
    expert (or group) index;
  * renormalise iff the affinity is not softmax (``renormalize=-1``), which
    is the code excerpt's rule extended to sqrt(softplus); 0/1 force it.

Hash gate ("How was DeepSeek V4's tid2eid derived?", background section, and
Ch.11.1 of the FFN history): indices = tid2eid[token_id]; every selected
expert gets weight route_scale / k (uniform 1/k at route_scale = 1).

2-gram hash gate ("How was DeepSeek V4's tid2eid derived?", section "An
extreme case"): expert j of the pair (previous id a, current id b) is
(a * q_j + b) mod n, q_j the j-th smallest prime above the vocabulary size.
Readings: no preceding token -> a = m; duplicates kept; weights
route_scale / k.  Pins: tests/test_oracle_ngram.py (hand-worked pairs in
tests/golden/ngram_small.json, the primes checked by an independent
Miller-Rabin test and gap scan, the a = 0 closed form, near-uniform loads on
random pairs).

Pins: tests/test_oracle_route.py (distinct ids, masked groups never win,
weight sums, full-sort agreement, monotone-affinity reduction to argsort of
the raw logits, g = G reduction, softmax closed form, bias-invariance of the
weights, hand-worked fixture tests/golden/route_small.json).
"""

import numpy as np

SCORE_FUNCS = ("softmax", "sigmoid", "sqrtsoftplus")


def affinity(z, score_func):
    """Affinity scores s from logits z [T, E] (float64)."""
    z = np.asarray(z, dtype=np.float64)
    if score_func == "softmax":
        zmax = z.max(axis=-1, keepdims=True)
        e = np.exp(z - zmax)
        return e / e.sum(axis=-1, keepdims=True)
    if score_func == "sigmoid":
        return 1.0 / (1.0 + np.exp(-z))
    if score_func == "sqrtsoftplus":
        # softplus(z) = log(1 + e^z), written in the overflow-free form
        softplus = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
        return np.sqrt(softplus)
    raise ValueError(f"unknown score_func {score_func!r}")


def selection_keys(s, bias):
    """fp32 selection keys: fp32(s) + bias, added in fp32 as on the page."""
    keys = np.asarray(s, dtype=np.float64).astype(np.float32)
    if bias is not None:
        keys = (keys + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    return keys


def _order_desc(values):
    """Positions sorted by value descending, equal values by position ascending."""
    values = np.asarray(values)
    pos = np.arange(values.shape[0])
    # lexsort sorts by the last key first; negate via ordering on -value
    return np.lexsort((pos, -values.astype(np.float64)))


def _group_scores(keys_row, n_groups, has_bias):
    per = keys_row.shape[0] // n_groups
    scores = np.empty(n_groups, dtype=np.float32)
    for g in range(n_groups):
        grp = keys_row[g * per:(g + 1) * per]
        if has_bias:
            top = np.sort(grp)[::-1]
            scores[g] = np.float32(top[0]) + np.float32(top[1])
        else:
            scores[g] = grp.max()
    return scores


def mask_groups(keys, n_groups, topk_groups, has_bias):
    """Apply the group limit: keys of non-kept groups become -inf.

    Returns (masked keys [T,E] fp32, kept-group mask [T,G] bool, group scores [T,G]).
    """
    keys = np.array(keys, dtype=np.float32, copy=True)
    T, E = keys.shape
    if n_groups <= 1:
        return keys, np.ones((T, 1), dtype=bool), keys.max(axis=1, keepdims=True)
    per = E // n_groups
    kept = np.zeros((T, n_groups), dtype=bool)
    gscores = np.empty((T, n_groups), dtype=np.float32)
    for t in range(T):
        gs = _group_scores(keys[t], n_groups, has_bias)
        gscores[t] = gs
        best = _order_desc(gs)[:topk_groups]
        kept[t, best] = True
        for g in range(n_groups):
            if not kept[t, g]:
                keys[t, g * per:(g + 1) * per] = -np.inf
    return keys, kept, gscores


def learned_gate(x, gate_w, bias, *, score_func, n_groups, topk_groups, topk,
                 route_scale, renormalize=-1):
    """Learned routing for tokens x [T, d] with gate weight [E, d].

    Returns (weights [T,k] float64, indices [T,k] int64, aux dict).
    aux holds the fp32 selection keys before/after masking, the group
    scores and kept-group mask, and the unbiased scores s (float64).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(gate_w, dtype=np.float64)
    T = x.shape[0]
    E = w.shape[0]
    if score_func not in SCORE_FUNCS:
        raise ValueError(score_func)
    if n_groups > 1 and E % n_groups:
        raise ValueError("n_routed_experts must be divisible by n_expert_groups")
    z = x @ w.T                      # step 1: fp32 linear of the page, exact here
    s = affinity(z, score_func)      # step 2
    keys = selection_keys(s, bias)   # step 3
    masked, kept, gscores = mask_groups(keys, n_groups, topk_groups, bias is not None)  # step 4
    indices = np.empty((T, topk), dtype=np.int64)
    for t in range(T):               # step 5
        indices[t] = _order_desc(masked[t])[:topk]
    weights = np.take_along_axis(s, indices, axis=1)   # step 6: unbiased scores
    renorm = (score_func != "softmax") if renormalize < 0 else bool(renormalize)
    if renorm:
        weights = weights / weights.sum(axis=1, keepdims=True)
    weights = weights * route_scale
    aux = {"logits": z, "scores": s, "keys": keys, "masked_keys": masked,
           "group_scores": gscores, "kept_groups": kept}
    return weights, indices, aux


def hash_gate(token_ids, tid2eid, route_scale=1.0):
    """Hash routing: the expert set of a token is its tid2eid row."""
    token_ids = np.asarray(token_ids, dtype=np.int64)
    table = np.asarray(tid2eid)
    k = table.shape[1]
    indices = table[token_ids].astype(np.int64)
    weights = np.full(indices.shape, route_scale / k, dtype=np.float64)
    return weights, indices


def smallest_primes_above(m, k):
    """The k smallest primes larger than m, by trial division."""
    out = []
    q = m + 1
    while len(out) < k:
        if q >= 2 and all(q % d for d in range(2, int(q ** 0.5) + 1)):
            out.append(q)
        q += 1
    return out


def ngram_hash_gate(prev_ids, token_ids, vocab_size, n_experts, k, route_scale=1.0):
    """2-gram hash routing ("How was DeepSeek V4's tid2eid derived?", section
    "An extreme case"): for the pair (a, b) of the preceding and the current
    token id, expert j is (a * q_j + b) mod n with q_j the j-th smallest prime
    larger than the vocabulary size m.  Reading: a token with no preceding
    token (prev id < 0) uses a = m; duplicate experts are kept, as the page
    allows; the weights are route_scale / k as for the table-based hash."""
    prev_ids = np.asarray(prev_ids, dtype=np.int64)
    token_ids = np.asarray(token_ids, dtype=np.int64)
    primes = smallest_primes_above(vocab_size, k)
    T = token_ids.shape[0]
    indices = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        a = int(prev_ids[t]) if prev_ids[t] >= 0 else vocab_size
        b = int(token_ids[t])
        for j in range(k):
            indices[t, j] = (a * primes[j] + b) % n_experts
    weights = np.full((T, k), route_scale / k, dtype=np.float64)
    return weights, indices
