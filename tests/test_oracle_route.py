"""Pins of the oracle's learned and hash gates (CPU only).

Each check is chosen so that a plausible slip in oracle/route.py (wrong
affinity, bias in the weights, group score by max instead of top-2 sum, a
dropped renormalisation or route_scale, reversed tie order) fails one of
them.  None of them re-runs the oracle's own formula.
"""

import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gate(x, w, bias, **kw):
    return oracle.learned_gate(x, w, bias, **kw)


def _random(T=300, d=48, E=64, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((E, d)) / np.sqrt(d)
    bias = rng.uniform(-0.01, 0.01, E).astype(np.float32)
    return x, w, bias


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "route_small.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    z = np.asarray(case["z"], dtype=np.float64)
    x = np.ones((1, 1))
    w = z[:, None]
    bias = None if case["bias"] is None else np.asarray(case["bias"], dtype=np.float32)
    weights, idx, _ = _gate(x, w, bias, score_func=case["score_func"], n_groups=case["n_groups"],
                            topk_groups=case["topk_groups"], topk=case["topk"],
                            route_scale=case["route_scale"])
    assert idx[0].tolist() == case["indices"]
    np.testing.assert_allclose(weights[0], case["weights"], rtol=1e-12)


@pytest.mark.parametrize("score_func", ["softmax", "sigmoid", "sqrtsoftplus"])
@pytest.mark.parametrize("groups", [(1, 1), (8, 4), (8, 8), (4, 1)])
def test_distinct_ids_and_masked_groups_never_win(score_func, groups):
    G, g = groups
    x, w, bias = _random(seed=1)
    E, k = w.shape[0], 4
    weights, idx, aux = _gate(x, w, bias, score_func=score_func, n_groups=G, topk_groups=g,
                              topk=k, route_scale=1.0)
    assert idx.shape == (x.shape[0], k)
    assert np.all((idx >= 0) & (idx < E))
    assert all(len(set(r)) == k for r in idx.tolist())
    if G > 1:
        per = E // G
        keys = aux["keys"]
        for t in range(x.shape[0]):
            # group scores from a library sort: sum of the two largest keys
            gs = np.array([np.float32(np.sort(keys[t, j * per:(j + 1) * per])[-1]) +
                           np.float32(np.sort(keys[t, j * per:(j + 1) * per])[-2])
                           for j in range(G)], dtype=np.float32)
            kept = set(np.argsort(-gs.astype(np.float64), kind="stable")[:g].tolist())
            assert set((idx[t] // per).tolist()) <= kept


@pytest.mark.parametrize("score_func,scale", [("sigmoid", 2.5), ("sqrtsoftplus", 1.0)])
def test_weights_sum_to_route_scale(score_func, scale):
    x, w, bias = _random(seed=2)
    weights, _, _ = _gate(x, w, bias, score_func=score_func, n_groups=8, topk_groups=4, topk=8,
                          route_scale=scale)
    np.testing.assert_allclose(weights.sum(axis=1), scale, rtol=1e-12)


def test_full_sort_agrees_with_selection():
    x, w, bias = _random(seed=3)
    _, idx, aux = _gate(x, w, bias, score_func="sigmoid", n_groups=8, topk_groups=3, topk=6,
                        route_scale=1.0)
    masked = aux["masked_keys"].astype(np.float64)
    for t in range(x.shape[0]):
        order = np.argsort(-masked[t], kind="stable")      # library sort, ties by index
        assert idx[t].tolist() == order[:6].tolist()


@pytest.mark.parametrize("score_func", ["softmax", "sigmoid", "sqrtsoftplus"])
def test_monotone_affinity_reduces_to_logit_topk(score_func):
    """bias = 0, no groups: every affinity is increasing in z, so the choice is
    the top-k of the raw logits x.W^T (computed here by a plain matmul)."""
    x, w, _ = _random(seed=4)
    _, idx, _ = _gate(x, w, None, score_func=score_func, n_groups=1, topk_groups=1, topk=5,
                      route_scale=1.0)
    z = x @ w.T
    for t in range(x.shape[0]):
        zs = np.sort(z[t])[::-1][:6]
        if np.min(np.abs(np.diff(zs))) < 1e-5:       # fp32 keys may merge a near tie
            continue
        assert idx[t].tolist() == np.argsort(-z[t], kind="stable")[:5].tolist()


def test_all_groups_kept_equals_no_groups():
    x, w, bias = _random(seed=5)
    a = _gate(x, w, bias, score_func="sigmoid", n_groups=8, topk_groups=8, topk=8, route_scale=2.5)
    b = _gate(x, w, bias, score_func="sigmoid", n_groups=1, topk_groups=1, topk=8, route_scale=2.5)
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_allclose(a[0], b[0], rtol=1e-15)


def test_softmax_closed_form_not_renormalised():
    x, w, _ = _random(seed=6)
    weights, idx, aux = _gate(x, w, None, score_func="softmax", n_groups=1, topk_groups=1, topk=3,
                              route_scale=1.0)
    s = softmax(x @ w.T, axis=1)                        # scipy's softmax
    np.testing.assert_allclose(aux["scores"].sum(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(weights, np.take_along_axis(s, idx, 1), rtol=1e-12)
    assert np.all(weights.sum(axis=1) < 1.0)


def test_bias_changes_selection_not_weights():
    """Weights are the renormalised UNbiased sigmoid scores of the chosen
    experts (scipy's expit), and a large bias can force an expert in."""
    x, w, bias = _random(seed=7)
    weights, idx, _ = _gate(x, w, bias, score_func="sigmoid", n_groups=1, topk_groups=1, topk=4,
                            route_scale=2.5)
    s = expit(x @ w.T)
    chosen = np.take_along_axis(s, idx, 1)
    np.testing.assert_allclose(weights, 2.5 * chosen / chosen.sum(1, keepdims=True), rtol=1e-12)
    big = np.zeros(w.shape[0], dtype=np.float32)
    big[17] = 10.0
    _, idx2, _ = _gate(x, w, big, score_func="sigmoid", n_groups=1, topk_groups=1, topk=4,
                       route_scale=1.0)
    assert np.all(idx2[:, 0] == 17)


def test_sqrtsoftplus_values():
    # sqrt(log(1 + e^z)) at a few points, from the definition with math.log1p/exp
    import math
    z = np.array([[-30.0, -1.0, 0.0, 2.0, 40.0]])
    s = oracle.affinity(z, "sqrtsoftplus")[0]
    ref = [math.sqrt(math.log1p(math.exp(v))) if v < 30 else math.sqrt(v) for v in z[0]]
    np.testing.assert_allclose(s[1:4], ref[1:4], rtol=1e-14)
    assert s[0] == pytest.approx(math.sqrt(math.exp(-30.0)), rel=1e-6)
    assert s[4] == pytest.approx(math.sqrt(40.0), rel=1e-12)


def test_renormalize_override():
    x, w, bias = _random(seed=8)
    w0, idx0, _ = _gate(x, w, None, score_func="softmax", n_groups=1, topk_groups=1, topk=3,
                        route_scale=1.0, renormalize=1)
    np.testing.assert_allclose(w0.sum(1), 1.0, rtol=1e-12)
    w1, idx1, _ = _gate(x, w, bias, score_func="sigmoid", n_groups=1, topk_groups=1, topk=3,
                        route_scale=1.0, renormalize=0)
    np.testing.assert_allclose(w1, np.take_along_axis(expit(x @ w.T), idx1, 1), rtol=1e-12)


def test_hash_gate_is_table_lookup():
    rng = np.random.default_rng(9)
    table = rng.integers(0, 16, size=(100, 4)).astype(np.int32)
    ids = rng.integers(0, 100, size=50)
    weights, idx = oracle.hash_gate(ids, table, route_scale=1.0)
    np.testing.assert_array_equal(idx, table[ids])
    np.testing.assert_array_equal(weights, np.full((50, 4), 0.25))
    # counts depend only on the ids, never on activations (constant hash load)
    np.testing.assert_array_equal(np.bincount(idx.ravel(), minlength=16),
                                  np.bincount(table[ids].ravel(), minlength=16))
