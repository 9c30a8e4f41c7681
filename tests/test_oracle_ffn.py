"""Pins of the oracle's SwiGLU experts, FP4 decode and layer forward (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _experts(E, d, I, seed):
    rng = np.random.default_rng(seed)
    ws = [(rng.standard_normal((I, d)) / math.sqrt(d), rng.standard_normal((I, d)) / math.sqrt(d),
           rng.standard_normal((d, I)) / math.sqrt(I)) for _ in range(E)]
    return ws


def test_e2m1_codes_match_published_set():
    g = json.load(open(os.path.join(GOLDEN, "e2m1_codes.json")))
    vals = oracle.E2M1_VALUES
    np.testing.assert_array_equal(vals, np.array(g["values"]))
    assert all(np.signbit(vals[8:])) and not any(np.signbit(vals[:8]))


def test_fp4_decode_cases():
    g = json.load(open(os.path.join(GOLDEN, "e2m1_codes.json")))
    for c in g["decode_cases"]:
        packed = np.zeros((1, 16), dtype=np.uint8)
        packed[0, 0] = c["packed"][0]
        scales = np.array([[c["scale"]]], dtype=np.uint8)
        out = oracle.fp4_decode(packed, scales)
        np.testing.assert_array_equal(out[0, :2], c["values"])
        np.testing.assert_array_equal(out[0, 2:], 0.0)
    nan = oracle.fp4_decode(np.full((1, 16), 0x22, np.uint8), np.array([[255]], np.uint8))
    assert np.all(np.isnan(nan))
    # one scale per 32 consecutive inputs
    two = oracle.fp4_decode(np.full((1, 32), 0x22, np.uint8), np.array([[127, 128]], np.uint8))
    np.testing.assert_array_equal(two[0, :32], 1.0)
    np.testing.assert_array_equal(two[0, 32:], 2.0)


def test_swiglu_scalar_worked_example():
    """d = I = 1: u = 4, W_gate = 5, W_up = -3, W_down = 1.
    No clamp: g = 20, v = -12, h = 20 * sigmoid(20) * (-12).
    Clamp L = 10: g -> min(20, 10) = 10, v -> clip(-12) = -10,
    h = 10 / (1 + e^-10) * (-10) = -100 / (1 + e^-10) ~ -99.9954602."""
    u, wg, wu, wd = np.array([[4.0]]), np.array([[5.0]]), np.array([[-3.0]]), np.array([[1.0]])
    y = oracle.swiglu_expert(u, wg, wu, wd)
    assert y[0, 0] == pytest.approx(20.0 / (1.0 + math.exp(-20.0)) * -12.0, rel=1e-15)
    yc = oracle.swiglu_expert(u, wg, wu, wd, swiglu_limit=10.0)
    assert yc[0, 0] == pytest.approx(-100.0 / (1.0 + math.exp(-10.0)), rel=1e-13)
    # gate at zero kills the output whatever the value branch
    assert oracle.swiglu_expert(u, np.zeros((1, 1)), wu, wd)[0, 0] == 0.0
    # the clamp caps the gate only from above
    yn = oracle.swiglu_expert(np.array([[-4.0]]), wg, np.array([[3.0]]), wd, swiglu_limit=10.0)
    assert yn[0, 0] == pytest.approx(-20.0 / (1.0 + math.exp(20.0)) * -10.0, rel=1e-13)


def test_clamp_identity_when_inactive_and_bound_when_active():
    d, I = 32, 16
    (wg, wu, wd), = _experts(1, d, I, 1)
    x = np.random.default_rng(2).standard_normal((40, d))
    base = oracle.swiglu_expert(x, wg, wu, wd)
    np.testing.assert_array_equal(base, oracle.swiglu_expert(x, wg, wu, wd, swiglu_limit=0.0))
    np.testing.assert_array_equal(base, oracle.swiglu_expert(x, wg, wu, wd, swiglu_limit=np.inf))
    np.testing.assert_allclose(base, oracle.swiglu_expert(x, wg, wu, wd, swiglu_limit=1e9), rtol=0)
    # large inputs: clamped h is bounded by L*sigmoid(L)*L per element, so
    # |y| <= I * L^2 * max|W_down|; unclamped output exceeds that bound
    L = 10.0
    xb = 40.0 * x
    yc = oracle.swiglu_expert(xb, wg, wu, wd, swiglu_limit=L)
    bound = I * L * L * expit(L) * np.abs(wd).max()
    assert np.abs(yc).max() <= bound
    assert np.abs(oracle.swiglu_expert(xb, wg, wu, wd)).max() > bound


def test_single_expert_top1_is_dense_swiglu():
    """E = 1, k = 1: softmax over one expert is 1, sigmoid renormalised gives
    route_scale; the layer is then a dense SwiGLU (+ shared), written here
    with plain matmuls and scipy's expit."""
    d, I, T = 24, 40, 30
    (wg, wu, wd), sh = _experts(2, d, I, 3)
    x = np.random.default_rng(4).standard_normal((T, d))
    dense = lambda W, x: ((x @ W[0].T) * expit(x @ W[0].T) * (x @ W[1].T)) @ W[2].T
    gw = np.random.default_rng(5).standard_normal((1, d))
    for score_func, scale, expect_w in [("softmax", 1.0, 1.0), ("sigmoid", 2.5, 2.5)]:
        w, idx, _ = oracle.learned_gate(x, gw, None, score_func=score_func, n_groups=1,
                                        topk_groups=1, topk=1, route_scale=scale)
        np.testing.assert_allclose(w, expect_w, rtol=1e-15)
        y = oracle.layer_forward(x, w, idx, lambda e: (wg, wu, wd), sh)
        np.testing.assert_allclose(y, expect_w * dense((wg, wu, wd), x) + dense(sh, x), rtol=1e-12)


def test_identical_experts_make_routing_irrelevant():
    d, I, T, E, k = 16, 24, 50, 8, 3
    (wg, wu, wd), = _experts(1, d, I, 6)
    x = np.random.default_rng(7).standard_normal((T, d))
    rng = np.random.default_rng(8)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, (T, k))
    y = oracle.layer_forward(x, w, idx, lambda e: (wg, wu, wd))
    single = oracle.swiglu_expert(x, wg, wu, wd)
    np.testing.assert_allclose(y, w.sum(1, keepdims=True) * single, rtol=1e-12)


def test_dense_routing_map_form_agrees():
    """Brute force over all experts with the dense map G[t,e] (non-zero only
    for the selected experts) equals the per-expert dispatch loop."""
    d, I, T, E, k = 16, 12, 40, 6, 2
    experts = _experts(E, d, I, 9)
    sh = _experts(1, d, I, 10)[0]
    x = np.random.default_rng(11).standard_normal((T, d))
    gw = np.random.default_rng(12).standard_normal((E, d))
    w, idx, _ = oracle.learned_gate(x, gw, None, score_func="sigmoid", n_groups=1, topk_groups=1,
                                    topk=k, route_scale=1.0)
    G = np.zeros((T, E))
    np.put_along_axis(G, idx, w, axis=1)
    y1 = oracle.layer_forward(x, w, idx, lambda e: experts[e], sh)
    y2 = oracle.dense_map_forward(x, G, lambda e: experts[e], sh)
    np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-14)


def test_position_wise():
    """The layer never mixes tokens: permuting tokens permutes outputs."""
    d, I, T, E, k = 16, 12, 33, 5, 2
    experts = _experts(E, d, I, 13)
    x = np.random.default_rng(14).standard_normal((T, d))
    gw = np.random.default_rng(15).standard_normal((E, d))
    kw = dict(score_func="softmax", n_groups=1, topk_groups=1, topk=k, route_scale=1.0)
    w, idx, _ = oracle.learned_gate(x, gw, None, **kw)
    y = oracle.layer_forward(x, w, idx, lambda e: experts[e])
    perm = np.random.default_rng(16).permutation(T)
    wp, idxp, _ = oracle.learned_gate(x[perm], gw, None, **kw)
    yp = oracle.layer_forward(x[perm], wp, idxp, lambda e: experts[e])
    np.testing.assert_allclose(yp, y[perm], rtol=1e-12)
