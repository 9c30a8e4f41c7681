"""Pins of the oracle's permutation by expert (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_case():
    g = json.load(open(os.path.join(GOLDEN, "permute_small.json")))
    counts, offsets, st, ss, inv = oracle.permute(np.array(g["indices"]), g["E"])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert st.tolist() == g["sorted_tok"]
    assert ss.tolist() == g["sorted_slot"]
    assert inv.tolist() == g["inverse"]


@pytest.mark.parametrize("E,k,T,seed", [(16, 2, 64, 0), (64, 8, 500, 1), (5, 3, 1, 2), (300, 4, 50, 3)])
def test_matches_stable_library_sort(E, k, T, seed):
    indices = np.random.default_rng(seed).integers(0, E, size=(T, k))
    counts, offsets, st, ss, inv = oracle.permute(indices, E)
    order = np.argsort(indices.ravel(), kind="stable")   # numpy's stable sort
    np.testing.assert_array_equal(st, order // k)
    np.testing.assert_array_equal(ss, order % k)
    np.testing.assert_array_equal(counts, np.bincount(indices.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    # sorted[inverse] is the identity on pairs
    np.testing.assert_array_equal(st[inv], np.repeat(np.arange(T), k).reshape(T, k))
    np.testing.assert_array_equal(ss[inv], np.tile(np.arange(k), (T, 1)))
    for e in range(E):
        seg = (st * k + ss)[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_empty_batch():
    counts, offsets, st, ss, inv = oracle.permute(np.zeros((0, 3), dtype=np.int64), 4)
    assert counts.tolist() == [0, 0, 0, 0] and offsets.tolist() == [0, 0, 0, 0, 0]
    assert st.size == 0 and inv.shape == (0, 3)
