"""Pins for the oracle's router: top-k selection, tie-break and weights (CPU only)."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _brute_topk(row, k):
    # selection by repeated scan: take the largest remaining value, the first
    # (lowest index) one on ties
    left = list(range(len(row)))
    chosen = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        chosen.append(best)
        left.remove(best)
    return chosen


@pytest.mark.parametrize("E", [2, 3, 4, 5, 6])
def test_topk_exhaustive_ties(E):
    # every logit pattern over a 3-value alphabet: all tie structures
    for pattern in itertools.product([0.0, 0.5, 1.0], repeat=E):
        row = np.array([pattern])
        for k in range(1, E + 1):
            idx, w = oracle.topk_from_logits(row, k)
            assert list(idx[0]) == _brute_topk(list(pattern), k)


def test_topk_random_against_brute():
    rng = np.random.default_rng(1)
    lg = rng.integers(-3, 4, (200, 16)).astype(np.float64) * 0.25
    for k in (1, 2, 5, 10, 16):
        idx, _ = oracle.topk_from_logits(lg, k)
        for t in range(lg.shape[0]):
            assert list(idx[t]) == _brute_topk(list(lg[t]), k)


def test_k1_is_argmax_lowest_index():
    rng = np.random.default_rng(2)
    lg = rng.integers(0, 3, (300, 9)).astype(np.float64)
    idx, w = oracle.topk_from_logits(lg, 1)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))
    assert np.all(w == 1.0)


def test_weights_invariants():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((64, 512)) * 0.905
    idx, w = oracle.topk_from_logits(lg, 10)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(lg.shape[0]):
        assert len(set(idx[t])) == 10
        for a in range(10):
            for b in range(10):
                assert math.isclose(w[t, a] / w[t, b], math.exp(lg[t, idx[t, a]] - lg[t, idx[t, b]]),
                                    rel_tol=1e-12)


def test_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((20, 16)) * 2
    idx, w = oracle.topk_from_logits(lg, 16)
    ref = softmax(lg, axis=1)
    for t in range(20):
        assert np.allclose(w[t], ref[t, idx[t]], rtol=1e-13, atol=0)


def test_renormalised_equals_softmax_restricted():
    # softmax over all E then renormalised over the chosen k
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((30, 64))
    idx, w = oracle.topk_from_logits(lg, 6)
    full = softmax(lg, axis=1)
    for t in range(30):
        sel = full[t, idx[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=1e-12, atol=0)


def test_router_logits_definition():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 8)).astype(np.float32)
    wr = rng.standard_normal((5, 8)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    lg = oracle.router_logits(x, wr, b)
    for t in range(3):
        for e in range(5):
            s = sum(float(x[t, c]) * float(wr[e, c]) for c in range(8)) + float(b[e])
            assert math.isclose(lg[t, e], s, rel_tol=1e-12, abs_tol=1e-12)


def test_topk_gap():
    lg = np.array([[3.0, 1.0, 2.0, 2.0]])
    assert oracle.topk_gap(lg, 2)[0] == 0.0
    assert oracle.topk_gap(lg, 1)[0] == 1.0
    assert np.isinf(oracle.topk_gap(lg, 4)[0])
