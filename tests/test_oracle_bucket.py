"""Pins for the oracle's token -> expert bucketing (CPU only)."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (8, 2, 16), (5, 10, 512), (333, 10, 512), (64, 16, 16)])
def test_bucket_matches_library_routines(T, k, E):
    rng = np.random.default_rng(T * 7 + k)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = oracle.bucket(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))


def test_bucket_brute_force_small():
    idx = np.array([[3, 1], [1, 0], [3, 2]], dtype=np.int32)
    counts, offsets, perm = oracle.bucket(idx, 5)
    assert counts.tolist() == [1, 2, 1, 2, 0]
    assert offsets.tolist() == [0, 1, 3, 4, 6, 6]
    assert perm.tolist() == [3, 1, 2, 5, 0, 4]
