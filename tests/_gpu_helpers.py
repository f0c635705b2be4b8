"""Shared checks for the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

import oracle

# max |err| <= TOL * RMS(oracle output of the call), the bar for fp32 outputs
TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.abs(np.asarray(got, dtype=np.float64) - ref).max() / rms)


def check_routing(gpu, x, wr, bias, k):
    """idx bit-exact against the oracle's top-k of the GPU's own fp32 logits,
    weights within 1e-6 relative; against the oracle's float64 logits, picks
    must agree wherever the k-th margin exceeds the near-tie bound.
    Returns the number of accepted near-ties."""
    lg32 = gpu["logits"].astype(np.float64)
    idx_ref, w_ref = oracle.topk_from_logits(lg32, k)
    assert np.array_equal(gpu["idx"], idx_ref), "idx differs from top-k of the GPU logits"
    assert np.all(np.abs(gpu["w"] - w_ref) <= 1e-6 * np.abs(w_ref) + 1e-12), "routing weights"
    lg64 = oracle.router_logits(x, wr, bias)
    scale = np.maximum(1.0, np.abs(lg64).max(axis=1))
    assert np.all(np.abs(lg32 - lg64) <= 1e-5 * scale[:, None]), "fp32 logits drift"
    idx64, _ = oracle.topk_from_logits(lg64, k)
    gap = oracle.topk_gap(lg64, k)
    tie = gap <= 1e-5 * scale
    same = np.all(np.sort(gpu["idx"], axis=1) == np.sort(idx64, axis=1), axis=1)
    assert np.all(same | tie), "routing differs away from a near-tie"
    # selected experts distinct; weights sum to one
    for row in gpu["idx"]:
        assert len(set(row.tolist())) == k
    assert np.all(np.abs(gpu["w"].sum(axis=1) - 1) <= 1e-5)
    return int(np.sum(~same))


def check_bucket(gpu_offsets, gpu_perm, idx, E):
    _, off, perm = oracle.bucket(idx, E)
    assert np.array_equal(gpu_offsets, off), "offsets"
    assert np.array_equal(gpu_perm, perm), "perm"
