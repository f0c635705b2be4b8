"""The allocation-free bucketing entry point (moe_bucket_noalloc) against the
context's entry point (moe_bucket) and the oracle, through the C ABI: two
calls in a row on the static-scratch path (past 1,024 pairs), the second
smaller, then the one-workgroup path, then a size past the maximum."""
import numpy as np
import pytest
import torch

from _gpu_helpers import check_bucket, say
from quantized_expert_ffn_softmax_amd import binding as B
from quantized_expert_ffn_softmax_amd.runtime import MoeContext

pytestmark = pytest.mark.gpu


def _zipf_idx(rng, T, E, k):
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p = p[rng.permutation(E)]
    p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def test_noalloc_bucketing_matches_the_context_call():
    E, k = 512, 10
    ctx = MoeContext(256, 128, E, k, 1, None, 12288)
    rng = np.random.default_rng(5)
    for T in (12288, 3001, 60):
        say(f"  bucketing T={T} x k={k} over E={E}: context call and allocation-free call")
        idx = _zipf_idx(rng, T, E, k)
        d_idx = torch.from_numpy(idx).cuda()
        off_a = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
        perm_a = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
        off_b, perm_b = torch.full_like(off_a, -9), torch.full_like(perm_a, -9)
        B.moe_bucket(ctx.ctx, d_idx, T, off_a, perm_a)
        B.moe_bucket_noalloc(d_idx, T, k, E, off_b, perm_b)
        torch.cuda.synchronize()
        assert torch.equal(off_a, off_b) and torch.equal(perm_a, perm_b)
        check_bucket(off_b.cpu().numpy(), perm_b.cpu().numpy(), idx, E)
    # past the static scratch's size: refused before anything is enqueued
    big = torch.zeros((13108, k), dtype=torch.int32, device="cuda")
    keep = perm_b.clone()
    with pytest.raises(B.MoeError) as ei:
        B.moe_bucket_noalloc(big, 13108, k, E, off_b, perm_b)
    assert ei.value.status == B.MOE_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.equal(perm_b, keep)
    ctx.close()
