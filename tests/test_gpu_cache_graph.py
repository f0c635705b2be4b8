"""GPU checks beyond single-layer parity, through the C ABI:

* the capped expert cache (LRU slot table, miss fill from pinned host memory)
  against the oracle's LRU, call by call, and the FFN computed through it;
* the capacity error and the reset path;
* a layer captured in a HIP graph, replayed on new inputs, against eager runs;
* exact identities of the decode FFN (zero codes, doubled down scales);
* the prefill chunk at its full size (12,288 tokens), checked on sampled tokens
  and on the full bucketing.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from _gpu_helpers import TOL, check_bucket, rel_err, say
from moe_synth.harness import SyntheticLayer, fill_pool
from quantized_expert_ffn_softmax_amd import binding as B
from quantized_expert_ffn_softmax_amd.runtime import MoeContext

pytestmark = pytest.mark.gpu

D, F, E, K = 256, 128, 16, 2


def _capped(L, S, T, seed=3):
    ctx = MoeContext(D, F, E, K, L, S, T)
    fill_pool(ctx.host_store, list(range(L * E)), seed, D, F, E)
    fill_pool(ctx.shared_pool, [(l, E) for l in range(L)], seed, D, F, E)
    return ctx


def _resident(L, T, seed=3):
    ctx = MoeContext(D, F, E, K, L, None, T)
    fill_pool(ctx.slot_pool, list(range(L * E)), seed, D, F, E)
    fill_pool(ctx.shared_pool, [(l, E) for l in range(L)], seed, D, F, E)
    return ctx


def _zipf_idx(rng, T, p):
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def test_lru_cache_matches_oracle_and_feeds_the_ffn():
    L, S, T, steps = 3, 10, 2, 60
    say(f"  capped cache L={L} E={E} S={S} T={T} steps={steps}")
    cap, res = _capped(L, S, T), _resident(L, T)
    stride = cap.stride
    orc = oracle.LRUCache(L, E, S)
    rng = np.random.default_rng(7)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    slot = torch.empty((T, K), dtype=torch.int32, device="cuda")
    x = torch.from_numpy(moe_synth.gen_x(3, 0, T, D)).cuda()
    bufs = [cap.buffers(T), res.buffers(T)]
    host = cap.host_store
    for step in range(steps):
        layer = step % L
        idx = _zipf_idx(rng, T, p)
        idx_d = torch.from_numpy(idx).cuda()
        info = B.moe_cache_resolve(cap.ctx, layer, idx_d, T, slot, True)
        torch.cuda.synchronize()
        so, misses = orc.resolve(layer, idx, stride)
        got = slot.cpu().numpy()
        assert np.array_equal(got, so), (step, got, so)
        assert info["misses"] == len(misses) and info["hits"] == info["lookups"] - len(misses)
        assert info["bytes_h2d"] == len(misses) * stride
        ids = (layer * E + idx).reshape(-1)
        for s_, i_ in zip(got.reshape(-1), ids):
            assert torch.equal(cap.slot_pool[int(s_)].cpu(), host[int(i_)]), (step, s_, i_)
        if step % 7 == 0:
            # the FFN through the cache equals the FFN on the resident identity map
            for ctx, buf, sl in ((cap, bufs[0], slot), (res, bufs[1], None)):
                B.moe_expert_ffn(ctx.ctx, layer, x, T, idx_d, sl, buf["y_pairs"], buf["y_shared"],
                                 B.MOE_PATH_DECODE)
            torch.cuda.synchronize()
            assert torch.equal(bufs[0]["y_pairs"], bufs[1]["y_pairs"])
            assert torch.equal(bufs[0]["y_shared"], bufs[1]["y_shared"])
    so_ = np.zeros(L * E, np.int32)
    io_ = np.zeros(S, np.int32)
    st_ = np.zeros(S, np.uint32)
    B.moe_cache_snapshot(cap.ctx, so_, io_, st_)
    assert so_.tolist() == orc.slot_of and io_.tolist() == orc.id_of.tolist() and st_.tolist() == orc.stamp.tolist()
    st = B.moe_get_stats(cap.ctx)
    assert (st["lookups"], st["hits"], st["misses"]) == (orc.lookups, orc.hits, orc.misses)
    say(f"    hits {orc.hits}/{orc.lookups}, misses {orc.misses}")
    cap.close()
    res.close()


def test_capacity_error_leaves_the_table_and_reset_frees_it():
    L, S, T = 1, 3, 2
    cap = _capped(L, S, T)
    slot = torch.empty((T, K), dtype=torch.int32, device="cuda")
    ok = torch.tensor([[0, 1], [1, 2]], dtype=torch.int32, device="cuda")
    B.moe_cache_resolve(cap.ctx, 0, ok, T, slot)
    before = [np.zeros(E, np.int32), np.zeros(S, np.int32), np.zeros(S, np.uint32)]
    B.moe_cache_snapshot(cap.ctx, *before)
    too_many = torch.tensor([[0, 5], [6, 7]], dtype=torch.int32, device="cuda")  # 4 identities, 3 slots
    with pytest.raises(B.MoeError) as ei:
        B.moe_cache_resolve(cap.ctx, 0, too_many, T, slot)
    assert ei.value.status == B.MOE_ERR_CAPACITY
    after = [np.zeros(E, np.int32), np.zeros(S, np.int32), np.zeros(S, np.uint32)]
    B.moe_cache_snapshot(cap.ctx, *after)
    for a, b in zip(before, after):
        assert np.array_equal(a, b)
    B.moe_cache_reset(cap.ctx)
    B.moe_cache_snapshot(cap.ctx, *after)
    assert np.all(after[0] == -1) and np.all(after[1] == -1) and np.all(after[2] == 0)
    # usable again after the reset
    B.moe_cache_resolve(cap.ctx, 0, ok, T, slot)
    torch.cuda.synchronize()
    assert sorted(slot.cpu().numpy().reshape(-1).tolist()) == [0, 1, 1, 2]
    cap.close()


@pytest.mark.parametrize("shape", ["tiny", "real"])
def test_graph_replay_matches_eager(shape):
    dims = dict(d_model=D, d_ff=F, n_experts=E, top_k=K) if shape == "tiny" else \
        dict(d_model=2048, d_ff=768, n_experts=512, top_k=10)
    T = 8 if shape == "tiny" else 15
    layer = SyntheticLayer(seed=5, n_tokens=T, alpha=0.75, device="cuda:0", **dims)
    ctx = layer.ctx
    x_static = layer.x.clone()
    gbuf, ebuf = ctx.buffers(T), ctx.buffers(T)
    # warm-up on a side stream, then capture route -> resolve -> ffn -> combine
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ctx.layer(0, x_static, layer.wr, layer.bias, gbuf, B.MOE_PATH_DECODE, logits=False)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ctx.layer(0, x_static, layer.wr, layer.bias, gbuf, B.MOE_PATH_DECODE, logits=False)
    for rep in range(4):
        x_new = torch.from_numpy(moe_synth.gen_x(5, 100 + rep, T, dims["d_model"])).cuda()
        x_static.copy_(x_new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ctx.layer(0, x_new, layer.wr, layer.bias, ebuf, B.MOE_PATH_DECODE, logits=False)
        torch.cuda.synchronize()
        for key in ("idx", "w", "y_pairs", "y_shared", "out"):
            assert torch.equal(gbuf[key], ebuf[key]), (rep, key)
    say(f"    {shape}: 4 replays equal to eager")
    layer.close()


def test_decode_exact_identities():
    # zero codes in one expert's down matrix give exactly zero rows; doubled down
    # scales give exactly doubled outputs (a power-of-two factor is exact in
    # fp16 and fp32)
    T = 8
    ctx = _resident(1, T)
    secs, _ = oracle.blob_sections(D, F)
    _name, rows, cols, co, so = secs[2]
    wpr = oracle.words_per_row(cols)
    base = ctx.slot_pool.cpu().numpy()
    shared = ctx.shared_pool.cpu().numpy()
    idx = np.array([[3, 7]] * T, dtype=np.int32)
    idx_d = torch.from_numpy(idx).cuda()
    x = torch.from_numpy(moe_synth.gen_x(9, 0, T, D)).cuda()
    buf = ctx.buffers(T)

    def run():
        B.moe_expert_ffn(ctx.ctx, 0, x, T, idx_d, None, buf["y_pairs"], buf["y_shared"], B.MOE_PATH_DECODE)
        torch.cuda.synchronize()
        return buf["y_pairs"].cpu().numpy().copy(), buf["y_shared"].cpu().numpy().copy()

    yp0, ys0 = run()
    pool = base.copy()
    pool[7, co:co + rows * wpr * 4] = np.frombuffer(np.full(rows * wpr, 0x49244924, np.uint32).tobytes(), np.uint8)
    for e in range(E):
        sc = pool[e, so:so + rows * (cols // 32) * 2].view(np.float16)
        sc *= np.float16(2.0)
    sh = shared.copy()
    sh[0, so:so + rows * (cols // 32) * 2].view(np.float16)[:] *= np.float16(2.0)
    ctx.slot_pool.copy_(torch.from_numpy(pool))
    ctx.shared_pool.copy_(torch.from_numpy(sh))
    yp1, ys1 = run()
    assert np.array_equal(yp1[1::2], np.zeros_like(yp1[1::2]))  # pairs of expert 7: all codes 4
    assert np.array_equal(yp1[0::2], 2 * yp0[0::2])
    assert np.array_equal(ys1, 2 * ys0)
    ctx.close()


def test_prefill_full_chunk_sampled():
    """The 12,288-token prefill chunk at its full size, in the launch the bench
    times: full bucketing against the oracle; expert outputs row by row on a
    sample of pairs -- one pair in every 128-token entry of the hottest expert,
    up to 20 pairs of each of 20 other experts (8 among the 40 fullest, 12 among
    the rest; seeded), and one token in every
    128-token entry of the shared expert plus 64 more -- against the oracle's
    'fp16_weights' mode (tight) and the exact definition (the stated bar); routing
    and the combine on the tokens those pairs belong to."""
    T = 12288
    dims = dict(d_model=2048, d_ff=768, n_experts=512, top_k=10)
    say(f"  prefill chunk T={T} (full size), sampled pairs")
    layer = SyntheticLayer(seed=11, n_tokens=T, alpha=0.75, device="cuda:0", **dims)
    ctx, k, E = layer.ctx, dims["top_k"], dims["n_experts"]
    buf = ctx.buffers(T)
    ctx.layer(0, layer.x, layer.wr, layer.bias, buf, B.MOE_PATH_PREFILL)
    torch.cuda.synchronize()
    idx = buf["idx"].cpu().numpy()
    # full bucketing of the chunk (large path) against the oracle
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    B.moe_bucket(ctx.ctx, buf["idx"], T, off, perm)
    torch.cuda.synchronize()
    off_np, perm_np = off.cpu().numpy(), perm.cpu().numpy()
    check_bucket(off_np, perm_np, idx, E)
    counts = np.diff(off_np)
    rng = np.random.default_rng(0)
    hot = int(np.argmax(counts))
    picks = {}  # expert -> pair ids
    seg = perm_np[off_np[hot]:off_np[hot + 1]]
    picks[hot] = np.array([seg[i + rng.integers(0, min(128, seg.size - i))] for i in range(0, seg.size, 128)])
    big = np.argsort(-counts)[1:40]  # well-filled experts after the hottest: 8 of them
    small = np.flatnonzero((counts > 0) & ~np.isin(np.arange(E), np.append(big, hot)))
    others = np.concatenate([rng.choice(big, 8, replace=False), rng.choice(small, 12, replace=False)])
    for e in others:
        seg = perm_np[off_np[e]:off_np[e + 1]]
        picks[int(e)] = np.sort(rng.choice(seg, min(20, seg.size), replace=False))
    n_pairs = sum(v.size for v in picks.values())
    shared_toks = np.unique(np.concatenate([np.arange(0, T, 128) + rng.integers(0, 128, T // 128),
                                            rng.choice(T, 64, replace=False), [0, T - 1]]))
    say(f"    hottest expert {hot}: {counts[hot]} pairs, {picks[hot].size} entries sampled; {n_pairs} pairs over "
        f"{len(picks)} experts; {shared_toks.size} shared-expert tokens")
    assert n_pairs >= 256
    yp_gpu = buf["y_pairs"].cpu().numpy()
    ys_gpu = buf["y_shared"].cpu().numpy()
    got, ref_w, ref_x = [], [], []
    for e, pairs in list(picks.items()) + [(E, None)]:
        blob = layer.blob_np(e)
        rows_x = layer.x_np[pairs // k] if pairs is not None else layer.x_np[shared_toks]
        ref_w.append(oracle.expert_ffn(rows_x, oracle.expert_weights(blob, 2048, 768, True), "fp16_weights"))
        ref_x.append(oracle.expert_ffn(rows_x, oracle.expert_weights(blob, 2048, 768), "exact"))
        got.append(yp_gpu[pairs] if pairs is not None else ys_gpu[shared_toks])
    got, ref_w, ref_x = np.concatenate(got), np.concatenate(ref_w), np.concatenate(ref_x)
    e_w, e_x = rel_err(got, ref_w), rel_err(got, ref_x)
    # routing and combine on the tokens of the sampled pairs
    toks = np.unique(np.concatenate([v // k for v in picks.values()] + [shared_toks]))
    lg = buf["logits"][torch.from_numpy(toks).cuda()].cpu().numpy().astype(np.float64)
    idx_ref, w_ref = oracle.topk_from_logits(lg, k)
    assert np.array_equal(idx[toks], idx_ref)
    w_gpu = buf["w"][torch.from_numpy(toks).cuda()].cpu().numpy()
    assert np.all(np.abs(w_gpu - w_ref) <= 1e-6 * np.abs(w_ref) + 1e-12)
    rows = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    comb = oracle.combine(yp_gpu[rows].astype(np.float64), w_gpu.astype(np.float64), ys_gpu[toks].astype(np.float64))
    e_c = rel_err(buf["out"][torch.from_numpy(toks).cuda()].cpu().numpy(), comb)
    say(f"    {got.shape[0]} rows: vs fp16_weights {e_w:.2e}, vs exact {e_x:.2e}; combine on {toks.size} tokens "
        f"{e_c:.2e}")
    assert e_w <= 1e-4 and e_x <= TOL and e_c <= 1e-6
    layer.close()
