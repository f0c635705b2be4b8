"""GPU checks of moe_cache_resolve_async, the miss path with no host round
trip (a fill kernel reads the mapped pinned host store), through the C ABI:

* slot for slot equal to the synchronous resolve and to the oracle's LRU over
  a sequence of calls, every used slot holding its identity's blob, the FFN
  through it equal to the FFN on the resident map, the same table, stamps and
  counts at the end;
* a call that cannot pin its working set changes nothing, gives every pair
  slot -1 (the FFN then writes none of their rows) and is counted;
* a capped layer (route -> async resolve -> FFN -> combine) captured in a HIP
  graph and replayed on new inputs, against eager runs on a second context.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from _gpu_helpers import say
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


def test_async_resolve_matches_sync_and_oracle():
    L, S, T, steps = 3, 10, 2, 60
    say(f"  async resolve L={L} E={E} S={S} T={T} steps={steps}")
    a, b, res = _capped(L, S, T), _capped(L, S, T), _resident(L, T)
    stride = a.stride
    orc = oracle.LRUCache(L, E, S)
    rng = np.random.default_rng(11)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    sa = torch.empty((T, K), dtype=torch.int32, device="cuda")
    sb = torch.empty((T, K), dtype=torch.int32, device="cuda")
    x = torch.from_numpy(moe_synth.gen_x(4, 0, T, D)).cuda()
    bb, br = b.buffers(T), res.buffers(T)
    for step in range(steps):
        layer = step % L
        idx = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)
        idx_d = torch.from_numpy(idx).cuda()
        B.moe_cache_resolve(a.ctx, layer, idx_d, T, sa)
        B.moe_cache_resolve_async(b.ctx, layer, idx_d, T, sb)
        torch.cuda.synchronize()
        so, _misses = orc.resolve(layer, idx, stride)
        ga, gb = sa.cpu().numpy(), sb.cpu().numpy()
        assert np.array_equal(ga, so) and np.array_equal(gb, so), (step, ga, gb, so)
        for s_, i_ in zip(gb.reshape(-1), (layer * E + idx).reshape(-1)):
            assert torch.equal(b.slot_pool[int(s_)].cpu(), b.host_store[int(i_)]), (step, s_, i_)
        if step % 5 == 0:
            for ctx, buf, sl in ((b, bb, sb), (res, br, None)):
                B.moe_expert_ffn(ctx.ctx, layer, x, T, idx_d, sl, buf["y_pairs"], buf["y_shared"], B.MOE_PATH_DECODE)
            torch.cuda.synchronize()
            assert torch.equal(bb["y_pairs"], br["y_pairs"]) and torch.equal(bb["y_shared"], br["y_shared"])
    for ctx in (a, b):
        so_, io_, st_ = np.zeros(L * E, np.int32), np.zeros(S, np.int32), np.zeros(S, np.uint32)
        B.moe_cache_snapshot(ctx.ctx, so_, io_, st_)
        assert so_.tolist() == orc.slot_of and io_.tolist() == orc.id_of.tolist() and st_.tolist() == orc.stamp.tolist()
        st = B.moe_get_stats(ctx.ctx)
        assert (st["lookups"], st["hits"], st["misses"]) == (orc.lookups, orc.hits, orc.misses)
        assert st["bytes_h2d"] == orc.misses * stride and st["failed_calls"] == 0
    say(f"    hits {orc.hits}/{orc.lookups}, misses {orc.misses}")
    for ctx in (a, b, res):
        ctx.close()


def test_async_capacity_failure_changes_nothing():
    L, S, T = 1, 3, 2
    cap = _capped(L, S, T)
    slot = torch.empty((T, K), dtype=torch.int32, device="cuda")
    ok = torch.tensor([[0, 1], [1, 2]], dtype=torch.int32, device="cuda")
    B.moe_cache_resolve_async(cap.ctx, 0, ok, T, slot)
    torch.cuda.synchronize()
    before = [np.zeros(E, np.int32), np.zeros(S, np.int32), np.zeros(S, np.uint32)]
    B.moe_cache_snapshot(cap.ctx, *before)
    too_many = torch.tensor([[0, 5], [6, 7]], dtype=torch.int32, device="cuda")  # 4 identities, 3 slots
    B.moe_cache_resolve_async(cap.ctx, 0, too_many, T, slot)
    buf = cap.buffers(T)
    buf["y_pairs"].fill_(7.0)
    x = torch.from_numpy(moe_synth.gen_x(2, 0, T, D)).cuda()
    B.moe_expert_ffn(cap.ctx, 0, x, T, too_many, slot, buf["y_pairs"], buf["y_shared"], B.MOE_PATH_DECODE)
    torch.cuda.synchronize()
    assert torch.all(slot == -1)
    assert torch.all(buf["y_pairs"] == 7.0)  # no pair got a slot: no row written
    after = [np.zeros(E, np.int32), np.zeros(S, np.int32), np.zeros(S, np.uint32)]
    B.moe_cache_snapshot(cap.ctx, *after)
    for u, v in zip(before, after):
        assert np.array_equal(u, v)
    st = B.moe_get_stats(cap.ctx)
    assert st["failed_calls"] == 1 and st["resolve_calls"] == 1
    # the next call works and hits
    B.moe_cache_resolve_async(cap.ctx, 0, ok, T, slot)
    torch.cuda.synchronize()
    assert sorted(slot.cpu().numpy().reshape(-1).tolist()) == [0, 1, 1, 2]
    assert B.moe_get_stats(cap.ctx)["hits"] == 3
    cap.close()


def test_async_resolve_in_graph_matches_eager():
    # two layers per step over 16 slots for 32 identities: every step evicts
    L, S, T = 2, 16, 8
    say(f"  capped layers in a HIP graph, L={L} S={S} T={T}")
    g, e = _capped(L, S, T), _capped(L, S, T)
    wr = [torch.from_numpy(moe_synth.gen_router(5, l, E, D)).cuda() for l in range(L)]
    bias = [torch.from_numpy(moe_synth.gen_bias(5, l, E, 0.75)).cuda() for l in range(L)]
    x_static = torch.from_numpy(moe_synth.gen_x(5, 0, T, D)).cuda()
    gbuf = [g.buffers(T) for _ in range(L)]
    ebuf = [e.buffers(T) for _ in range(L)]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        for l in range(L):
            g.layer(l, x_static, wr[l], bias[l], gbuf[l], B.MOE_PATH_DECODE, logits=False, async_resolve=True)
    torch.cuda.synchronize()
    assert B.moe_get_stats(g.ctx)["resolve_calls"] == 0  # capture runs nothing
    for rep in range(6):
        x_new = torch.from_numpy(moe_synth.gen_x(5, 200 + rep, T, D)).cuda()
        x_static.copy_(x_new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            e.layer(l, x_new, wr[l], bias[l], ebuf[l], B.MOE_PATH_DECODE, logits=False)
        torch.cuda.synchronize()
        for l in range(L):
            for key in ("idx", "w", "slot", "y_pairs", "y_shared", "out"):
                assert torch.equal(gbuf[l][key], ebuf[l][key]), (rep, l, key)
    sg, se = B.moe_get_stats(g.ctx), B.moe_get_stats(e.ctx)
    assert sg == se, (sg, se)
    assert sg["misses"] > 0 and sg["hits"] > 0 and sg["resolve_calls"] == 6 * L
    say(f"    6 replays equal to eager; hits {sg['hits']}/{sg['lookups']}, misses {sg['misses']}")
    g.close()
    e.close()
