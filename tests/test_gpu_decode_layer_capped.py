"""moe_decode_layer on a capped cache, through the C ABI, against the separate
calls it replaces (moe_route -> moe_cache_resolve_async -> moe_expert_ffn on
the decode path -> moe_combine_norm) on a twin context over the same host
store:

* every output bit for bit, call after call, with misses, hits and
  evictions; the same table, stamps and counters after every call (a single
  token takes the top-k and the resolve in one workgroup, more tokens the
  router's own finishing kernel and the resolve kernel);
* no fill kernel runs (the bucketing launch copies the misses in spare
  workgroups): every slot in use then holds its identity's blob, byte for byte
  up to the end of the last section, and later calls that hit those slots
  still match the twin;
* a 4-layer stack captured in a HIP graph and replayed on new inputs,
  against eager separate calls;
* a call that cannot pin its working set changes nothing and writes no
  y_pairs row.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from _gpu_helpers import say
from moe_synth.harness import fill_pool
from quantized_expert_ffn_softmax_amd import binding as B
from quantized_expert_ffn_softmax_amd.runtime import MoeContext

pytestmark = pytest.mark.gpu

REAL = dict(d=2048, f=768, E=512, k=10)
TINY = dict(d=256, f=128, E=16, k=2)


def _used_bytes(d, f):
    """The blob's bytes up to the end of its last section (the down scales)."""
    secs, _stride = oracle.blob_sections(d, f)
    _name, rows, cols, _code_off, scale_off = secs[-1]
    return scale_off + oracle.matrix_bytes(rows, cols)[1]


def _host_store(s, L, seed=3):
    d, f, E = s["d"], s["f"], s["E"]
    stride = B.moe_expert_bytes(d, f)
    host = torch.empty((L * E, stride), dtype=torch.uint8, pin_memory=True)
    fill_pool(host, list(range(L * E)), seed, d, f, E)
    return host


def _capped(s, L, S, T, host, seed=3):
    d, f, E, k = s["d"], s["f"], s["E"], s["k"]
    ctx = MoeContext(d, f, E, k, L, S, T, host_store=host)
    fill_pool(ctx.shared_pool, [(l, E) for l in range(L)], seed, d, f, E)
    ctx.slot_pool.fill_(0x5a)  # slots start with bytes no blob is made of
    return ctx


def _inputs(d, E, L, seed, alpha):
    wr = [torch.from_numpy(moe_synth.gen_router(seed, l, E, d)).cuda() for l in range(L)]
    bias = [torch.from_numpy(moe_synth.gen_bias(seed, l, E, alpha)).cuda() for l in range(L)]
    return wr, bias


def _separate(c, l, x, T, wr, bias, buf, x_next):
    B.moe_route(c, l, x, T, wr, bias, None, buf["idx"], buf["w"])
    B.moe_cache_resolve_async(c, l, buf["idx"], T, buf["slot"])
    B.moe_expert_ffn(c, l, x, T, buf["idx"], buf["slot"], buf["y_pairs"], buf["y_shared"], B.MOE_PATH_DECODE)
    B.moe_combine_norm(c, buf["y_pairs"], buf["w"], buf["y_shared"], T, buf["out"], x_next)


def _fused(c, l, x, T, wr, bias, buf, x_next):
    B.moe_decode_layer(c, l, x, T, wr, bias, None, buf["idx"], buf["w"], buf["y_pairs"], buf["y_shared"],
                       buf["out"], x_next)


def _snapshot(ctx, L, E, S):
    so, io, st = np.zeros(L * E, np.int32), np.zeros(S, np.int32), np.zeros(S, np.uint32)
    B.moe_cache_snapshot(ctx.ctx, so, io, st)
    return so, io, st


def _slots_hold_blobs(ctx, host, used):
    _so, io, _st = _snapshot(ctx, ctx.L, ctx.E, ctx.n_slots)
    pool = ctx.slot_pool.cpu()
    for s_, i_ in enumerate(io.tolist()):
        if i_ >= 0:
            assert torch.equal(pool[s_, :used], host[i_, :used]), (s_, i_)
    return int(np.sum(io >= 0))


@pytest.mark.parametrize("shape,T,S,calls,alpha", [
    ("REAL", 1, 40, 14, 0.75), ("REAL", 2, 40, 12, 0.75), ("REAL", 4, 60, 10, 0.75), ("REAL", 5, 80, 8, 0.75),
    ("TINY", 1, 5, 30, 0.75), ("TINY", 2, 6, 30, 0.0), ("TINY", 3, 7, 30, 0.75), ("TINY", 9, 16, 20, 0.0),
], ids=lambda v: str(v))
def test_capped_layer_equals_separate_calls(shape, T, S, calls, alpha):
    s = REAL if shape == "REAL" else TINY
    d, f, E, k = s["d"], s["f"], s["E"], s["k"]
    L = 2
    say(f"  capped decode layer {shape} T={T} S={S}: {calls} calls against the separate calls")
    host = _host_store(s, L)
    a, b = _capped(s, L, S, T, host), _capped(s, L, S, T, host)
    wr, bias = _inputs(d, E, L, seed=4, alpha=alpha)
    ba, bb = a.buffers(T), b.buffers(T)
    xa, xb = torch.empty((T, d), device="cuda"), torch.empty((T, d), device="cuda")
    used = _used_bytes(d, f)
    for c in range(calls):
        l = c % L
        x = torch.from_numpy(moe_synth.gen_x(5, c, T, d)).cuda()
        _separate(a.ctx, l, x, T, wr[l], bias[l], ba, xa)
        _fused(b.ctx, l, x, T, wr[l], bias[l], bb, xb)
        torch.cuda.synchronize()
        for key in ("idx", "w", "y_pairs", "y_shared", "out"):
            assert torch.equal(ba[key].view(torch.int32), bb[key].view(torch.int32)), (c, key)
        assert torch.equal(xa.view(torch.int32), xb.view(torch.int32)), c
        for u, v in zip(_snapshot(a, L, E, S), _snapshot(b, L, E, S)):
            assert np.array_equal(u, v), c
        assert B.moe_get_stats(a.ctx) == B.moe_get_stats(b.ctx), c
    st = B.moe_get_stats(b.ctx)
    say(f"    lookups {st['lookups']}, hits {st['hits']}, misses {st['misses']}, failed {st['failed_calls']}")
    assert st["hits"] > 0 and st["misses"] > S and st["failed_calls"] == 0  # the table filled and evicted
    na, nb = _slots_hold_blobs(a, host, used), _slots_hold_blobs(b, host, used)
    assert na == nb == S
    a.close()
    b.close()


def test_capped_stack_in_graph_equals_eager_separate():
    s = REAL
    d, f, E, k = s["d"], s["f"], s["E"], s["k"]
    L, T, S = 4, 1, 48
    say(f"  capped {L}-layer stack, T={T}, S={S}: moe_decode_layer in a HIP graph against eager separate calls")
    host = _host_store(s, L)
    g, e = _capped(s, L, S, T, host), _capped(s, L, S, T, host)
    wr, bias = _inputs(d, E, L, seed=6, alpha=0.75)
    bg, be = g.buffers(T), e.buffers(T)
    xin = torch.zeros((T, d), device="cuda")
    xg = [torch.empty((T, d), device="cuda") for _ in range(2)]
    xe = [torch.empty((T, d), device="cuda") for _ in range(2)]

    def stack(run, ctx, buf, xs, x0):
        x = x0
        for l in range(L):
            run(ctx.ctx, l, x, T, wr[l], bias[l], buf, xs[l % 2])
            x = xs[l % 2]
        return x

    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cs):
        stack(_fused, g, bg, xg, xin)
    torch.cuda.synchronize()
    for rep in range(5):
        x0 = torch.from_numpy(moe_synth.gen_x(6, 10 + rep, T, d)).cuda()
        xin.copy_(x0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        xe_last = stack(_separate, e, be, xe, x0)
        torch.cuda.synchronize()
        assert torch.equal(xg[(L - 1) % 2].view(torch.int32), xe_last.view(torch.int32)), rep
        for key in ("idx", "w", "y_pairs", "y_shared", "out"):
            assert torch.equal(bg[key].view(torch.int32), be[key].view(torch.int32)), (rep, key)
        for u, v in zip(_snapshot(g, L, E, S), _snapshot(e, L, E, S)):
            assert np.array_equal(u, v), rep
        assert B.moe_get_stats(g.ctx) == B.moe_get_stats(e.ctx), rep
    st = B.moe_get_stats(g.ctx)
    say(f"    lookups {st['lookups']}, hits {st['hits']}, misses {st['misses']}")
    assert st["misses"] > S and st["hits"] > 0
    assert _slots_hold_blobs(g, host, _used_bytes(d, f)) == S
    del graph
    g.close()
    e.close()


def test_capped_layer_capacity_failure_changes_nothing():
    s = TINY
    d, f, E, k = s["d"], s["f"], s["E"], s["k"]
    L, T, S = 1, 2, 1  # every call touches at least top_k = 2 identities: none can pin its set
    host = _host_store(s, L)
    cap = _capped(s, L, S, T, host)
    wr, bias = _inputs(d, E, L, seed=7, alpha=0.0)
    buf = cap.buffers(T)
    buf["y_pairs"].fill_(7.0)
    x = torch.from_numpy(moe_synth.gen_x(7, 0, T, d)).cuda()
    before = _snapshot(cap, L, E, S)
    for _ in range(2):
        _fused(cap.ctx, 0, x, T, wr[0], bias[0], buf, None)
    torch.cuda.synchronize()
    assert torch.all(buf["y_pairs"] == 7.0)  # no pair got a slot: no row written
    for u, v in zip(before, _snapshot(cap, L, E, S)):
        assert np.array_equal(u, v)
    st = B.moe_get_stats(cap.ctx)
    assert st["failed_calls"] == 2 and st["resolve_calls"] == 0 and st["misses"] == 0
    assert torch.all(cap.slot_pool == 0x5a)  # nothing was filled
    cap.close()


def test_capped_layer_refuses_an_unmapped_store():
    s = TINY
    d, f, E, k = s["d"], s["f"], s["E"], s["k"]
    stride = B.moe_expert_bytes(d, f)
    plain = torch.zeros((E, stride), dtype=torch.uint8)  # pageable: not mapped into the device address space
    cap = MoeContext(d, f, E, k, 1, 4, 2, host_store=plain)
    wr, bias = _inputs(d, E, 1, seed=8, alpha=0.0)
    buf = cap.buffers(2)
    buf["out"].fill_(3.0)
    x = torch.from_numpy(moe_synth.gen_x(8, 0, 2, d)).cuda()
    with pytest.raises(B.MoeError) as ei:
        _fused(cap.ctx, 0, x, 2, wr[0], bias[0], buf, None)
    assert ei.value.status == B.MOE_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.all(buf["out"] == 3.0)  # nothing was enqueued
    assert B.moe_get_stats(cap.ctx)["resolve_calls"] == 0
    cap.close()
