"""moe_decode_layer -- a whole decode layer on a resident cache in six
launches, five for a single token (the capped cache:
test_gpu_decode_layer_capped.py) -- against the seven-launch sequence of
separate calls it replaces
(moe_route -> moe_cache_resolve -> moe_expert_ffn on the decode path ->
moe_combine_norm / moe_combine), through the C ABI: every output bit for bit,
the cumulative counters equal, at the real shape (T = 1 .. 64) and small ones
(up to 300 tokens: the router's large-batch path),
with and without logits, bias and x_next; then chained through a 6-layer stack
captured in a HIP graph and replayed, against eager separate calls; and the
layer against the oracle at the usual bars.  Shapes the call does not take are
refused with nothing enqueued."""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu_helpers import say
from moe_synth.harness import fill_pool
from quantized_expert_ffn_softmax_amd import binding as B
from quantized_expert_ffn_softmax_amd.runtime import MoeContext

pytestmark = pytest.mark.gpu

REAL = dict(d=2048, f=768, E=512, k=10)
TINY = dict(d=256, f=128, E=16, k=2)


def _ctx(d, f, E, k, L, T, seed=3):
    ctx = MoeContext(d, f, E, k, L, None, T)
    fill_pool(ctx.slot_pool, list(range(L * E)), seed, d, f, E)
    fill_pool(ctx.shared_pool, [(l, E) for l in range(L)], seed, d, f, E)
    return ctx


def _inputs(d, E, L, T, seed, alpha):
    wr = [torch.from_numpy(moe_synth.gen_router(seed, l, E, d)).cuda() for l in range(L)]
    bias = [torch.from_numpy(moe_synth.gen_bias(seed, l, E, alpha)).cuda() for l in range(L)]
    x = torch.from_numpy(moe_synth.gen_x(seed, 0, T, d)).cuda()
    return wr, bias, x


def _separate(c, l, x, T, wr, bias, buf, logits, x_next):
    B.moe_route(c, l, x, T, wr, bias, buf["logits"] if logits else None, buf["idx"], buf["w"])
    B.moe_cache_resolve(c, l, buf["idx"], T, None)
    B.moe_expert_ffn(c, l, x, T, buf["idx"], None, buf["y_pairs"], buf["y_shared"], B.MOE_PATH_DECODE)
    if x_next is not None:
        B.moe_combine_norm(c, buf["y_pairs"], buf["w"], buf["y_shared"], T, buf["out"], x_next)
    else:
        B.moe_combine(c, buf["y_pairs"], buf["w"], buf["y_shared"], T, buf["out"])


def _fused(c, l, x, T, wr, bias, buf, logits, x_next):
    B.moe_decode_layer(c, l, x, T, wr, bias, buf["logits"] if logits else None, buf["idx"], buf["w"],
                       buf["y_pairs"], buf["y_shared"], buf["out"], x_next)


def _fresh(buf):
    for v in buf.values():
        if v.dtype == torch.int32:
            v.fill_(-7)
        else:
            v.fill_(float("nan"))


@pytest.mark.parametrize("shape,T,opts", [
    ("REAL", 15, "logits,bias,norm"), ("REAL", 1, "norm"), ("REAL", 2, "logits,bias,norm"), ("REAL", 5, "bias,norm"),
    ("TINY", 1, "logits,bias,norm"), ("TINY", 2, "bias"),
    ("REAL", 28, "logits,bias"), ("REAL", 64, "bias,norm"), ("TINY", 9, "logits,bias,norm"),
    ("TINY", 40, "bias"), ("TINY", 300, "logits,bias,norm"),
], ids=lambda v: str(v))
def test_fused_layer_equals_separate_calls(shape, T, opts):
    s = REAL if shape == "REAL" else TINY
    d, f, E, k = s["d"], s["f"], s["E"], s["k"]
    logits, use_bias, norm = "logits" in opts, "bias" in opts, "norm" in opts
    say(f"  decode layer {shape} T={T} ({opts}): six launches against seven")
    a, b = _ctx(d, f, E, k, 2, T), _ctx(d, f, E, k, 2, T)
    wr, bias, x = _inputs(d, E, 2, T, seed=4, alpha=0.75)
    ba, bb = a.buffers(T), b.buffers(T)
    _fresh(ba)
    _fresh(bb)
    xa = torch.full((T, d), float("nan"), device="cuda") if norm else None
    xb = torch.full((T, d), float("nan"), device="cuda") if norm else None
    for l in range(2):
        _separate(a.ctx, l, x, T, wr[l], bias[l] if use_bias else None, ba, logits, xa)
        _fused(b.ctx, l, x, T, wr[l], bias[l] if use_bias else None, bb, logits, xb)
        torch.cuda.synchronize()
        keys = ["idx", "w", "y_pairs", "y_shared", "out"] + (["logits"] if logits else [])
        for key in keys:
            assert torch.equal(ba[key].view(torch.int32), bb[key].view(torch.int32)), (l, key)
        if norm:
            assert torch.equal(xa.view(torch.int32), xb.view(torch.int32)), l
    assert B.moe_get_stats(a.ctx) == B.moe_get_stats(b.ctx)
    a.close()
    b.close()


@pytest.mark.parametrize("T", [15, 1])
def test_fused_stack_in_graph_equals_eager_separate(T):
    d, f, E, k = REAL["d"], REAL["f"], REAL["E"], REAL["k"]
    L = 6
    say(f"  {L}-layer stack, T={T}: fused layers in a HIP graph against eager separate calls")
    g, e = _ctx(d, f, E, k, L, T), _ctx(d, f, E, k, L, T)
    wr, bias, _ = _inputs(d, E, L, T, seed=6, alpha=0.75)
    bg, be = g.buffers(T), e.buffers(T)
    xin = torch.zeros((T, d), device="cuda")
    xg = [torch.empty((T, d), device="cuda") for _ in range(2)]
    xe = [torch.empty((T, d), device="cuda") for _ in range(2)]

    def stack(run, ctx, buf, xs, x0):
        x = x0
        for l in range(L):
            run(ctx.ctx, l, x, T, wr[l], bias[l], buf, False, xs[l % 2])
            x = xs[l % 2]
        return x

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        stack(_fused, g, bg, xg, xin)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack(_fused, g, bg, xg, xin)
    torch.cuda.synchronize()
    st_g0 = B.moe_get_stats(g.ctx)
    for rep in range(4):
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
    st_g1, st_e = B.moe_get_stats(g.ctx), B.moe_get_stats(e.ctx)
    # the graph's replays counted exactly what the eager calls counted
    assert {kk: st_g1[kk] - st_g0[kk] for kk in ("lookups", "hits", "resolve_calls")} == \
        {kk: st_e[kk] for kk in ("lookups", "hits", "resolve_calls")}
    del graph
    g.close()
    e.close()


def test_fused_layer_against_oracle():
    import oracle
    from _gpu_helpers import TOL, check_routing, rel_err
    from moe_synth.harness import SyntheticLayer
    layer = SyntheticLayer(seed=2, n_tokens=15, alpha=0.75, device="cuda:0", d_model=2048, d_ff=768,
                           n_experts=512, top_k=10)
    T, buf = layer.T, layer.ctx.buffers(layer.T)
    B.moe_decode_layer(layer.ctx.ctx, 0, layer.x, T, layer.wr, layer.bias, buf["logits"], buf["idx"], buf["w"],
                       buf["y_pairs"], buf["y_shared"], buf["out"], None)
    torch.cuda.synchronize()
    gpu = {kk: buf[kk].cpu().numpy() for kk in ("logits", "idx", "w", "y_pairs", "y_shared", "out")}
    check_routing(gpu, layer.x_np, layer.wr_np, layer.bias_np, layer.k)
    for prec, tol in (("fp16_weights", 1e-4), ("exact", TOL)):
        ref = oracle.moe_layer(layer.x_np, layer.wr_np, layer.bias_np, layer.k, layer.blob_np, layer.shared_np,
                               layer.d_model, layer.d_ff, precision=prec, idx=gpu["idx"], w=gpu["w"])
        err = rel_err(gpu["out"], ref["out64"])
        say(f"    fused layer vs {prec}: out {err:.2e}")
        assert err <= tol
    layer.close()


def test_fused_layer_refusals():
    d, f, E, k = TINY["d"], TINY["f"], TINY["E"], TINY["k"]
    res = _ctx(d, f, E, k, 1, 520)
    buf = res.buffers(520)
    wr, bias, _ = _inputs(d, E, 1, 520, seed=1, alpha=0.0)
    x = torch.from_numpy(moe_synth.gen_x(1, 0, 520, d)).cuda()
    buf["out"].fill_(3.0)
    with pytest.raises(B.MoeError) as ei:  # T * top_k = 1,026 > 1,024
        B.moe_decode_layer(res.ctx, 0, x, 513, wr[0], bias[0], None, buf["idx"], buf["w"], buf["y_pairs"],
                           buf["y_shared"], buf["out"], None)
    assert ei.value.status == B.MOE_ERR_INVALID
    with pytest.raises(B.MoeError) as ei:  # x_next aliasing out
        B.moe_decode_layer(res.ctx, 0, x, 8, wr[0], bias[0], None, buf["idx"], buf["w"], buf["y_pairs"],
                           buf["y_shared"], buf["out"], buf["out"])
    assert ei.value.status == B.MOE_ERR_INVALID
    # a capped cache whose host store is pageable (not mapped into the device address space)
    cap = MoeContext(d, f, E, k, 1, 8, 8, host_store=torch.zeros((E, res.stride), dtype=torch.uint8))
    cbuf = cap.buffers(8)
    with pytest.raises(B.MoeError) as ei:
        B.moe_decode_layer(cap.ctx, 0, x, 8, wr[0], bias[0], None, cbuf["idx"], cbuf["w"], cbuf["y_pairs"],
                           cbuf["y_shared"], cbuf["out"], None)
    assert ei.value.status == B.MOE_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.all(buf["out"] == 3.0)  # nothing was enqueued
    st = B.moe_get_stats(res.ctx)
    assert st["resolve_calls"] == 0
    res.close()
    cap.close()
