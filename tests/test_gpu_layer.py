"""GPU parity of the routed MoE layer against the CPU oracle, through the C ABI.

Both paths round only the dequantised weights to fp16 (activations carried as
hi + lo fp16 halves, fp32 sums): they are compared with the oracle's
'fp16_weights' mode at a tight tolerance, and with the exact float64
definition at the stated bar (max |err| <= 2e-3 x RMS of the call's output).
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from _gpu_helpers import TOL, check_bucket, check_routing, rel_err, say
from quantized_expert_ffn_softmax_amd import binding as B

pytestmark = pytest.mark.gpu

TINY = dict(d_model=256, d_ff=128, n_experts=16, top_k=2)
REAL = dict(d_model=2048, d_ff=768, n_experts=512, top_k=10)


def _layer(seed=0, T=8, alpha=0.0, **shape):
    from moe_synth.harness import SyntheticLayer
    return SyntheticLayer(seed=seed, n_tokens=T, alpha=alpha, device="cuda:0", **shape)


def _oracle(layer, gpu, precision):
    return oracle.moe_layer(layer.x_np, layer.wr_np, layer.bias_np, layer.k, layer.blob_np, layer.shared_np,
                            layer.d_model, layer.d_ff, precision=precision, idx=gpu["idx"], w=gpu["w"])


def _check_layer(layer, path, tight_prec, tight_tol):
    say(f"  layer T={layer.T} E={layer.E} k={layer.k} d={layer.d_model} f={layer.d_ff} path={path}")
    gpu = layer.forward_gpu(path)
    ties = check_routing(gpu, layer.x_np, layer.wr_np, layer.bias_np, layer.k)
    ref = _oracle(layer, gpu, tight_prec)
    e_pairs = rel_err(gpu["y_pairs"], ref["y_pairs"])
    e_shared = rel_err(gpu["y_shared"], ref["y_shared"])
    e_out = rel_err(gpu["out"], ref["out64"])
    exact = _oracle(layer, gpu, "exact")
    e_exact = rel_err(gpu["out"], exact["out64"])
    say(f"    near-ties {ties}; vs {tight_prec}: pairs {e_pairs:.2e} shared {e_shared:.2e} out {e_out:.2e}; "
        f"vs exact: out {e_exact:.2e}")
    assert e_pairs <= tight_tol and e_shared <= tight_tol and e_out <= tight_tol
    assert e_exact <= TOL
    # combine on the GPU's own expert outputs
    comb = oracle.combine(gpu["y_pairs"].astype(np.float64), gpu["w"].astype(np.float64),
                          gpu["y_shared"].astype(np.float64))
    assert rel_err(gpu["out"], comb) <= 1e-6
    return gpu


@pytest.mark.parametrize("T", [1, 3, 8, 17, 40])
def test_tiny_decode(T):
    layer = _layer(T=T, **TINY)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


def test_tiny_decode_past_the_small_bucketing():
    # 140 tokens x 8 of 64 experts = 1,120 pairs: the multi-workgroup bucketing,
    # whose entries carry no row lists (the decode kernels then read perm)
    layer = _layer(T=140, **dict(TINY, n_experts=64, top_k=8))
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


@pytest.mark.parametrize("d_model,d_ff", [(64, 64), (1024, 512), (640, 2048)])
def test_decode_other_widths(d_model, d_ff):
    # the decode kernels are built per superblock count (160 columns each):
    # 1/1, 7/4 and 4/13 superblocks for gate-up/down, with the last scale
    # block of a row at the clamp and a wide down matrix
    layer = _layer(T=9, d_model=d_model, d_ff=d_ff, n_experts=16, top_k=3)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


def test_decode_width_limit():
    # d_model = 2112 is 14 superblocks: the decode path refuses it, the
    # automatic choice takes the prefill path (still checked at the bar)
    layer = _layer(T=6, d_model=2112, d_ff=128, n_experts=16, top_k=2)
    with pytest.raises(B.MoeError) as ei:
        layer.forward_gpu(B.MOE_PATH_DECODE)
    assert ei.value.status == B.MOE_ERR_INVALID
    _check_layer(layer, B.MOE_PATH_AUTO, "fp16_weights", 1e-4)
    layer.close()


@pytest.mark.parametrize("T", [1, 8, 65, 130])
def test_tiny_prefill(T):
    layer = _layer(T=T, **TINY)
    _check_layer(layer, B.MOE_PATH_PREFILL, "fp16_weights", 1e-4)
    layer.close()


@pytest.mark.parametrize("k", [1, 16])
def test_tiny_k_extremes(k):
    shape = dict(TINY, top_k=k)
    layer = _layer(T=8, **shape)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    _check_layer(layer, B.MOE_PATH_PREFILL, "fp16_weights", 1e-4)
    layer.close()


def _set_scales(layer, lo, hi, seed):
    """Overwrite every block scale of the layer's blobs (routed and shared) with
    seeded fp16 values of magnitude in [lo, hi] and random sign, on the GPU
    pools and in the copies the oracle reads."""
    rng = np.random.default_rng(seed)
    secs, _stride = oracle.blob_sections(layer.d_model, layer.d_ff)
    for e in range(layer.E + 1):
        blob = layer.blob_np(e)
        for _name, rows, cols, _co, so in secs:
            n = rows * (cols // 32)
            mag = rng.uniform(lo, hi, n) * rng.choice([-1.0, 1.0], n)
            blob[so:so + 2 * n] = np.frombuffer(mag.astype(np.float16).tobytes(), dtype=np.uint8)
        pool = layer.ctx.shared_pool[0] if e == layer.E else layer.ctx.slot_pool[e]
        pool.copy_(torch.from_numpy(blob).to(pool.device))
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", [B.MOE_PATH_DECODE, B.MOE_PATH_PREFILL])
@pytest.mark.parametrize("scales", ["large", "small"])
def test_block_scale_range_edges(path, scales):
    # the valid scale range is 2^-14 <= |s| <= 255.875: the kernels form
    # f fp16((q - 4) s) with f up to 64 in the in-place code slots.  x and h
    # travel as hi + lo fp16 halves of v / f, exact to ~2^-22 |v| while the lo
    # half is a normal fp16 number (|v| >= 1/8) and to an absolute 2^-25
    # below that: f 2^-25 = 2^-19 in x's units at f = 64.  Near 255.875
    # (|w| ~ 440) h stays below fp16's overflow only for |x| <~ 0.01 at
    # d_model 256 (h ~ (16 * 440 |x|)^2), so x there is a random sign times
    # U(0.004, 0.008) -- v / f still normal -- and the floor is
    # 2^-19 / 0.004 = 4.8e-4 of an element of x: tolerance 1e-3 against
    # 'fp16_weights' (plus the exact bar).  The smallest scales take x ~ 1000
    # and the usual 1e-4.
    x = moe_synth.gen_x(7, 0, 9, TINY["d_model"])
    if scales == "large":
        lo, hi, tol = 128.0, 255.875, 1e-3
        mag = np.random.default_rng(9).uniform(0.004, 0.008, x.shape)
        x = (np.where(x < 0, -1.0, 1.0) * mag).astype(np.float32)
    else:
        lo, hi, tol = 2.0 ** -14, 2.0 ** -10, 1e-4
        x = (x * 1e3).astype(np.float32)
    layer = _layer(seed=7, T=9, x=x, **TINY)
    _set_scales(layer, lo, hi, seed=8)
    _check_layer(layer, path, "fp16_weights", tol)
    layer.close()


@pytest.mark.parametrize("T,alpha", [(1, 0.0), (1, 0.75), (2, 0.75)])
def test_real_layer_decode_small_batches(T, alpha):
    # one token: gate/up's ~11 entries x 48 one-tile units fit in the CUs at
    # once, so K is split in four (13 = 4 + 3 + 3 + 3 superblocks); two tokens
    # take the halves
    layer = _layer(seed=11 + T, T=T, alpha=alpha, **REAL)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


def test_real_layer_decode_T5():
    layer = _layer(T=5, **REAL)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


def test_real_layer_decode_T15_zipf():
    layer = _layer(T=15, alpha=0.75, **REAL)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


def test_real_layer_decode_T28_zipf():
    # 4 request slots x (1 + 6) verified tokens: the decode-size router's largest
    # batches take two 16-token groups
    layer = _layer(T=28, alpha=0.75, **REAL)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


def test_real_layer_decode_T40_zipf():
    # past the K-split range (up to 32 tokens): the unsplit gate/up kernel at
    # the real width, and the router's third 16-token group
    layer = _layer(T=40, alpha=0.75, **REAL)
    _check_layer(layer, B.MOE_PATH_DECODE, "fp16_weights", 1e-4)
    layer.close()


def test_real_layer_prefill_small():
    layer = _layer(T=200, alpha=0.75, **REAL)
    _check_layer(layer, B.MOE_PATH_PREFILL, "fp16_weights", 1e-4)
    layer.close()


def test_deterministic():
    layer = _layer(T=15, alpha=0.75, **REAL)
    for path in (B.MOE_PATH_DECODE, B.MOE_PATH_PREFILL):
        a = layer.forward_gpu(path)
        b = layer.forward_gpu(path)
        for key in ("logits", "idx", "w", "y_pairs", "y_shared", "out"):
            assert np.array_equal(a[key], b[key]), (path, key)
    layer.close()


def test_bucket_small_and_large():
    for T in (8, 300, 2000):
        layer = _layer(T=T, **REAL) if T <= 300 else None
        ctx = layer.ctx if layer else None
        if ctx is None:
            from quantized_expert_ffn_softmax_amd.runtime import MoeContext
            ctx = MoeContext(256, 128, 512, 10, 1, None, T)
        rng = np.random.default_rng(T)
        idx = np.stack([rng.choice(512, 10, replace=False) for _ in range(T)]).astype(np.int32)
        idx_d = torch.from_numpy(idx).cuda()
        off = torch.empty(513, dtype=torch.int32, device="cuda")
        perm = torch.empty(T * 10, dtype=torch.int32, device="cuda")
        B.moe_bucket(ctx.ctx, idx_d, T, off, perm)
        torch.cuda.synchronize()
        check_bucket(off.cpu().numpy(), perm.cpu().numpy(), idx, 512)
        ctx.close()


@pytest.mark.parametrize("case", ["skewed", "n1024", "e1024", "one_expert", "e1k1"])
def test_bucket_small_path_edges(case):
    # the single-workgroup bucketing (<= 1024 pairs): long segments, the
    # pair and expert limits, every pair on one expert, the smallest shape
    from quantized_expert_ffn_softmax_amd.runtime import MoeContext
    E, k, T = {"skewed": (512, 10, 100), "n1024": (512, 8, 128), "e1024": (1024, 10, 60),
               "one_expert": (512, 4, 200), "e1k1": (1, 1, 37)}[case]
    assert T * k <= 1024
    rng = np.random.default_rng(7)
    if case == "skewed":
        # every token on experts 0..k-1 in shuffled order: segments of length T
        idx = np.stack([rng.permutation(k) for _ in range(T)])
    elif case == "one_expert":
        idx = np.full((T, k), 333)  # repeated ids inside a token too
    elif case == "e1k1":
        idx = np.zeros((T, k))
    else:
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    idx = idx.astype(np.int32)
    say(f"  bucketing {case}: E={E} k={k} T={T}")
    ctx = MoeContext(256, 128, E, k, 1, None, T)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    B.moe_bucket(ctx.ctx, torch.from_numpy(idx).cuda(), T, off, perm)
    torch.cuda.synchronize()
    check_bucket(off.cpu().numpy(), perm.cpu().numpy(), idx, E)
    ctx.close()


@pytest.mark.parametrize("E", [1000, 1024])
def test_bucket_large_path_expert_limit(E):
    # the histogram/scan/scatter bucketing (> 1024 pairs) up to 1,024 experts:
    # offsets[E] (the pair total) comes from thread 0, as no thread E exists
    # at E = 1024; the output buffers start poisoned so an unwritten entry shows
    from quantized_expert_ffn_softmax_amd.runtime import MoeContext
    k, T = 10, 300
    rng = np.random.default_rng(E)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    say(f"  bucketing past 1024 pairs: E={E} k={k} T={T}")
    ctx = MoeContext(256, 128, E, k, 1, None, T)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    B.moe_bucket(ctx.ctx, torch.from_numpy(idx).cuda(), T, off, perm)
    off2, perm2 = torch.full_like(off, -9), torch.full_like(perm, -9)
    B.moe_bucket_noalloc(torch.from_numpy(idx).cuda(), T, k, E, off2, perm2)
    torch.cuda.synchronize()
    check_bucket(off.cpu().numpy(), perm.cpu().numpy(), idx, E)
    assert torch.equal(off, off2) and torch.equal(perm, perm2)
    ctx.close()


@pytest.mark.parametrize("T", [8, 40, 100])
def test_router_exact_ties(T):
    # zero router weights: every logit is exactly its bias, and the bias holds
    # repeated values (and a -0.0 beside +0.0), so the top-k is decided by the
    # index rule alone; both router paths (T <= 64 and above) must pick the
    # lowest indices among equal logits and weight them by the softmax
    from quantized_expert_ffn_softmax_amd.runtime import MoeContext
    E, k, d = 64, 8, 256
    ctx = MoeContext(d, 128, E, k, 1, None, T)
    x = torch.from_numpy(moe_synth.gen_x(1, 0, T, d)).cuda()
    wr = torch.zeros((E, d), dtype=torch.float32, device="cuda")
    bias_np = np.array([(e * 7) % 5 for e in range(E)], dtype=np.float32) * np.float32(0.25)
    bias_np[[0, 5, 10]] = 0.0
    bias_np[[3, 8]] = -0.0
    bias = torch.from_numpy(bias_np).cuda()
    buf = ctx.buffers(T)
    B.moe_route(ctx.ctx, 0, x, T, wr, bias, buf["logits"], buf["idx"], buf["w"])
    torch.cuda.synchronize()
    logits = buf["logits"].cpu().numpy()
    assert np.array_equal(logits, np.broadcast_to(bias_np, (T, E)))
    want_idx, want_w = oracle.topk_from_logits(logits, k)
    assert np.array_equal(buf["idx"].cpu().numpy(), want_idx)
    assert np.abs(buf["w"].cpu().numpy() - want_w).max() <= 1e-6
    ctx.close()


@pytest.mark.parametrize("shape,T", [("tiny", 8), ("real", 1), ("real", 15), ("real", 64), ("k20_d1088", 5),
                                     ("d8192", 3)])
def test_combine_norm_equals_the_two_calls(shape, T):
    # k20_d1088: more than 16 pair rows (the looped path) and a row whose
    # columns end part-way through the threads; d8192: four float4 columns
    # per thread
    dims = {"tiny": TINY, "real": REAL,
            "k20_d1088": dict(d_model=1088, d_ff=128, n_experts=64, top_k=20),
            "d8192": dict(d_model=8192, d_ff=128, n_experts=16, top_k=4)}[shape]
    from quantized_expert_ffn_softmax_amd.runtime import MoeContext
    d, k = dims["d_model"], dims["top_k"]
    ctx = MoeContext(d, dims["d_ff"], dims["n_experts"], k, 1, None, T)
    g = torch.Generator().manual_seed(T)
    yp = torch.randn((T * k, d), generator=g).cuda()
    ys = torch.randn((T, d), generator=g).cuda()
    w = torch.softmax(torch.randn((T, k), generator=g), dim=1).cuda()
    out1, xn1 = torch.empty((T, d), device="cuda"), torch.empty((T, d), device="cuda")
    out2, xn2 = torch.empty_like(out1), torch.empty_like(xn1)
    B.moe_combine(ctx.ctx, yp, w, ys, T, out1)
    B.moe_chain_norm(ctx.ctx, out1, T, xn1)
    B.moe_combine_norm(ctx.ctx, yp, w, ys, T, out2, xn2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(xn1, xn2)
    ref = oracle.combine(yp.cpu().double().numpy(), w.cpu().double().numpy(), ys.cpu().double().numpy())
    assert rel_err(out2.cpu().numpy(), ref) <= 1e-6
    assert rel_err(xn2.cpu().numpy(), oracle.chain_norm(ref)) <= 1e-5
    ctx.close()
