#!/usr/bin/env python3
"""Benchmark of the routed MoE layer (libmoe) on one MI355X.

Workload (one "step"): 15 tokens -- 3 request slots x (1 + 4 draft tokens)
verified together -- through the 48-layer stack, every layer routing each
token to 10 of 512 experts plus the shared expert, with all 24,576 expert
identities resident in HBM (54.8 GB of 3-bit blobs) and Zipf-skewed router
bias (alpha 0.75).  Per layer: moe_route -> moe_cache_resolve ->
moe_expert_ffn (decode path) -> moe_combine_norm (moe_combine and the
stacking normalisation moe_chain_norm in one kernel; it feeds the next
layer).  Inputs are synthetic and seeded; weights are random.

Also timed: measured HBM-read and fp16-MFMA peaks of the device, the prefill
chunk (12,288 tokens through one layer, prefill path), a single layer at
5 tokens, the speculative-verify sweep, the 1-token stack through the
8,445-slot LRU cache, and the CPU oracle on bounded samples of the decode and
prefill workloads.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algo_blob_bytes(d_model, d_ff):
    """Algorithmic bytes of one expert: 3.2 code bits + 0.5 scale bits per weight."""
    weights = 3 * d_model * d_ff
    return weights * (3.2 + 0.5) / 8.0


def recorded_traffic():
    """HBM bytes per decode moe_expert_ffn call from the committed counter
    summary, or None when the summary is missing or the kernel sources it was
    taken on have changed since (their sha256 is stored with the figure)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "decode_ffn_T15_traffic.md")
    try:
        text = open(path).read()
        rec = json.loads(re.search(r"```json\n(.*?)```", text, re.S).group(1))
        h = hashlib.sha256()
        for f in rec["sources"]:
            with open(os.path.join(ROOT, "quantized_expert_ffn_softmax_amd", "csrc", f), "rb") as fh:
                h.update(fh.read())
        return int(rec["traffic"]) if h.hexdigest() == rec["sha256"] else None
    except (OSError, ValueError, KeyError, AttributeError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--cpu-sample-layers", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-layer", action="store_true", help="skip the single-layer T=5 decode measurement")
    ap.add_argument("--no-lru", action="store_true", help="skip the T=1 stack through the 8,445-slot LRU cache")
    ap.add_argument("--no-sweep", action="store_true", help="skip the speculative-verify batch sweep")
    ap.add_argument("--no-kv", action="store_true", help="skip the KV-tier leg (131,072-cell context reads)")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 48-layer decode stack (the headline figure is then null; for profiling other legs)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured HBM-read and MFMA-loop peaks")
    ap.add_argument("--lru-steps", type=int, default=256)
    ap.add_argument("--lru-warmup", type=int, default=64)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU layout is described in DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_synth
    from moe_synth.harness import fill_pool
    from quantized_expert_ffn_softmax_amd import binding as B
    from quantized_expert_ffn_softmax_amd.runtime import MoeContext

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    wl = moe_synth.WORKLOADS["batched_decode_stack"]
    d, f, E, k, L, T = wl["d_model"], wl["d_ff"], wl["n_experts"], wl["top_k"], wl["n_layers"], wl["n_tokens"]
    alpha, seed = wl["alpha"], args.seed
    stride = B.moe_expert_bytes(d, f)
    prefill_T = moe_synth.WORKLOADS["prefill_chunk"]["n_tokens"]

    t0 = time.time()
    # the stack and the sweep need all 48 layers; the other legs use layer 0
    L_gen = L if not (args.no_stack and args.no_sweep) else 1
    log(f"[bench] allocating {L * E} + {L} blobs x {stride} B in HBM (generating {L_gen} layer(s))")
    slot_pool = torch.empty((L * E, stride), dtype=torch.uint8, device="cuda")
    shared_pool = torch.empty((L, stride), dtype=torch.uint8, device="cuda")
    for l0 in range(0, L_gen, 8):
        l1 = min(l0 + 8, L_gen)
        fill_pool(slot_pool[l0 * E:l1 * E], list(range(l0 * E, l1 * E)), seed, d, f, E, chunk=512)
        log(f"[bench] generated layers {l0}..{l1 - 1} ({time.time() - t0:.0f}s)")
    fill_pool(shared_pool, [(l, E) for l in range(L)], seed, d, f, E)
    routers = torch.stack([torch.from_numpy(moe_synth.gen_router(seed, l, E, d)) for l in range(L)]).cuda()
    biases = torch.stack([torch.from_numpy(moe_synth.gen_bias(seed, l, E, alpha)) for l in range(L)]).cuda()
    max_tokens = max(T, prefill_T)
    ctx = MoeContext(d, f, E, k, L, None, max_tokens, slot_pool=slot_pool, shared_pool=shared_pool)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.time() - t0:.0f}s")

    peaks = None if args.no_peaks else measure_peaks(slot_pool)
    result = {
        "metric": "MoE decode tok/s (48 layers) + prefill tok/s; % of HBM BW / MFMA peak",
        "value": None,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "batched_decode_stack", "layers": L, "experts_per_layer": E, "top_k": k,
                   "shared_experts": 1, "tokens_per_step": T, "d_model": d, "d_ff": f,
                   "resident_identities": L * E, "zipf_alpha": alpha, "expert_blob_bytes": stride,
                   "seed": seed},
    }
    if peaks is not None:
        result["measured_peaks"] = peaks
    if not args.no_stack:
        result.update(bench_stack(ctx, routers, biases, seed, d, f, L, T, args.warmup, args.steps,
                                  not args.no_graph, peaks))
    if not args.no_prefill:
        result["prefill"] = bench_prefill(ctx, routers[0], biases[0], seed, d, f, k, prefill_T, args.prefill_reps,
                                          peaks)
    if not args.no_sweep:
        result["verify_sweep"] = verify_sweep(ctx, routers, biases, seed, d, f, L)
    if not args.no_layer:
        result["decode_layer"] = bench_decode_layer(ctx, routers[0], seed, d, f, E, k)
    ctx.close()
    del ctx, slot_pool
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_lru:
        result["decode_lru"] = bench_lru(seed, d, f, E, k, L, routers, biases, shared_pool, args.lru_warmup,
                                         args.lru_steps)
    if not args.no_kv:
        result["kv_tier"] = bench_kv(seed, peaks)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(seed, d, f, E, k, T, alpha, args.cpu_sample_layers, args.warmup,
                                              prefill_T)
    print(json.dumps(result), flush=True)


def _median_ms(pairs):
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in pairs]))


def measure_peaks(buf, read_bytes=4 << 30, reps=5):
    """Achievable peaks on this device: a streaming read of `read_bytes` of the
    (already filled) expert pool, and a loop of independent dense fp16 MFMAs
    (v_mfma_f32_32x32x16_f16).  Median of `reps` timed launches after one
    warm-up each."""
    import torch

    from quantized_expert_ffn_softmax_amd import binding as B
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    flat = buf.view(-1)
    nbytes = min(read_bytes, flat.numel()) // 16 * 16
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    blocks = n_cu * 8
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(reps + 1)]
    for a, b in ev:
        a.record()
        B.moe_peak_hbm_read(flat, nbytes, sink, blocks)
        b.record()
    torch.cuda.synchronize()
    hbm_ms = _median_ms(ev[1:])
    iters, mblocks = 32768, n_cu * 2  # ~2 ms a launch: long enough for clocks to settle
    flops = mblocks * 4 * iters * 4 * 32768.0
    for a, b in ev:
        a.record()
        B.moe_peak_mfma_f16(iters, mblocks, sink)
        b.record()
    torch.cuda.synchronize()
    mfma_ms = _median_ms(ev[1:])
    out = {"hbm_read_gbs": round(nbytes / (hbm_ms * 1e-3) / 1e9, 1), "hbm_read_bytes": nbytes,
           "hbm_frac_of_spec": round(nbytes / (hbm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "mfma_f16_tflops": round(flops / (mfma_ms * 1e-3) / 1e12, 1),
           "mfma_frac_of_spec": round(flops / (mfma_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
           "how": f"moe_peak_hbm_read over {nbytes >> 20} MiB ({blocks} workgroups); moe_peak_mfma_f16 "
                  f"{mblocks} x 4 waves x {iters} x 4 v_mfma_f32_32x32x16_f16; median of {reps} launches"}
    log(f"[bench] measured peaks: HBM read {out['hbm_read_gbs']} GB/s, fp16 MFMA {out['mfma_f16_tflops']} TFLOP/s")
    return out


def bench_stack(ctx, routers, biases, seed, d, f, L, T, W, K, use_graph, peaks):
    """The headline: the 48-layer batched-decode stack, eager with HIP events
    around every moe_expert_ffn call, then captured in a HIP graph."""
    import numpy as np
    import torch

    import moe_synth
    from quantized_expert_ffn_softmax_amd import binding as B
    c = ctx.ctx
    xs = [torch.from_numpy(moe_synth.gen_x(seed, s, T, d)).cuda() for s in range(W + K)]
    buf = ctx.buffers(T)
    xa = torch.empty((T, d), dtype=torch.float32, device="cuda")
    xb = torch.empty_like(xa)

    def step_fused(x0):
        # the same layers, six launches each (moe_decode_layer)
        x = x0
        for l in range(L):
            xn = xa if (l % 2 == 0) else xb
            B.moe_decode_layer(c, l, x, T, routers[l], biases[l], None, buf["idx"], buf["w"], buf["y_pairs"],
                               buf["y_shared"], buf["out"], xn)
            x = xn

    def step(x0, ev=None):
        x = x0
        for l in range(L):
            B.moe_route(c, l, x, T, routers[l], biases[l], None, buf["idx"], buf["w"])
            B.moe_cache_resolve(c, l, buf["idx"], T, None)
            if ev is not None:
                ev[l][0].record()
            B.moe_expert_ffn(c, l, x, T, buf["idx"], None, buf["y_pairs"], buf["y_shared"], B.MOE_PATH_DECODE)
            if ev is not None:
                ev[l][1].record()
            xn = xa if (l % 2 == 0) else xb
            B.moe_combine_norm(c, buf["y_pairs"], buf["w"], buf["y_shared"], T, buf["out"], xn)
            x = xn

    for s in range(W):
        step(xs[s])
    torch.cuda.synchronize()
    st0 = B.moe_get_stats(c)
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(L)]
           for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(K):
        step(xs[W + s], evs[s])
    end.record()
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(end)
    st1 = B.moe_get_stats(c)
    ffn_ms = [evs[s][l][0].elapsed_time(evs[s][l][1]) for s in range(K) for l in range(L)]
    calls = st1["resolve_calls"] - st0["resolve_calls"]
    uniq = st1["lookups"] - st0["lookups"]
    blob_algo = algo_blob_bytes(d, f)
    ffn_bytes_total = (uniq + calls) * blob_algo  # touched routed experts + one shared per layer call
    ffn_avg_ms = float(np.mean(ffn_ms))
    bytes_per_call = ffn_bytes_total / calls
    achieved = bytes_per_call / (ffn_avg_ms * 1e-3) / 1e9
    eager_ms = elapsed_ms / K
    log(f"[bench] decode stack (eager): {eager_ms:.3f} ms/step, {T * K / (elapsed_ms * 1e-3):.0f} tok/s; expert-FFN "
        f"call {ffn_avg_ms * 1e3:.1f} us for {bytes_per_call / 1e6:.1f} MB -> {achieved:.0f} GB/s; "
        f"distinct experts/layer {uniq / calls:.1f}")

    # the step captured once in a HIP graph (the deployable form of a
    # fixed-shape decode step), replayed on fresh inputs copied in beforehand:
    # first as the seven launches per layer of the separate calls, then as the
    # six of moe_decode_layer (the headline)
    spread = {}

    def graph_time(fn, xs=xs, Tn=T):
        xin = torch.empty((Tn, d), dtype=torch.float32, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            xin.copy_(xs[0])
            fn(xin)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn(xin)
        torch.cuda.synchronize()
        for s_ in range(W):
            xin.copy_(xs[s_])
            graph.replay()
        torch.cuda.synchronize()
        gev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(K)]
        for s_ in range(K):
            xin.copy_(xs[W + s_])
            gev[s_][0].record()
            graph.replay()
            gev[s_][1].record()
        torch.cuda.synchronize()
        del graph
        ts = [a.elapsed_time(b) for a, b in gev]
        spread["graph_ms"] = {"median": round(float(np.median(ts)), 4), "min": round(float(np.min(ts)), 4),
                              "max": round(float(np.max(ts)), 4)}
        return float(np.mean(ts))

    graph_ms = sep_graph_ms = None
    if use_graph:
        sep_graph_ms = graph_time(step)
        log(f"[bench] decode stack (graph, separate calls, 7 launches/layer): {sep_graph_ms:.3f} ms/step, "
            f"{T / (sep_graph_ms * 1e-3):.0f} tok/s")
        sep_spread = dict(spread)
        graph_ms = graph_time(step_fused)
        log(f"[bench] decode stack (graph, moe_decode_layer, 6 launches/layer): {graph_ms:.3f} ms/step, "
            f"{T / (graph_ms * 1e-3):.0f} tok/s")
        fused_spread = dict(spread)
        # one token per step through the same resident layers: where launch
        # gaps weigh most (moe_decode_layer: five launches per layer at T = 1)
        b1 = ctx.buffers(1)
        x1 = [torch.empty((1, d), dtype=torch.float32, device="cuda") for _ in range(2)]
        xs1 = [torch.from_numpy(moe_synth.gen_x(seed, 700000 + s_, 1, d)).cuda() for s_ in range(W + K)]

        def step1(x0, fused):
            x = x0
            for l in range(L):
                xn = x1[l % 2]
                if fused:
                    B.moe_decode_layer(c, l, x, 1, routers[l], biases[l], None, b1["idx"], b1["w"], b1["y_pairs"],
                                       b1["y_shared"], b1["out"], xn)
                else:
                    B.moe_route(c, l, x, 1, routers[l], biases[l], None, b1["idx"], b1["w"])
                    B.moe_cache_resolve(c, l, b1["idx"], 1, None)
                    B.moe_expert_ffn(c, l, x, 1, b1["idx"], None, b1["y_pairs"], b1["y_shared"], B.MOE_PATH_DECODE)
                    B.moe_combine_norm(c, b1["y_pairs"], b1["w"], b1["y_shared"], 1, b1["out"], xn)
                x = xn

        t1_sep = graph_time(lambda x0: step1(x0, False), xs1, 1)
        t1_fused = graph_time(lambda x0: step1(x0, True), xs1, 1)
        t1 = {"tokens_per_step": 1, "ms_per_step": round(t1_fused, 4), "tok_per_s": round(1 / (t1_fused * 1e-3), 1),
              "launches_per_layer": 5, "separate_calls_ms_per_step": round(t1_sep, 4),
              "separate_calls_tok_per_s": round(1 / (t1_sep * 1e-3), 1), "mode": "hip_graph, resident"}
        log(f"[bench] decode stack at T=1 (graph): moe_decode_layer (5 launches/layer) {t1_fused:.3f} ms/step "
            f"= {t1['tok_per_s']} tok/s; separate calls (7 launches/layer) {t1_sep:.3f} ms/step")
        spread = fused_spread
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    roof = {"bound": "hbm", "kernel": "moe_expert_ffn (decode path)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "bytes_per_launch": round(bytes_per_call), "avg_launch_us": round(ffn_avg_ms * 1e3, 2),
            "distinct_experts_per_layer": round(uniq / calls, 2),
            "measured_in": "eager timed region (HIP events around each moe_expert_ffn call)",
            "stack_bytes_per_step": round(ffn_bytes_total / K),
            "stack_frac": round(ffn_bytes_total / K / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if peaks is not None:
        roof["measured_peak"] = peaks["hbm_read_gbs"]
        roof["frac_of_measured"] = round(achieved / peaks["hbm_read_gbs"], 4)
    res = {"value": round(T / (ms_per_step * 1e-3), 1), "ms_per_step": round(ms_per_step, 4), "roofline": roof,
           "eager_ms_per_step": round(eager_ms, 4),
           "step_mode": "hip_graph, moe_decode_layer (6 launches per layer)" if graph_ms is not None
           else "eager, separate calls (7 launches per layer)"}
    if graph_ms is not None:
        res["ms_per_step_spread"] = spread["graph_ms"]
    if sep_graph_ms is not None:
        res["separate_calls_graph_ms_per_step"] = round(sep_graph_ms, 4)
        res["separate_calls_ms_per_step_spread"] = sep_spread["graph_ms"]
        res["decode_stack_T1"] = t1
        res["separate_calls_tok_per_s"] = round(T / (sep_graph_ms * 1e-3), 1)
    return res


def bench_prefill(ctx, router, bias, seed, d, f, k, T, reps, peaks):
    """The prefill chunk: T tokens through one real layer (route, resolve,
    expert FFN on the prefill path, combine); medians over `reps` after one
    warm-up."""
    import numpy as np
    import torch

    import moe_synth
    from quantized_expert_ffn_softmax_amd import binding as B
    c = ctx.ctx
    xp = torch.from_numpy(moe_synth.gen_x(seed, 100000, T, d)).cuda()
    pbuf = ctx.buffers(T)
    warm = 3
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps + warm)]
    for r in range(reps + warm):
        e = pev[r]
        e[0].record()
        B.moe_route(c, 0, xp, T, router, bias, None, pbuf["idx"], pbuf["w"])
        B.moe_cache_resolve(c, 0, pbuf["idx"], T, None)
        e[1].record()
        B.moe_expert_ffn(c, 0, xp, T, pbuf["idx"], None, pbuf["y_pairs"], pbuf["y_shared"], B.MOE_PATH_PREFILL)
        e[2].record()
        B.moe_combine(c, pbuf["y_pairs"], pbuf["w"], pbuf["y_shared"], T, pbuf["out"])
        e[3].record()
    torch.cuda.synchronize()
    layer_t = [pev[r][0].elapsed_time(pev[r][3]) for r in range(warm, reps + warm)]
    ffn_t = [pev[r][1].elapsed_time(pev[r][2]) for r in range(warm, reps + warm)]
    layer_ms, ffn_p_ms = float(np.median(layer_t)), float(np.median(ffn_t))
    flops = 6.0 * d * f * (T * k + T)
    tflops = flops / (ffn_p_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": "moe_expert_ffn (prefill path)",
            "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "flops_per_launch": flops}
    if peaks is not None:
        roof["measured_peak"] = peaks["mfma_f16_tflops"]
        roof["frac_of_measured"] = round(tflops / peaks["mfma_f16_tflops"], 4)
    log(f"[bench] prefill chunk: layer {layer_ms:.2f} ms ({T / (layer_ms * 1e-3):.0f} tok/s), "
        f"FFN {ffn_p_ms:.2f} ms = {tflops:.1f} TFLOP/s")
    return {"workload": "prefill_chunk", "tokens": T, "tok_per_s": round(T / (layer_ms * 1e-3), 1),
            "layer_ms": round(layer_ms, 4), "ffn_ms": round(ffn_p_ms, 4), "warmup": warm, "reps": reps,
            "layer_ms_min_max": [round(min(layer_t), 4), round(max(layer_t), 4)],
            "ffn_ms_min_max": [round(min(ffn_t), 4), round(max(ffn_t), 4)],
            "timing": "HIP events; medians over the timed reps", "roofline": roof}


def bench_decode_layer(ctx, router, seed, d, f, E, k, reps=200):
    """One real layer at T = 5 (one request: 1 + 4 draft tokens), no router
    bias, a fresh x per repetition and 1 GiB written between repetitions:
    route -> resolve -> expert FFN -> combine."""
    import numpy as np
    import torch

    import moe_synth
    from quantized_expert_ffn_softmax_amd import binding as B
    wl = moe_synth.WORKLOADS["decode_layer"]
    T = wl["n_tokens"]
    c = ctx.ctx
    xs = [torch.from_numpy(moe_synth.gen_x(seed, 200000 + r, T, d)).cuda() for r in range(reps + 10)]
    buf = ctx.buffers(T)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 10)]
    # one real layer's ~107 MB of expert bytes fit in the 256 MB last-level
    # cache: 1 GiB is written between repetitions (outside the timed events)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    st0 = None
    for r in range(reps + 10):
        if r == 10:
            torch.cuda.synchronize()
            st0 = B.moe_get_stats(c)
        flush.fill_(r & 0xff)
        e = ev[r]
        e[0].record()
        B.moe_route(c, 0, xs[r], T, router, None, None, buf["idx"], buf["w"])
        B.moe_cache_resolve(c, 0, buf["idx"], T, None)
        e[1].record()
        B.moe_expert_ffn(c, 0, xs[r], T, buf["idx"], None, buf["y_pairs"], buf["y_shared"], B.MOE_PATH_DECODE)
        e[2].record()
        B.moe_combine(c, buf["y_pairs"], buf["w"], buf["y_shared"], T, buf["out"])
    torch.cuda.synchronize()
    st1 = B.moe_get_stats(c)
    layer_t = [ev[r][0].elapsed_time(ev[r][2]) * 1e3 for r in range(10, reps + 10)]
    ffn_t = [ev[r][1].elapsed_time(ev[r][2]) * 1e3 for r in range(10, reps + 10)]
    layer_us, ffn_us = float(np.mean(layer_t)), float(np.mean(ffn_t))
    uniq = (st1["lookups"] - st0["lookups"]) / reps
    gbs = (uniq + 1) * algo_blob_bytes(d, f) / (ffn_us * 1e-6) / 1e9
    log(f"[bench] decode layer T={T}: route+resolve+ffn {layer_us:.1f} us, ffn {ffn_us:.1f} us for "
        f"{uniq:.1f} + 1 experts -> {gbs:.0f} GB/s")
    return {"workload": "decode_layer", "tokens": T, "reps": reps, "route_resolve_ffn_us": round(layer_us, 2),
            "ffn_us": round(ffn_us, 2),
            "ffn_us_median_min_max": [round(float(np.median(ffn_t)), 2), round(min(ffn_t), 2), round(max(ffn_t), 2)],
            "distinct_experts": round(uniq, 2), "ffn_hbm_gbs": round(gbs, 1),
            "ffn_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_lru(seed, d, f, E, k, L, routers, biases, shared_pool, warmup, steps):
    """The 48-layer stack at T = 1 through an LRU cache of 8,445 slots; all
    24,576 blobs in pinned host memory, misses copied on the library's side
    stream.  Cold start: the cache begins empty."""
    import numpy as np
    import torch

    import moe_synth
    from moe_synth.harness import fill_pool
    from quantized_expert_ffn_softmax_amd import binding as B
    from quantized_expert_ffn_softmax_amd.runtime import MoeContext
    wl = moe_synth.WORKLOADS["decode_stack_lru"]
    T, S = wl["n_tokens"], wl["n_slots"]
    t0 = time.time()
    stride = B.moe_expert_bytes(d, f)
    log(f"[bench] lru: pinning {L * E} blobs ({L * E * stride / 1e9:.1f} GB) in host memory, {S} slots in HBM")
    host = torch.empty((L * E, stride), dtype=torch.uint8, pin_memory=True)
    for l0 in range(0, L, 8):
        fill_pool(host[l0 * E:(l0 + 8) * E], list(range(l0 * E, (l0 + 8) * E)), seed, d, f, E, chunk=512)
    slot_pool = torch.empty((S, stride), dtype=torch.uint8, device="cuda")
    ctx = MoeContext(d, f, E, k, L, S, T, host_store=host, slot_pool=slot_pool, shared_pool=shared_pool)
    c = ctx.ctx
    buf = ctx.buffers(T)
    xa = torch.empty((T, d), dtype=torch.float32, device="cuda")
    xb = torch.empty_like(xa)
    # pinned H2D peak for reference: 256 MiB, host -> device
    hsrc = host[:(1 << 28) // stride].reshape(-1)
    dst = torch.empty(hsrc.numel(), dtype=torch.uint8, device="cuda")
    dst.copy_(hsrc, non_blocking=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        dst.copy_(hsrc, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    h2d_peak = 3 * hsrc.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
    del dst
    log(f"[bench] lru: setup {time.time() - t0:.0f}s; pinned H2D peak {h2d_peak:.1f} GB/s")

    # the miss path's link rate through the library's own calls: from an empty
    # cache, moe_cache_resolve_async calls whose ids all miss (1 or 10 distinct
    # experts of a layer, never seen before), timed with events; bytes = the
    # blobs the fill kernel copies, time = the call (resolve + fill kernels)
    def fill_rate(n_miss, reps=8):
        B.moe_cache_reset(c)
        torch.cuda.synchronize()
        ids = torch.empty((reps, 1, k), dtype=torch.int32, device="cuda")
        for r in range(reps):
            row = [(r * n_miss + j) % E for j in range(n_miss)]
            row += [row[-1]] * (k - n_miss)  # repeats of the last id: n_miss distinct
            ids[r, 0] = torch.tensor(row, dtype=torch.int32)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        st0 = B.moe_get_stats(c)
        for r in range(reps):
            ev[r][0].record()
            B.moe_cache_resolve_async(c, 1 + r % (L - 1), ids[r], 1, buf["slot"])
            ev[r][1].record()
        torch.cuda.synchronize()
        st1 = B.moe_get_stats(c)
        assert st1["misses"] - st0["misses"] == reps * n_miss
        us = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev])) * 1e3
        return {"misses_per_call": n_miss, "call_us": round(us, 1),
                "gbs": round(n_miss * stride / (us * 1e-6) / 1e9, 2)}

    fill_link = [fill_rate(1), fill_rate(10)]
    log(f"[bench] lru: miss fill through moe_cache_resolve_async: " +
        ", ".join(f"{r['misses_per_call']} blob(s) in {r['call_us']} us = {r['gbs']} GB/s" for r in fill_link))

    def step(x0, zero_copy, bl=biases, layer_call=False):
        x = x0
        for l in range(L):
            if layer_call:  # moe_decode_layer: the FFN kernels stream the misses and fill their slots
                xn = xa if (l % 2 == 0) else xb
                B.moe_decode_layer(c, l, x, T, routers[l], bl[l], None, buf["idx"], buf["w"], buf["y_pairs"],
                                   buf["y_shared"], buf["out"], xn)
                x = xn
                continue
            B.moe_route(c, l, x, T, routers[l], bl[l], None, buf["idx"], buf["w"])
            if zero_copy:
                B.moe_cache_resolve_async(c, l, buf["idx"], T, buf["slot"])
            else:
                B.moe_cache_resolve(c, l, buf["idx"], T, buf["slot"])
            B.moe_expert_ffn(c, l, x, T, buf["idx"], buf["slot"], buf["y_pairs"], buf["y_shared"],
                             B.MOE_PATH_DECODE)
            xn = xa if (l % 2 == 0) else xb
            B.moe_combine_norm(c, buf["y_pairs"], buf["w"], buf["y_shared"], T, buf["out"], xn)
            x = xn

    xs = [torch.from_numpy(moe_synth.gen_x(seed, 300000 + s, T, d)).cuda() for s in range(warmup + steps)]

    def run(mode, bl=biases, n_steps=steps):
        """Cold start (cache reset), warm-up steps, then the timed steps.
        'copy': moe_cache_resolve -- the host reads each layer's miss list back
        and copies the missed blobs with hipMemcpyAsync.  'zero_copy_graph':
        moe_cache_resolve_async (a fill kernel reads the pinned host store) and
        the 48-layer step captured once in a HIP graph and replayed."""
        B.moe_cache_reset(c)
        torch.cuda.synchronize()
        if mode in ("zero_copy_graph", "layer_graph"):
            x_static = torch.empty((T, d), dtype=torch.float32, device="cuda")
            graph = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.graph(graph, stream=cs):
                step(x_static, True, bl, layer_call=(mode == "layer_graph"))
            torch.cuda.synchronize()

            def one(x0):
                x_static.copy_(x0)
                graph.replay()
        else:
            def one(x0):
                step(x0, False, bl)
        st0 = B.moe_get_stats(c)
        for s_ in range(warmup):
            one(xs[s_])
        torch.cuda.synchronize()
        st1 = B.moe_get_stats(c)
        t1 = time.time()
        for s_ in range(n_steps):
            one(xs[warmup + s_])
        torch.cuda.synchronize()
        wall = time.time() - t1
        st2 = B.moe_get_stats(c)
        return wall, st0, st1, st2

    runs = {m: run(m) for m in ("copy", "zero_copy_graph", "layer_graph")}
    wall, st0, st1, st2 = runs["layer_graph"]
    same = all(runs[m][i][key] == runs["layer_graph"][i][key] for m in ("copy", "zero_copy_graph")
               for i in (1, 2, 3) for key in ("lookups", "hits", "misses"))
    cold = (st1["hits"] - st0["hits"]) / max(1, st1["lookups"] - st0["lookups"])
    lookups, hits = st2["lookups"] - st1["lookups"], st2["hits"] - st1["hits"]
    h2d = st2["bytes_h2d"] - st1["bytes_h2d"]
    hit_bytes = (lookups + L * steps) * algo_blob_bytes(d, f)
    cw, fw = runs["copy"][0], runs["zero_copy_graph"][0]
    out = {"workload": "decode_stack_lru", "tokens_per_step": T, "layers": L, "slots": S, "steps": steps,
           "warmup": warmup,
           "miss_path": "moe_decode_layer: the FFN kernels stream missed experts from pinned host memory and fill "
                        "their slots (no fill kernel), 48-layer step in a HIP graph",
           "tok_per_s": round(T * steps / wall, 2), "ms_per_step": round(wall / steps * 1e3, 3),
           "hit_rate": round(hits / max(1, lookups), 4), "cold_start_hit_rate": round(cold, 4),
           "misses_per_token": round((lookups - hits) / (T * steps), 2),
           "h2d_gbs": round(h2d / wall / 1e9, 2), "h2d_peak_gbs": round(h2d_peak, 2),
           "hit_path_hbm_gbs": round(hit_bytes / wall / 1e9, 1),
           "fill_kernel_path": {"miss_path": "separate calls, moe_cache_resolve_async (a fill kernel copies each "
                                             "missed blob before the FFN), HIP graph",
                                "tok_per_s": round(T * steps / fw, 2), "ms_per_step": round(fw / steps * 1e3, 3),
                                "h2d_gbs": round(h2d / fw / 1e9, 2)},
           "copy_path": {"miss_path": "host reads the miss list, hipMemcpyAsync per missed blob",
                         "tok_per_s": round(T * steps / cw, 2), "ms_per_step": round(cw / steps * 1e3, 3),
                         "h2d_gbs": round(h2d / cw / 1e9, 2)},
           "same_hits_and_misses": same,
           "timing": "host wall clock over the timed steps"}
    out["fill_link"] = fill_link
    # tok/s against hit rate: the same cache and steps under other Zipf skews
    # of the router bias (the pages' hit rates, 94-99%, sit in this range)
    sweep = []
    for alpha in (0.5, 1.0):
        bl = [torch.from_numpy(moe_synth.gen_bias(seed, l, E, alpha)).cuda() for l in range(L)]
        n_sw = max(1, steps // 2)
        w_, _s0, s1_, s2_ = run("layer_graph", bl, n_sw)
        lk, ht = s2_["lookups"] - s1_["lookups"], s2_["hits"] - s1_["hits"]
        sweep.append({"zipf_alpha": alpha, "hit_rate": round(ht / max(1, lk), 4),
                      "misses_per_token": round((lk - ht) / (T * n_sw), 2), "tok_per_s": round(T * n_sw / w_, 2),
                      "ms_per_step": round(w_ / n_sw * 1e3, 3),
                      "h2d_gbs": round((s2_["bytes_h2d"] - s1_["bytes_h2d"]) / w_ / 1e9, 2)})
    sweep.insert(1, {"zipf_alpha": 0.75, "hit_rate": out["hit_rate"], "misses_per_token": out["misses_per_token"],
                     "tok_per_s": out["tok_per_s"], "ms_per_step": out["ms_per_step"], "h2d_gbs": out["h2d_gbs"]})
    out["hit_rate_sweep"] = sweep
    log("[bench] lru: tok/s against hit rate: " +
        ", ".join(f"alpha {r['zipf_alpha']}: hit {r['hit_rate']:.4f} -> {r['tok_per_s']} tok/s" for r in sweep))
    log(f"[bench] lru: moe_decode_layer+graph {out['tok_per_s']} tok/s ({out['ms_per_step']} ms/step), fill kernel "
        f"{out['fill_kernel_path']['tok_per_s']} tok/s, copy path "
        f"{out['copy_path']['tok_per_s']} tok/s; hit rate {out['hit_rate']:.4f} (cold start {cold:.4f}), "
        f"{out['misses_per_token']} misses/token, H2D {out['h2d_gbs']} GB/s (peak {h2d_peak:.1f}); "
        f"identical cache traffic in all three modes: {same}")
    ctx.close()
    del host, slot_pool
    return out


def bench_kv(seed, peaks, reps=5):
    """The KV tier at the pages' shape: one layer of 131,072 int8 cells of
    1,024 values, the first 32,768 resident in HBM, the rest in pinned host
    memory.  A whole-context read (what a prefill chunk's attention takes) in
    4,096-cell chunks: without prefetch (host cells read over the link by the
    read kernel) and with prefetch (the next host chunk DMA-copied into a
    staging slot on a side stream while the current chunk is read).  Also
    the read kernel alone on resident chunks against the HBM roofline, and the
    write (quantise) rate."""
    import numpy as np
    import torch

    import moe_synth
    from quantized_expert_ffn_softmax_amd import binding as B
    from quantized_expert_ffn_softmax_amd.runtime import KvTier
    wl = moe_synth.WORKLOADS["kv_tier"]
    total, R, V, blk, ch = wl["cells_total"], wl["cells_resident"], wl["values"], wl["block_cells"], wl["chunk_cells"]
    big = 4 * ch  # the sweep is also run in chunks this size (larger DMA copies)
    t = KvTier(1, total, R, V, blk, big)
    kv, cb = t.kv, t.cb
    src = torch.empty((ch, V), dtype=torch.float32, device="cuda")
    wev = []
    for first in range(0, total, ch):
        src.copy_(torch.from_numpy(moe_synth.gen_kv(seed, 0, first, ch, V)))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.moe_kv_write(kv, 0, first, ch, src)
        b.record()
        wev.append((first, a, b))
    torch.cuda.synchronize()
    w_res = float(np.median([a.elapsed_time(b) for f_, a, b in wev if f_ < R]))
    w_host = float(np.median([a.elapsed_time(b) for f_, a, b in wev if f_ >= R]))
    out = torch.empty((big, V), dtype=torch.float32, device="cuda")
    # reads and prefetches on two streams of their own (the default stream
    # would serialise with the side stream)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    main.wait_stream(torch.cuda.current_stream())

    def context_read(prefetch, ch):
        chunks = list(range(0, total, ch))
        ev_read = {}
        ev_pref = {}
        if prefetch:
            side.wait_stream(main)
            first_host = [c for c in chunks if c >= R]
            with torch.cuda.stream(side):
                for c in first_host[:1]:
                    B.moe_kv_prefetch(kv, 0, c, ch, side)
                    ev_pref[c] = torch.cuda.Event()
                    ev_pref[c].record(side)
        for i, c in enumerate(chunks):
            if prefetch and c in ev_pref:
                main.wait_event(ev_pref[c])
            B.moe_kv_read(kv, 0, c, ch, out, main)
            ev_read[c] = torch.cuda.Event()
            ev_read[c].record(main)
            nxt = c + ch
            if prefetch and nxt < total and nxt >= R and nxt not in ev_pref:
                # the slot it takes held the chunk read two steps ago
                prev = c - ch
                if prev in ev_read:
                    side.wait_event(ev_read[prev])
                B.moe_kv_prefetch(kv, 0, nxt, ch, side)
                ev_pref[nxt] = torch.cuda.Event()
                ev_pref[nxt].record(side)

    res = {}
    # (the runs without prefetch first: a staging slot keeps its copy until a
    # later prefetch replaces it, and reads use it)
    for mode, csz in (("no_prefetch", ch), ("no_prefetch_16k", big), ("prefetch", ch), ("prefetch_16k", big)):
        st0 = B.moe_kv_get_stats(kv)
        context_read(mode.startswith("prefetch"), csz)  # warm-up
        torch.cuda.synchronize()
        st1 = B.moe_kv_get_stats(kv)
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(main)
            context_read(mode.startswith("prefetch"), csz)
            b.record(main)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        st2 = B.moe_kv_get_stats(kv)
        blocks = st2["block_reads"] - st1["block_reads"]
        m = float(np.median(ms))
        res[mode] = {"chunk_cells": csz, "ms_per_context_read": round(m, 3), "cells_per_s": round(total / (m * 1e-3), 0),
                     "cell_gbs": round(total * cb / (m * 1e-3) / 1e9, 1),
                     "vram_block_read_rate": round((st2["vram_block_reads"] - st1["vram_block_reads"]) / blocks, 4),
                     "host_gbs": round((st2["host_bytes"] - st1["host_bytes"]) / reps / (m * 1e-3) / 1e9, 2),
                     "prefetch_gbs": round((st2["prefetch_bytes"] - st1["prefetch_bytes"]) / reps / (m * 1e-3) / 1e9,
                                           2)}
        del st0
    # the read kernel alone on resident chunks: HBM-bound, 1,056 B in + 4,096 B out per cell
    ev = []
    torch.cuda.synchronize()
    for r in range(reps * 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(main)
        B.moe_kv_read(kv, 0, (r % (R // ch)) * ch, ch, out, main)
        b.record(main)
        ev.append((a, b))
    torch.cuda.synchronize()
    rd = _median_ms(ev)
    per_cell = cb + 4 * V
    achieved = ch * per_cell / (rd * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": "kv_read_kernel (resident cells)", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": ch * per_cell, "avg_launch_us": round(rd * 1e3, 2)}
    if peaks is not None:
        roof["measured_peak"] = peaks["hbm_read_gbs"]
        roof["frac_of_measured"] = round(achieved / peaks["hbm_read_gbs"], 4)
    out_d = {"workload": "kv_tier", "cells_total": total, "cells_resident": R, "values_per_cell": V,
             "cell_bytes": cb, "block_cells": blk, "chunk_cells": ch, "stage_cells": big,
             "write_us_per_chunk": {"resident": round(w_res * 1e3, 1), "host": round(w_host * 1e3, 1)},
             "write_host_gbs": round(ch * cb / (w_host * 1e-3) / 1e9, 2),
             "context_read": res, "roofline": roof,
             "timing": "HIP events on the read stream around each whole-context read (median of reps)"}
    log("[bench] kv: context read " + ", ".join(
        f"{k_}: {r_['ms_per_context_read']} ms ({r_['vram_block_read_rate']:.3f} of block reads from HBM)"
        for k_, r_ in res.items()) + f"; resident read kernel {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.3f} of HBM peak)")
    t.close()
    return out_d


def verify_sweep(ctx, routers, biases, seed, d, f, L, reps=5, warm=2):
    """Speculative verify as a batch: `slots` requests each verify 1 + `spec`
    tokens in one pass, T = slots * (1 + spec) tokens per step, for spec 1..6
    and slots 1..4.  Each T: the 48-layer resident stack of moe_decode_layer
    captured in a HIP graph, replayed on fresh inputs; reports tok/s and the
    expert bytes each token costs (touched routed experts + the shared one,
    per layer)."""
    import numpy as np
    import torch

    import moe_synth
    from quantized_expert_ffn_softmax_amd import binding as B
    c, k = ctx.ctx, ctx.k
    blob = algo_blob_bytes(d, f)
    rows = []
    for slots in range(1, 5):
        for spec in range(1, 7):
            T = slots * (1 + spec)
            buf = ctx.buffers(T)
            xin = torch.empty((T, d), dtype=torch.float32, device="cuda")
            xa, xb = torch.empty_like(xin), torch.empty_like(xin)

            def step():
                x = xin
                for l in range(L):
                    xn = xa if (l % 2 == 0) else xb
                    B.moe_decode_layer(c, l, x, T, routers[l], biases[l], None, buf["idx"], buf["w"],
                                       buf["y_pairs"], buf["y_shared"], buf["out"], xn)
                    x = xn

            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.graph(graph, stream=cs):
                step()
            torch.cuda.synchronize()
            xs = [torch.from_numpy(moe_synth.gen_x(seed, 500000 + 100 * T + i, T, d)).cuda() for i in range(warm + reps)]
            for i in range(warm):
                xin.copy_(xs[i])
                graph.replay()
            torch.cuda.synchronize()
            st0 = B.moe_get_stats(c)
            ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(reps)]
            for i in range(reps):
                xin.copy_(xs[warm + i])
                ev[i][0].record()
                graph.replay()
                ev[i][1].record()
            torch.cuda.synchronize()
            st1 = B.moe_get_stats(c)
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            distinct = (st1["lookups"] - st0["lookups"]) / (st1["resolve_calls"] - st0["resolve_calls"])
            rows.append({"slots": slots, "spec": spec, "T": T, "tok_per_s": round(T / (ms * 1e-3), 1),
                         "ms_per_step": round(ms, 3), "distinct_experts_per_layer": round(distinct, 2),
                         "expert_mb_per_token": round((distinct + 1) * blob * L / T / 1e6, 1)})
            del graph
    log("[bench] verify sweep: " + ", ".join(f"T={r['T']}: {r['tok_per_s']:.0f} tok/s "
                                             f"{r['expert_mb_per_token']} MB/tok" for r in rows))
    return {"workload": "verify_sweep", "layers": L, "reps": reps, "rows": rows}


def cpu_baseline(seed, d, f, E, k, T, alpha, n_layers, step, prefill_T, prefill_experts=24):
    """The oracle, as it stands, on bounded samples of two workloads:
    the first `n_layers` layers of one decode step of the stack (scaled to the
    48 layers), and the prefill chunk with its router on every token and the
    expert FFNs of a seeded sample of the experts that receive tokens (scaled
    by the number of such experts)."""
    import numpy as np

    import moe_synth
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    L = moe_synth.WORKLOADS["batched_decode_stack"]["n_layers"]
    x = moe_synth.gen_x(seed, step, T, d)
    spent = 0.0
    for l in range(n_layers):
        wr = moe_synth.gen_router(seed, l, E, d)
        bias = moe_synth.gen_bias(seed, l, E, alpha)
        _, idx, _ = oracle.route(x, wr, bias, k)
        blobs = {int(e): moe_synth.gen_blob(seed, l, int(e), d, f) for e in np.unique(idx)}
        shared = moe_synth.gen_blob(seed, l, E, d, f)
        t = time.time()
        r = oracle.moe_layer(x, wr, bias, k, lambda e: blobs[e], shared, d, f, precision="exact")
        spent += time.time() - t
        x = oracle.chain_norm(r["out64"])
        log(f"[bench] cpu oracle decode layer {l}: {spent:.1f}s so far")
    per_layer = spent / n_layers
    out = {"value": round(T / (per_layer * L), 3), "unit": "tok/s", "cores": cores, "blas_threads": blas_threads,
           "kind": "oracle",
           "sample": f"{n_layers} of {L} layers of one {T}-token decode step (float64 numpy oracle, exact "
                     f"precision), scaled to the 48-layer stack; {per_layer:.2f} s per layer"}
    # prefill chunk: route every token, then the FFNs of a sample of experts
    xp = moe_synth.gen_x(seed, 100000, prefill_T, d)
    wr = moe_synth.gen_router(seed, 0, E, d)
    bias = moe_synth.gen_bias(seed, 0, E, alpha)
    t = time.time()
    _, idx, w = oracle.route(xp, wr, bias, k)
    t_route = time.time() - t
    flat = idx.reshape(-1)
    used = np.unique(flat)
    rng = np.random.default_rng(seed)
    pick = rng.choice(used, size=min(prefill_experts, used.size), replace=False)
    t_ffn, rows = 0.0, 0
    for e in pick:
        blob = moe_synth.gen_blob(seed, 0, int(e), d, f)
        pairs = np.nonzero(flat == e)[0]
        t = time.time()
        oracle.expert_ffn(xp[pairs // k], oracle.expert_weights(blob, d, f), "exact")
        t_ffn += time.time() - t
        rows += pairs.size
    shared = moe_synth.gen_blob(seed, 0, E, d, f)
    t = time.time()
    oracle.expert_ffn(xp, oracle.expert_weights(shared, d, f), "exact")
    t_shared = time.time() - t
    est = t_route + t_ffn * used.size / pick.size + t_shared
    out["prefill"] = {"value": round(prefill_T / est, 2), "unit": "tok/s", "cores": cores, "kind": "oracle",
                      "sample": f"prefill chunk of {prefill_T} tokens: router and top-k on every token "
                                f"({t_route:.1f} s), shared expert on every token ({t_shared:.1f} s), expert FFNs "
                                f"of {pick.size} of the {used.size} experts with tokens (seeded pick, {rows} pairs, "
                                f"{t_ffn:.1f} s) scaled by {used.size}/{pick.size}; estimated {est:.1f} s per chunk"}
    # the two small configurations, each timed whole: the tiny layer (T = 8,
    # 16 experts of 256 x 128) and one real layer at T = 5 (no router bias)
    for name in ("tiny", "decode_layer"):
        wl = moe_synth.WORKLOADS[name]
        dd, ff, EE, kk, TT = wl["d_model"], wl["d_ff"], wl["n_experts"], wl["top_k"], wl["n_tokens"]
        xw = moe_synth.gen_x(seed, 200000, TT, dd)
        wrw = moe_synth.gen_router(seed, 0, EE, dd)
        bw = moe_synth.gen_bias(seed, 0, EE, wl["alpha"])
        _, idw, _ = oracle.route(xw, wrw, bw, kk)
        blobs_w = {int(e): moe_synth.gen_blob(seed, 0, int(e), dd, ff) for e in np.unique(idw)}
        shared_w = moe_synth.gen_blob(seed, 0, EE, dd, ff)
        t = time.time()
        oracle.moe_layer(xw, wrw, bw, kk, lambda e: blobs_w[e], shared_w, dd, ff, precision="exact")
        tw = time.time() - t
        out[name] = {"value": round(TT / tw, 3), "unit": "tok/s", "cores": cores, "kind": "oracle",
                     "sample": f"the whole layer: {TT} tokens, {EE} experts of {dd} x {ff}, top-{kk} "
                               f"(route, {len(blobs_w)} + 1 expert FFNs, combine), {tw:.2f} s"}
    log(f"[bench] cpu oracle: decode {out['value']} tok/s, prefill {out['prefill']['value']} tok/s, tiny layer "
        f"{out['tiny']['value']} tok/s, one real layer at T=5 {out['decode_layer']['value']} tok/s on {cores} cores")
    return out


if __name__ == "__main__":
    main()
