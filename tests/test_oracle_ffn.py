"""Pins for the oracle's expert FFN, combine and whole layer (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import moe_synth
import oracle
from test_oracle_format import _make_blob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blob_from_codes(d, f, rng, code_fn=None, scale=None):
    shapes = [(f, d), (f, d), (d, f)]
    codes = [rng.integers(0, 8, s) if code_fn is None else code_fn(s) for s in shapes]
    scales = []
    for (r, c) in shapes:
        if scale is None:
            scales.append(rng.uniform(0.01, 0.05, (r, c // 32)).astype(np.float16))
        else:
            scales.append(np.full((r, c // 32), scale, dtype=np.float16))
    return _make_blob(d, f, codes, scales), codes, scales


def _py_ffn(x, codes, scales):
    # explicit loops over Python floats: y = Wd (silu(Wg x) * (Wu x))
    (qg, qu, qd), (sg, su, sd) = codes, scales
    f, d = qg.shape

    def w(q, s, r, c):
        return (int(q[r, c]) - 4) * float(s[r, c // 32])

    h = []
    for r in range(f):
        g = sum(w(qg, sg, r, c) * float(x[c]) for c in range(d))
        u = sum(w(qu, su, r, c) * float(x[c]) for c in range(d))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [sum(w(qd, sd, r, c) * h[c] for c in range(f)) for r in range(d)]


def test_ffn_brute_force_tiny():
    d, f = 64, 32
    rng = np.random.default_rng(11)
    blob, codes, scales = _blob_from_codes(d, f, rng)
    x = rng.standard_normal((3, d)).astype(np.float32)
    y = oracle.expert_ffn(x, oracle.expert_weights(blob, d, f))
    for t in range(3):
        ref = _py_ffn(x[t], codes, scales)
        assert np.allclose(y[t], ref, rtol=1e-11, atol=1e-13)


def test_all_codes_four_gives_zero():
    d, f = 64, 64
    rng = np.random.default_rng(12)
    blob, _, _ = _blob_from_codes(d, f, rng, code_fn=lambda s: np.full(s, 4))
    x = rng.standard_normal((4, d)).astype(np.float32)
    for prec in ("exact", "fp16_weights"):
        y = oracle.expert_ffn(x, oracle.expert_weights(blob, d, f, prec != "exact"), prec)
        assert np.all(y == 0.0)


def test_down_scale_doubling_doubles_output():
    d, f = 96, 64
    rng = np.random.default_rng(13)
    shapes = [(f, d), (f, d), (d, f)]
    codes = [rng.integers(0, 8, s) for s in shapes]
    scales = [rng.uniform(0.01, 0.05, (r, c // 32)).astype(np.float16) for r, c in shapes]
    b1 = _make_blob(d, f, codes, scales)
    b2 = _make_blob(d, f, codes, scales[:2] + [(scales[2].astype(np.float32) * 2).astype(np.float16)])
    x = rng.standard_normal((5, d)).astype(np.float32)
    y1 = oracle.expert_ffn(x, oracle.expert_weights(b1, d, f))
    y2 = oracle.expert_ffn(x, oracle.expert_weights(b2, d, f))
    assert np.array_equal(y2, 2 * y1)


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert math.isclose(s[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(s[2], -1 / (1 + math.e), rel_tol=1e-15)
    assert math.isclose(s[3], 40.0, rel_tol=1e-15)
    assert abs(s[4]) < 1e-15


def test_fp16_modes_equal_exact_when_operands_representable():
    # power-of-two scales: every (q-4)*s is exact in fp16; fp16-valued x
    d, f = 64, 32
    rng = np.random.default_rng(14)
    blob, _, _ = _blob_from_codes(d, f, rng, scale=0.03125)
    x = rng.standard_normal((2, d)).astype(np.float16).astype(np.float32)
    ex = oracle.expert_ffn(x, oracle.expert_weights(blob, d, f), "exact")
    fw = oracle.expert_ffn(x, oracle.expert_weights(blob, d, f, True), "fp16_weights")
    assert np.array_equal(ex, fw)


def _layer_inputs(d, f, E, T, seed=0):
    rng = np.random.default_rng(seed)
    blobs = [moe_synth.gen_blob(seed, 0, e, d, f) for e in range(E)]
    shared = moe_synth.gen_blob(seed, 0, E, d, f)
    wr = moe_synth.gen_router(seed, 0, E, d) * 8  # spread the logits
    x = rng.standard_normal((T, d)).astype(np.float32)
    return blobs, shared, wr, x


def test_k_equals_E_dense_equivalence():
    d, f, E, T = 64, 32, 6, 4
    blobs, shared, wr, x = _layer_inputs(d, f, E, T)
    r = oracle.moe_layer(x, wr, None, E, lambda e: blobs[e], shared, d, f)
    lg = x.astype(np.float64) @ wr.astype(np.float64).T
    p = softmax(lg, axis=1)
    dense = oracle.expert_ffn(x, oracle.expert_weights(shared, d, f))
    for e in range(E):
        dense = dense + p[:, e:e + 1] * oracle.expert_ffn(x, oracle.expert_weights(blobs[e], d, f))
    assert np.allclose(r["out64"], dense, rtol=1e-12, atol=1e-12)


def test_k1_is_shared_plus_argmax_expert():
    d, f, E, T = 64, 32, 8, 5
    blobs, shared, wr, x = _layer_inputs(d, f, E, T, seed=1)
    r = oracle.moe_layer(x, wr, None, 1, lambda e: blobs[e], shared, d, f)
    lg = x.astype(np.float64) @ wr.astype(np.float64).T
    for t in range(T):
        e = int(np.argmax(lg[t]))
        ref = oracle.expert_ffn(x[t:t + 1], oracle.expert_weights(shared, d, f))[0] + \
            oracle.expert_ffn(x[t:t + 1], oracle.expert_weights(blobs[e], d, f))[0]
        assert np.allclose(r["out64"][t], ref, rtol=1e-13, atol=1e-13)


def test_combine_order_and_definition():
    rng = np.random.default_rng(3)
    T, k, d = 3, 4, 5
    yp = rng.standard_normal((T * k, d))
    w = rng.dirichlet(np.ones(k), T)
    ys = rng.standard_normal((T, d))
    out = oracle.combine(yp, w, ys)
    for t in range(T):
        for c in range(d):
            acc = 0.0
            for j in range(k):
                acc += w[t, j] * yp[t * k + j, c]
            assert out[t, c] == acc + ys[t, c]


def test_teacher_forced_routing_reuses_given_idx():
    d, f, E, T = 64, 32, 8, 3
    blobs, shared, wr, x = _layer_inputs(d, f, E, T, seed=2)
    free = oracle.moe_layer(x, wr, None, 2, lambda e: blobs[e], shared, d, f)
    forced = oracle.moe_layer(x, wr, None, 2, lambda e: blobs[e], shared, d, f, idx=free["idx"])
    assert np.array_equal(free["out64"], forced["out64"])


def test_chain_norm():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((3, 64)) * 20 + 7.0
    xn = oracle.chain_norm(o).astype(np.float64)
    assert np.allclose(xn.mean(axis=1), 0.0, atol=1e-6)
    assert np.allclose(np.sqrt(np.mean(xn ** 2, axis=1)), 1.0, rtol=1e-6)
    # a constant row maps to zero; a shift of the row does not change the result
    assert np.all(oracle.chain_norm(np.full((1, 8), 3.0)) == 0.0)
    assert np.allclose(oracle.chain_norm(o + 5.0), xn, atol=1e-6)


def test_page_constants():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    L = g["layers"]["value"]
    E = g["routed_experts_per_layer"]["value"]
    assert L * E == g["identities"]["value"]
    wl = moe_synth.WORKLOADS
    assert wl["decode_layer"]["n_experts"] == E and wl["decode_layer"]["top_k"] == g["top_k"]["value"]
    assert wl["batched_decode_stack"]["n_layers"] == L
    assert wl["decode_stack_lru"]["n_slots"] == g["slots_headline"]["value"]
    assert g["slots_per_card_4gpu"]["value"] * g["slots_per_card_4gpu"]["cards"] == g["identities"]["value"]
    # hit rate = hits / lookups, as the engine prints it
    for hits, lookups, pct in g["hit_counts"]["value"]:
        c = oracle.LRUCache(1, 1, 1)
        c.hits, c.lookups = hits, lookups
        assert round(100 * c.hits / c.lookups, 1) == pct
    n, tot, pct = g["coverage"]["value"]
    assert abs(100 * n / tot - pct) < 0.1  # the page prints 48.0 for 47.95
    es = g["expert_size"]
    assert round(es["gib_total"] * 1024 / es["slots"], 2) == es["mib_each"]
    # the stand-in shape at IQ3_S's bit rate lands within 2% of the printed size
    weights = 3 * 2048 * 768
    mib = weights * g["iq3_s_bits"]["value"] / 8 / 2 ** 20
    assert abs(mib - es["mib_each"]) / es["mib_each"] < 0.02
