"""Seeded synthetic inputs for the routed MoE layer.

This module is the one piece shared by the HIP path's tests/bench and by the
CPU oracle.  It draws random bytes and numbers and places them where the expert
blob layout says they go; it implements none of the layer's arithmetic (no
unpacking, dequantisation, routing, caching or FFN math).

Shapes follow the engine described on the pages ("一张 RTX 4090 跑千亿模型，
Strata 实测 155 tok/s", section 如何做到：三层存储): 512 routed experts per layer,
top-10 plus one shared expert, 48 layers, 24,576 (layer, expert) identities.
The pages never give the weight values or the quantised layout, so everything
here is synthetic:

* every stream is a NumPy PCG64 generator keyed by
  ``SeedSequence([seed, tag, layer, expert])`` so that any blob can be redrawn
  on its own, in any order, on any machine;
* expert codes are uniform on {0..7}: each 15-bit half word is drawn uniformly
  (which is the same as ten iid uniform 3-bit codes per word) and code slots
  past the row end and pad words are zero;
* block scales are ``float16(U[0.01, 0.05])`` (NumPy's round-to-nearest-even);
* router weights ``N(0, 0.02)`` as float32, activations ``N(0, 1)`` float32;
* the Zipf-skew router bias is ``-alpha * 1.1 * ln(rank)`` with ``rank`` a
  seeded permutation of 1..E per layer (zero when ``alpha == 0``);
* the shared expert of a layer is drawn as expert index ``E``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

TAG_BLOB = 1
TAG_ROUTER = 2
TAG_BIAS = 3
TAG_X = 4
TAG_KV = 5

BLOB_ALIGN = 256


def _rng(seed: int, tag: int, layer: int, expert: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag), int(layer), int(expert)])))


def _words_per_row(cols: int) -> int:
    w = -(-cols // 10)
    return -(-w // 4) * 4


def _slot_shift(j: int) -> int:
    return 3 * j if j < 5 else 16 + 3 * (j - 5)


def _row_mask(cols: int) -> np.ndarray:
    """Per-word mask of the bits that carry a code inside one row."""
    wpr = _words_per_row(cols)
    mask = np.zeros(wpr, dtype=np.uint32)
    for w in range(wpr):
        m = 0
        for j in range(10):
            if 10 * w + j < cols:
                m |= 7 << _slot_shift(j)
        mask[w] = m
    return mask


def _matrices(d_model: int, d_ff: int):
    # (rows, cols) of gate, up, down, in blob order
    return ((d_ff, d_model), (d_ff, d_model), (d_model, d_ff))


def blob_stride(d_model: int, d_ff: int) -> int:
    """Bytes between consecutive blobs (the layout's size rounded up to 256)."""
    total = 0
    for rows, cols in _matrices(d_model, d_ff):
        total += rows * _words_per_row(cols) * 4 + rows * (cols // 32) * 2
    return -(-total // BLOB_ALIGN) * BLOB_ALIGN


_MASK_CACHE: dict = {}


def fill_blob(out: np.ndarray, seed: int, layer: int, expert: int, d_model: int, d_ff: int) -> None:
    """Write one expert blob (gate, up, down) into the uint8 array ``out``."""
    if d_model % 32 or d_ff % 32:
        raise ValueError("d_model and d_ff must be multiples of 32")
    rng = _rng(seed, TAG_BLOB, layer, expert)
    pos = 0
    out[:] = 0
    for rows, cols in _matrices(d_model, d_ff):
        wpr = _words_per_row(cols)
        key = cols
        if key not in _MASK_CACHE:
            _MASK_CACHE[key] = _row_mask(cols)
        mask = _MASK_CACHE[key]
        n = rows * wpr
        raw = rng.bit_generator.random_raw((n + 1) // 2).view(np.uint32)[:n].reshape(rows, wpr)
        np.bitwise_and(raw, mask[None, :], out=raw)
        out[pos:pos + 4 * n] = raw.reshape(-1).view(np.uint8)
        pos += 4 * n
        ns = rows * (cols // 32)
        sc = rng.uniform(0.01, 0.05, ns).astype(np.float16)
        out[pos:pos + 2 * ns] = sc.view(np.uint8)
        pos += 2 * ns


def gen_blob(seed: int, layer: int, expert: int, d_model: int, d_ff: int) -> np.ndarray:
    out = np.empty(blob_stride(d_model, d_ff), dtype=np.uint8)
    fill_blob(out, seed, layer, expert, d_model, d_ff)
    return out


def fill_blobs(out: np.ndarray, ids, seed: int, d_model: int, d_ff: int, n_experts: int,
               threads: int | None = None) -> None:
    """Fill ``out[i]`` with the blob of identity ``ids[i]`` (= layer * E + expert).

    ``out`` is a uint8 array of shape [len(ids)][stride]; shared experts are
    requested with expert index ``n_experts`` (pass identities as (layer, E)
    tuples for those).
    """
    stride = blob_stride(d_model, d_ff)
    if out.shape[-1] != stride:
        raise ValueError("row stride mismatch")

    def one(i):
        ident = ids[i]
        if isinstance(ident, tuple):
            layer, expert = ident
        else:
            layer, expert = divmod(int(ident), n_experts)
        fill_blob(out[i], seed, layer, expert, d_model, d_ff)

    n = len(ids)
    threads = threads or min(16, os.cpu_count() or 1)
    if n < 8 or threads == 1:
        for i in range(n):
            one(i)
        return
    with _cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(n), chunksize=max(1, n // (threads * 8))))


def gen_router(seed: int, layer: int, n_experts: int, d_model: int) -> np.ndarray:
    rng = _rng(seed, TAG_ROUTER, layer, 0)
    return (rng.standard_normal((n_experts, d_model)) * 0.02).astype(np.float32)


def gen_bias(seed: int, layer: int, n_experts: int, alpha: float) -> np.ndarray:
    if alpha == 0:
        return np.zeros(n_experts, dtype=np.float32)
    rng = _rng(seed, TAG_BIAS, layer, 0)
    rank = rng.permutation(n_experts) + 1
    return (-alpha * 1.1 * np.log(rank.astype(np.float64))).astype(np.float32)


def gen_x(seed: int, step: int, n_tokens: int, d_model: int) -> np.ndarray:
    rng = _rng(seed, TAG_X, step, 0)
    return rng.standard_normal((n_tokens, d_model)).astype(np.float32)


# ---------------------------------------------------------------------------
# Workloads.  Sizes are those of the pages' engine (48 layers x 512 experts,
# top-10 + 1 shared) at d_model=2048, d_ff=768, plus a tiny case for parity.
# ---------------------------------------------------------------------------
KV_BLOCK = 256  # cells drawn together (any split of a range gives the same values)


def gen_kv(seed: int, layer: int, first: int, n: int, values: int = 1024) -> np.ndarray:
    """KV cell values [n][values] float32 for cells first .. first + n - 1 of a
    layer: Gaussian rows times a per-channel scale that is log-normal over the
    channels (a few channels carry most of the magnitude, as attention keys
    do), the same channel scales for every cell of the layer.  Every 97th cell
    gets the special groups the quantiser has to get right: an all-zero group,
    a group far below fp16's normal range, a group of multiples of 0.125 whose
    largest is 31.75 (scale exactly 0.25: halves of the step are rounding
    ties), and one group 1e4 larger than the rest."""
    chan = np.exp(_rng(seed, TAG_KV, layer, 1 << 30).normal(0.0, 1.0, values)).astype(np.float32)
    out = np.empty((n, values), dtype=np.float32)
    b0, b1 = first // KV_BLOCK, (first + n - 1) // KV_BLOCK
    for b in range(b0, b1 + 1):
        rows = _rng(seed, TAG_KV, layer, b).standard_normal((KV_BLOCK, values)).astype(np.float32) * chan
        lo, hi = max(first, b * KV_BLOCK), min(first + n, (b + 1) * KV_BLOCK)
        out[lo - first:hi - first] = rows[lo - b * KV_BLOCK:hi - b * KV_BLOCK]
    for c in range(-(-first // 97) * 97, first + n, 97):
        v = out[c - first]
        r = _rng(seed, TAG_KV, layer, (1 << 30) + 1 + c)
        v[0:64] = 0.0
        v[64:128] *= np.float32(1e-9)
        v[128:192] = (np.round(r.uniform(-254.0, 254.0, 64)) / 8.0).astype(np.float32)
        v[128] = np.float32(31.75)
        v[192:256] *= np.float32(1e4)
    return out


WORKLOADS = {
    "tiny": dict(d_model=256, d_ff=128, n_experts=16, top_k=2, n_layers=1, n_tokens=8,
                 n_slots=None, alpha=0.0, steps=1),
    "decode_layer": dict(d_model=2048, d_ff=768, n_experts=512, top_k=10, n_layers=1, n_tokens=5,
                         n_slots=None, alpha=0.0, steps=1),
    "decode_stack_lru": dict(d_model=2048, d_ff=768, n_experts=512, top_k=10, n_layers=48, n_tokens=1,
                             n_slots=8445, alpha=0.75, steps=256),
    "prefill_chunk": dict(d_model=2048, d_ff=768, n_experts=512, top_k=10, n_layers=1, n_tokens=12288,
                          n_slots=None, alpha=0.75, steps=1),
    "batched_decode_stack": dict(d_model=2048, d_ff=768, n_experts=512, top_k=10, n_layers=48, n_tokens=15,
                                 n_slots=None, alpha=0.75, steps=64),
    # KV tier: 131,072 cells per layer, the first 32,768 resident, int8 cells
    # of 1,024 values (1,056 bytes); read in 4,096-cell chunks
    "kv_tier": dict(cells_total=131072, cells_resident=32768, values=1024, block_cells=256, chunk_cells=4096),
}
