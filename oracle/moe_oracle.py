"""CPU oracle for the routed MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it, and it
shares no code with ``quantized_expert_ffn_softmax_amd``: it has its own blob
layout, its own unpacking and its own arithmetic, all in float64 NumPy.

What the pages fix, and where:

* "一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s", section 如何做到：三层存储:
  each MoE layer has 512 routed experts, a token activates 10 of them plus
  one shared expert; (layer, expert) pairs give 24,576 identities of about
  1.7 MB; hits are computed from the VRAM hot cache, misses are fetched over
  PCIe from host RAM; the hot cache is a pool of slots (8,445 in the headline
  table, section 先看结果).
* "从一张到四张 RTX 4090 ...", section 先看结果: the model has 48 layers.
* "单卡5090跑125B 大模型 ...", section 7.2: the engine reports expert-cache hits
  over lookups (95.3% = 58,084 / 60,919).

The pages name the IQ3_XXS / IQ3_S quantisation but give neither its layout
nor the router's scoring function, the activation, the eviction policy or the
precision.  Every such step below is a stated reading (listed again in the
project's design notes):

* weights: 3-bit codes q, value (q - 4) * scale, ten codes per uint32 word in
  two 15-bit halves (code j < 5 at bit 3j, code j >= 5 at bit 16 + 3(j-5)),
  one fp16 scale per 32 consecutive inputs of a row; rows padded to a multiple
  of four words; gate [f][d], up [f][d], down [d][f], each codes then scales;
* router: logits = x W_r^T + b, top-k by (logit desc, index asc), weights =
  softmax over all experts renormalised over the k chosen (the full softmax
  denominator cancels, so it is the softmax of the k chosen logits);
* expert: y = W_d (silu(W_g x) * W_u x); the shared expert is ungated (weight 1)
  and is added after the k routed terms, taken in ascending j;
* cache: LRU with the tie rules documented on ``LRUCache``;
* precision: 'exact' is float64 on the exactly dequantised weights;
  'fp16_weights' models where both GPU paths round: every dequantised weight
  (q - 4) * s is rounded once to fp16 (round to nearest, ties to even), the
  activations x and h are kept at fp32 accuracy, and all arithmetic after the
  rounding is float64.  It is pinned on the CPU against hand-worked values
  (the fp16 rounding written out from its definition, sums in exact
  rationals), against the exact mode where every weight is representable, and
  against a tie case of the rounding in each direction.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Blob layout (reading: the stand-in for IQ3 named on the pages)
# ---------------------------------------------------------------------------

SCALE_BLOCK = 32
CODES_PER_WORD = 10
BLOB_ALIGN = 256


def words_per_row(cols: int) -> int:
    """Words in one row: ceil(cols / 10) rounded up to a multiple of 4."""
    w = (cols + CODES_PER_WORD - 1) // CODES_PER_WORD
    return (w + 3) // 4 * 4


def matrix_bytes(rows: int, cols: int) -> tuple[int, int]:
    """(code bytes, scale bytes) of one matrix."""
    return rows * words_per_row(cols) * 4, rows * (cols // SCALE_BLOCK) * 2


def blob_sections(d_model: int, d_ff: int):
    """[(name, rows, cols, code_offset, scale_offset)] and the blob stride."""
    out = []
    pos = 0
    for name, rows, cols in (("gate", d_ff, d_model), ("up", d_ff, d_model), ("down", d_model, d_ff)):
        cb, sb = matrix_bytes(rows, cols)
        out.append((name, rows, cols, pos, pos + cb))
        pos += cb + sb
    stride = (pos + BLOB_ALIGN - 1) // BLOB_ALIGN * BLOB_ALIGN
    return out, stride


def code_shift(j: int) -> int:
    """Bit position of code slot j (0..9) inside its word."""
    return 3 * j if j < 5 else 16 + 3 * (j - 5)


def unpack_codes(words: np.ndarray, cols: int) -> np.ndarray:
    """Codes [rows][cols] (int64, 0..7) from the words [rows][wpr] of a matrix."""
    rows = words.shape[0]
    w = words.astype(np.int64)
    out = np.empty((rows, cols), dtype=np.int64)
    for c in range(cols):
        out[:, c] = (w[:, c // CODES_PER_WORD] >> code_shift(c % CODES_PER_WORD)) & 7
    return out


def dequant_matrix(blob: np.ndarray, rows: int, cols: int, code_off: int, scale_off: int,
                   fp16_round: bool = False) -> np.ndarray:
    """W[r][c] = (q[r][c] - 4) * scale[r][c // 32], exact in float64.

    With ``fp16_round`` each product is rounded once to fp16 (round to
    nearest even), the operand the GPU's MFMA paths consume.
    """
    wpr = words_per_row(cols)
    words = np.frombuffer(blob, dtype=np.uint32, count=rows * wpr, offset=code_off).reshape(rows, wpr)
    scales = np.frombuffer(blob, dtype=np.float16, count=rows * (cols // SCALE_BLOCK),
                           offset=scale_off).reshape(rows, cols // SCALE_BLOCK).astype(np.float64)
    q = unpack_codes(words, cols)
    w = (q - 4).astype(np.float64) * np.repeat(scales, SCALE_BLOCK, axis=1)
    if fp16_round:
        w = w.astype(np.float16).astype(np.float64)
    return w


def expert_weights(blob: np.ndarray, d_model: int, d_ff: int, fp16_round: bool = False):
    """(W_gate [f][d], W_up [f][d], W_down [d][f]) as float64."""
    secs, stride = blob_sections(d_model, d_ff)
    if blob.size < stride:
        raise ValueError("blob shorter than its layout")
    mats = []
    for _name, rows, cols, co, so in secs:
        mats.append(dequant_matrix(blob, rows, cols, co, so, fp16_round))
    return tuple(mats)


# ---------------------------------------------------------------------------
# Router (reading: softmax scoring, top-k with lower-index tie-break,
# renormalised over the k chosen)
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """logits[t][e] = sum_c x[t][c] * W_r[e][c] + b[e], in float64."""
    lg = x.astype(np.float64) @ w_router.astype(np.float64).T
    if bias is not None:
        lg = lg + bias.astype(np.float64)[None, :]
    return lg


def topk_from_logits(logits: np.ndarray, k: int):
    """Top-k per row by (logit descending, expert index ascending), and weights.

    weights[t][j] = exp(l_j - m) / sum_j' exp(l_j' - m), m = the row maximum,
    i.e. the softmax over all experts renormalised over the chosen k.
    Returns (idx int32 [T][k], w float64 [T][k]).
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    experts = np.broadcast_to(np.arange(E), logits.shape)
    # lexsort: the last key is the primary one -> logit descending, then index
    order = np.lexsort((experts, -logits), axis=-1)[:, :k]
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(np.take_along_axis(logits, order, axis=1) - m)
    w = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


def route(x, w_router, bias, k):
    """(logits float64 [T][E], idx int32 [T][k], w float64 [T][k])."""
    lg = router_logits(x, w_router, bias)
    idx, w = topk_from_logits(lg, k)
    return lg, idx, w


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """l_(k) - l_(k+1) per row (inf when k == E): the margin of the k-th pick."""
    s = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# ---------------------------------------------------------------------------
# Expert cache (reading: LRU over slots; the pages say only "hot cache")
# ---------------------------------------------------------------------------

class CapacityError(RuntimeError):
    pass


class LRUCache:
    """Slot table for (layer, expert) identities, id = layer * E + expert.

    State: slot_of[L*E] = -1, id_of[S] = -1, stamp[S] = 0, clock = 0.
    One ``resolve`` call (one layer's routing result):

    1. clock += 1;
    2. U = the sorted unique identities the call touches;
    3. each hit gets stamp = clock;
    4. each miss, in ascending identity order, takes the lowest-index free
       slot, else the slot with the smallest (stamp, slot) among slots whose
       stamp < clock (a slot touched in this call is never evicted); the
       evicted identity maps to -1 again; the new slot gets stamp = clock and
       (identity, slot) is appended to the miss list;
    5. lookups += |U|, hits += |U| - misses.

    Every miss finds a slot exactly when |U| <= S (each miss uses one slot not
    touched in this call, and S - hits of them exist), so a call with
    |U| > S fails with CapacityError before it changes anything, the clock
    included.

    With n_slots == n_layers * n_experts the cache is the identity map
    (slot = id) and every lookup is a hit.
    """

    def __init__(self, n_layers: int, n_experts: int, n_slots: int):
        self.L, self.E, self.S = n_layers, n_experts, n_slots
        self.identity = n_slots == n_layers * n_experts
        self.reset()

    def reset(self):
        self.slot_of = [-1] * (self.L * self.E)
        self.id_of = np.full(self.S, -1, dtype=np.int64)
        self.stamp = np.zeros(self.S, dtype=np.int64)
        self.clock = 0
        self.lookups = 0
        self.hits = 0
        self.misses = 0
        self.bytes_h2d = 0

    def resolve(self, layer: int, idx: np.ndarray, blob_bytes: int = 0):
        """Returns (slot_of_pair int32 like idx, [(id, slot)] misses)."""
        idx = np.asarray(idx)
        ids = layer * self.E + idx.astype(np.int64)
        uniq = sorted(set(int(i) for i in ids.reshape(-1)))
        if not self.identity and len(uniq) > self.S:
            raise CapacityError("one call touches more identities than there are slots")
        self.clock += 1
        misses = []
        if self.identity:
            self.lookups += len(uniq)
            self.hits += len(uniq)
            return ids.astype(np.int32), misses
        for i in uniq:
            s = self.slot_of[i]
            if s >= 0:
                self.stamp[s] = self.clock
        for i in uniq:
            if self.slot_of[i] >= 0:
                continue
            free = np.flatnonzero(self.id_of == -1)
            if free.size:
                victim = int(free[0])  # the lowest-index free slot
            else:
                # the smallest (stamp, slot) among slots not touched in this call
                elig = np.flatnonzero(self.stamp < self.clock)
                victim = int(elig[np.argmin(self.stamp[elig])])  # argmin takes the first (lowest slot) of equal stamps
                self.slot_of[int(self.id_of[victim])] = -1
            self.id_of[victim] = i
            self.slot_of[i] = victim
            self.stamp[victim] = self.clock
            misses.append((i, victim))
        self.lookups += len(uniq)
        self.hits += len(uniq) - len(misses)
        self.misses += len(misses)
        self.bytes_h2d += len(misses) * blob_bytes
        slot_of_pair = np.array([self.slot_of[int(i)] for i in ids.reshape(-1)], dtype=np.int32).reshape(idx.shape)
        return slot_of_pair, misses


# ---------------------------------------------------------------------------
# Token -> expert bucketing
# ---------------------------------------------------------------------------

def bucket(idx: np.ndarray, n_experts: int):
    """counts[E], offsets[E+1] (exclusive scan) and perm[T*k].

    perm lists the pair ids p = t*k + j grouped by expert in ascending expert
    order, ascending p inside each group.
    """
    flat = np.asarray(idx).reshape(-1)
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in flat:
        counts[int(e)] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    perm = np.empty(flat.size, dtype=np.int64)
    for p, e in enumerate(flat):
        perm[fill[int(e)]] = p
        fill[int(e)] += 1
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32)


# ---------------------------------------------------------------------------
# Expert FFN, combine
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


PRECISIONS = ("exact", "fp16_weights")


def expert_ffn(x_rows: np.ndarray, weights, precision: str = "exact") -> np.ndarray:
    """y[t] = W_d (silu(W_g x_t) * W_u x_t) for every row of x_rows.

    ``weights`` are the float64 matrices from ``expert_weights`` (already
    fp16-rounded for 'fp16_weights'); x and h are never rounded.
    """
    if precision not in PRECISIONS:
        raise ValueError(f"unknown precision {precision!r}")
    wg, wu, wd = weights
    x = np.asarray(x_rows, dtype=np.float64)
    g = x @ wg.T
    u = x @ wu.T
    h = silu(g) * u
    return h @ wd.T


def combine(y_pairs: np.ndarray, w: np.ndarray, y_shared: np.ndarray) -> np.ndarray:
    """out[t] = sum_{j ascending} w[t][j] * y_pairs[t*k+j] + y_shared[t]."""
    T, k = w.shape
    out = np.zeros((T, y_shared.shape[1]), dtype=np.float64)
    for t in range(T):
        acc = np.zeros(y_shared.shape[1], dtype=np.float64)
        for j in range(k):
            acc = acc + w[t, j] * y_pairs[t * k + j]
        out[t] = acc + y_shared[t]
    return out


def moe_layer(x, w_router, bias, k, blob_of_expert, shared_blob, d_model, d_ff,
              precision: str = "exact", idx=None, w=None):
    """One MoE layer.  ``blob_of_expert(e)`` returns expert e's blob bytes.

    Teacher forcing: pass ``idx`` (and optionally ``w``) to use a given routing
    instead of recomputing it (weights are recomputed from the oracle's own
    logits when ``w`` is None).
    Returns dict with logits, idx, w, y_pairs [T*k][d], y_shared [T][d],
    out (float32 [T][d]).
    """
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    lg = router_logits(x, w_router, bias)
    if idx is None:
        idx, w_o = topk_from_logits(lg, k)
    else:
        idx = np.asarray(idx, dtype=np.int32)
        m = lg.max(axis=1, keepdims=True)
        ex = np.exp(np.take_along_axis(lg, idx.astype(np.int64), axis=1) - m)
        w_o = ex / ex.sum(axis=1, keepdims=True)
    if w is None:
        w = w_o
    w = np.asarray(w, dtype=np.float64)
    y_pairs = np.zeros((T * k, d_model), dtype=np.float64)
    flat = idx.reshape(-1)
    for e in sorted(set(int(v) for v in flat)):
        pairs = np.nonzero(flat == e)[0]
        wts = expert_weights(blob_of_expert(e), d_model, d_ff, fp16_round=(precision != "exact"))
        y_pairs[pairs] = expert_ffn(x[pairs // k], wts, precision)
    wts = expert_weights(shared_blob, d_model, d_ff, fp16_round=(precision != "exact"))
    y_shared = expert_ffn(x, wts, precision)
    out = combine(y_pairs, w, y_shared)
    return dict(logits=lg, idx=idx, w=w, y_pairs=y_pairs, y_shared=y_shared, out=out.astype(np.float32),
                out64=out)


def chain_norm(out: np.ndarray) -> np.ndarray:
    """Next layer's input in a stacked run: each token's output centred over
    its features, then scaled to unit RMS:  c = out[t] - mean(out[t]);
    x_next[t] = c / sqrt(mean(c^2) + 1e-6).

    Not part of the pages' layer: it only keeps a 48-layer synthetic stack
    bounded while keeping each layer's dependence on the previous one.  The
    centring matters: the stand-in weights have mean -0.5 * scale, so expert
    outputs share a large common component; scaling alone would let it take
    over within a few layers and route every token to the same experts.
    """
    o = np.asarray(out, dtype=np.float64)
    c = o - o.mean(axis=1, keepdims=True)
    r = np.sqrt(np.mean(c * c, axis=1, keepdims=True) + 1e-6)
    return (c / r).astype(np.float32)
