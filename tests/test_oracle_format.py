"""Pins for the oracle's blob layout and dequantisation (CPU only).

The oracle unpacks codes with its own shift table; these tests pack codes with
an independent bit-placement rule and hand-worked words, and check the exact
values it dequantises to.
"""
import json
import os

import numpy as np
import pytest

import moe_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pack_word(codes):
    # independent statement of the rule: low half holds codes 0..4 in 3-bit
    # fields from bit 0, high half holds codes 5..9 from bit 16
    lo = sum(c << (3 * j) for j, c in enumerate(codes[:5]))
    hi = sum(c << (3 * j) for j, c in enumerate(codes[5:10]))
    return lo | (hi << 16)


def _pack_matrix(codes):
    rows, cols = codes.shape
    wpr = -(-cols // 10)
    wpr = -(-wpr // 4) * 4
    words = np.zeros((rows, wpr), dtype=np.uint32)
    for r in range(rows):
        for w in range(wpr):
            chunk = [int(v) for v in codes[r, 10 * w:10 * w + 10]]
            words[r, w] = _pack_word(chunk)
    return words


def _make_blob(d, f, codes, scales):
    """Blob from explicit code matrices and fp16 scale matrices (gate, up, down)."""
    parts = []
    for q, s in zip(codes, scales):
        parts.append(_pack_matrix(q).reshape(-1).view(np.uint8))
        parts.append(np.asarray(s, dtype=np.float16).reshape(-1).view(np.uint8))
    raw = np.concatenate(parts)
    stride = -(-raw.size // 256) * 256
    out = np.zeros(stride, dtype=np.uint8)
    out[:raw.size] = raw
    return out


def test_worked_words():
    g = json.load(open(os.path.join(GOLDEN, "format_words.json")))
    for item in g["words"]:
        codes = item["codes"]
        word = int(item["word"], 16)
        assert _pack_word(codes) == word
        n = len(codes)
        words = np.array([[word, 0, 0, 0]], dtype=np.uint32)
        got = oracle.unpack_codes(words, n)[0]
        assert list(got) == codes
        assert list(got - 4) == item["values"]


def test_fp16_scale_value():
    g = json.load(open(os.path.join(GOLDEN, "format_words.json")))
    for item in g["fp16"]:
        h = np.array([item["value"]], dtype=np.float16)
        assert int(h.view(np.uint16)[0]) == int(item["bits"], 16)
        assert float(h[0]) == item["exact"]


def test_blob_bytes():
    g = json.load(open(os.path.join(GOLDEN, "format_words.json")))
    assert oracle.blob_sections(2048, 768)[1] == g["blob_bytes"]["2048x768"]
    assert oracle.blob_sections(256, 128)[1] == g["blob_bytes"]["256x128"]
    # the generator's own layout arithmetic agrees
    assert moe_synth.blob_stride(2048, 768) == g["blob_bytes"]["2048x768"]
    assert moe_synth.blob_stride(256, 128) == g["blob_bytes"]["256x128"]


@pytest.mark.parametrize("cols", [32, 64, 96, 128, 160, 256, 768, 2048])
def test_pack_unpack_every_code_every_slot(cols):
    # every code value at every slot position, rows whose last word holds
    # 2, 4, 6 or 8 valid codes
    rows = 8
    c = np.arange(rows * cols) % 8
    codes = ((c + np.arange(rows * cols) // 7) % 8).reshape(rows, cols)
    words = _pack_matrix(codes)
    assert np.array_equal(oracle.unpack_codes(words, cols), codes)
    assert words.shape[1] == oracle.words_per_row(cols)


def test_dequant_values_exact():
    d, f = 64, 32
    rng = np.random.default_rng(5)
    codes = [rng.integers(0, 8, (f, d)), rng.integers(0, 8, (f, d)), rng.integers(0, 8, (d, f))]
    scales = [rng.uniform(0.01, 0.05, (f, d // 32)).astype(np.float16),
              rng.uniform(0.01, 0.05, (f, d // 32)).astype(np.float16),
              rng.uniform(0.01, 0.05, (d, f // 32)).astype(np.float16)]
    blob = _make_blob(d, f, codes, scales)
    wg, wu, wd = oracle.expert_weights(blob, d, f)
    for W, q, s in zip((wg, wu, wd), codes, scales):
        rows, cols = q.shape
        for r in range(rows):
            for cc in range(cols):
                assert W[r, cc] == (int(q[r, cc]) - 4) * float(s[r, cc // 32])


def test_dequant_fp16_rounding_is_single_rounding():
    d, f = 32, 32
    q = [np.full((f, d), 7), np.full((f, d), 1), np.full((d, f), 0)]
    s = [np.full((f, 1), 0.0301, dtype=np.float16)] * 2 + [np.full((d, 1), 0.0301, dtype=np.float16)]
    blob = _make_blob(d, f, q, s)
    exact = oracle.expert_weights(blob, d, f)
    r16 = oracle.expert_weights(blob, d, f, fp16_round=True)
    sv = float(np.float16(0.0301))
    assert exact[0][0, 0] == 3 * sv
    assert r16[0][0, 0] == float(np.float16(3 * sv))
    assert r16[2][0, 0] == -4 * sv  # power-of-two multiple: exact either way


def test_generator_codes_and_pads():
    d, f = 256, 128
    blob = moe_synth.gen_blob(0, 0, 3, d, f)
    secs, stride = oracle.blob_sections(d, f)
    assert blob.size == stride
    for _n, rows, cols, co, so in secs:
        wpr = oracle.words_per_row(cols)
        words = np.frombuffer(blob, np.uint32, rows * wpr, co).reshape(rows, wpr)
        # bits 15 and 31 and every slot past the row end are zero
        assert not np.any(words & np.uint32(0x80008000))
        full = oracle.unpack_codes(words, wpr * 10)
        assert not np.any(full[:, cols:])
        q = oracle.unpack_codes(words, cols)
        assert abs(q.mean() - 3.5) < 0.1
        sc = np.frombuffer(blob, np.float16, rows * (cols // 32), so).astype(np.float64)
        assert sc.min() >= 0.0099 and sc.max() <= 0.0501
    # deterministic and keyed by identity
    assert np.array_equal(blob, moe_synth.gen_blob(0, 0, 3, d, f))
    assert not np.array_equal(blob, moe_synth.gen_blob(0, 0, 4, d, f))
