"""Pins of the KV-tier oracle (oracle/kv_oracle.py) against values written out
by hand from its definition and against the pages' byte counts:

* 1,056 bytes per int8 cell ("单卡5090跑125B 大模型 ...", section 2.2), and the
  same page's log line: 32,768 of 131,072 cells per layer in VRAM, the rest
  in 1.55 GiB of pinned RAM -- which the cell size has to divide into a whole
  number of layers;
* codes and scales of hand-worked groups: an exact scale of 1, the fp16
  rounding of 1/127, ties to even in both directions, a zero group, a scale
  that underflows fp16, a subnormal scale where the clamp to +-127 acts;
* the read-back error bound |q s - v| <= s / 2 on random groups;
* the VRAM / host accounting of block reads on hand-drawn ranges.
"""
import numpy as np
import pytest

from oracle import kv_oracle as kv


def _group(vals):
    v = np.zeros((1, kv.KV_VALUES), np.float32)
    v[0, :len(vals)] = vals
    return v


def _codes(cells, n):
    return cells[0, :n].view(np.int8).tolist()


def _scale_bits(cells, g=0):
    return int(cells[0, kv.KV_VALUES + 2 * g:kv.KV_VALUES + 2 * g + 2].view(np.uint16)[0])


def test_cell_bytes_and_the_pages_pinned_ram():
    assert kv.cell_bytes() == 1056
    streamed = (131072 - 32768) * kv.cell_bytes()
    layers = 1.55 * 2 ** 30 / streamed
    assert abs(layers - round(layers)) < 0.01 * layers  # 16.03: a whole number of layers
    assert round(layers) * streamed / 2 ** 30 == pytest.approx(1.55, abs=0.005)


def test_exact_scale_and_ties_to_even():
    # absmax 127 -> s = 127 / 127 = 1 exactly (fp16 0x3c00); codes = rint(v)
    c = kv.quantize_cells(_group([127, -127, 63.5, 0.5, 1.5, 2.5, -0.5, -3.5, 3.49]))
    assert _codes(c, 9) == [127, -127, 64, 0, 2, 2, 0, -4, 3]
    assert _scale_bits(c) == 0x3C00
    assert kv.dequantize_cells(c)[0, :9].tolist() == [127, -127, 64, 0, 2, 2, 0, -4, 3]


def test_fp16_rounding_of_the_scale():
    # absmax 1: 1/127 = 0.0078740157..., 2^-7 * (1 + m/1024) with m = 8.06 -> 8:
    # s16 = 0.00787353515625 (0x2008); 1/s16 = 127.0078, 0.5/s16 = 63.504,
    # 0.25/s16 = 31.752, 0.1/s16 = 12.70
    c = kv.quantize_cells(_group([1.0, -1.0, 0.5, 0.25, 0.1]))
    assert _scale_bits(c) == 0x2008
    assert _codes(c, 5) == [127, -127, 64, 32, 13]
    back = kv.dequantize_cells(c)[0, :5]
    assert back.tolist() == [127 * 0.00787353515625, -127 * 0.00787353515625, 64 * 0.00787353515625,
                             32 * 0.00787353515625, 13 * 0.00787353515625]


def test_zero_and_underflowing_groups():
    v = np.zeros((1, kv.KV_VALUES), np.float32)
    v[0, 64:67] = [1e-10, -5e-11, 0.0]  # group 1: absmax / 127 underflows fp16 -> s = 0
    c = kv.quantize_cells(v)
    assert _scale_bits(c, 0) == 0 and _scale_bits(c, 1) == 0
    assert not np.any(c[0, :kv.KV_VALUES])
    assert not np.any(kv.dequantize_cells(c))


def test_subnormal_scale_and_the_clamp():
    # absmax 1e-5: 1e-5 / 127 = 7.87e-8 rounds to the fp16 subnormal 2^-24 =
    # 5.96e-8 (0x0001); 1e-5 / 2^-24 = 167.8 -> clamped to 127; 5e-6 -> 83.9 -> 84
    c = kv.quantize_cells(_group([1e-5, -1e-5, 5e-6]))
    assert _scale_bits(c) == 0x0001
    assert _codes(c, 3) == [127, -127, 84]


def test_read_back_error_bound_random_groups():
    rng = np.random.default_rng(3)
    mags = 10.0 ** rng.uniform(-3, 3, size=(64, 16))  # per-group magnitudes over six decades
    v = (rng.standard_normal((64, 16, 64)) * mags[:, :, None]).astype(np.float32).reshape(64, 1024)
    c = kv.quantize_cells(v)
    back = kv.dequantize_cells(c)
    s = c[:, 1024:].copy().view(np.float16).astype(np.float32)
    err = np.abs(back - v).reshape(64, 16, 64)
    assert np.all(err <= s[:, :, None] * (0.5 + 1e-6) + 1e-30)
    codes = c[:, :1024].view(np.int8).reshape(64, 16, 64)
    assert np.all(np.abs(codes) <= 127)
    assert np.all(np.max(np.abs(codes), axis=2) >= 126)  # the largest value of a group maps to ~+-127


def test_tiers_and_block_read_accounting():
    assert kv.tier_of(0, 32768) == ("vram", 0) and kv.tier_of(32767, 32768) == ("vram", 32767)
    assert kv.tier_of(32768, 32768) == ("host", 0) and kv.tier_of(131071, 32768) == ("host", 98303)
    # cells 32,700..32,899 with 256-cell blocks: block 127 (32,512..32,767) all
    # resident; block 128 (32,768..33,023) 132 cells from host
    assert kv.read_accounting(32700, 200, 32768, 256, None, 1056) == (2, 1, 132 * 1056)
    # the same read after a prefetch of 4,096 cells from 32,768: both blocks from VRAM
    assert kv.read_accounting(32700, 200, 32768, 256, (32768, 4096), 1056) == (2, 2, 0)
    # cells 33,000..33,099 after a prefetch of block 128 (32,768..33,023): its 24
    # cells come from the staging copy, block 129's 76 from host
    assert kv.read_accounting(33000, 100, 32768, 256, (32768, 256), 1056) == (2, 1, 76 * 1056)
    # a prefetch ending at 33,008 covers only part of what the read takes from
    # block 128: that block is a host read too (16 + 76 cells from host)
    assert kv.read_accounting(33000, 100, 32768, 256, (32768, 240), 1056) == (2, 0, 92 * 1056)
    # a whole 131,072-cell context in 256-cell blocks: 128 of 512 blocks resident
    assert kv.read_accounting(0, 131072, 32768, 256, None, 1056) == (512, 128, 98304 * 1056)
