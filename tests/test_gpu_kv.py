"""GPU parity of the KV tier (moe_kv_*) against the oracle (oracle/kv_oracle),
through the C ABI, on seeded synthetic cells (moe_synth.gen_kv: log-normal
channel scales, and zero, underflowing, tie and 1e4-scaled groups):

* every written cell byte for byte -- the resident window read from HBM, the
  host tier from pinned memory -- and every read-back value exactly, over
  ranges that span both tiers with ragged ends, at 1,024 and 2,048 values per
  cell, on two layers;
* reads through the two prefetch slots, a write into a staged range (the
  staged copy follows), and the block accounting against the oracle's;
* the pages' shape (131,072 cells, the first 32,768 resident) written in full
  and read back on sampled cells;
* refusals that enqueue nothing.
"""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu_helpers import say
from oracle import kv_oracle as kvo
from quantized_expert_ffn_softmax_amd import binding as B
from quantized_expert_ffn_softmax_amd.runtime import KvTier

pytestmark = pytest.mark.gpu


def _write(t, layer, first, n, seed=5):
    v = moe_synth.gen_kv(seed, layer, first, n, t.values)
    B.moe_kv_write(t.kv, layer, first, n, torch.from_numpy(v).cuda())
    return v


def _cells(t, layer, first, n):
    """The stored bytes of cells [first, first + n) from both stores."""
    R = t.cells_resident
    res = t.resident[layer, first:min(first + n, R)].cpu().numpy() if first < R else np.zeros((0, t.cb), np.uint8)
    h0 = max(first, R)
    host = t.host[layer, h0 - R:first + n - R].numpy() if first + n > R else np.zeros((0, t.cb), np.uint8)
    return np.concatenate([res, host])


def _read(t, layer, first, n):
    out = torch.full((n, t.values), float("nan"), device="cuda")
    B.moe_kv_read(t.kv, layer, first, n, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("values", [1024, 2048])
def test_write_read_both_tiers(values):
    say(f"  KV tier: 2 layers x 1,000 cells (first 333 resident), {values} values per cell")
    t = KvTier(n_layers=2, cells_total=1000, cells_resident=333, values=values, block_cells=64, stage_cells=200)
    for layer in (0, 1):
        for first, n in ((0, 300), (300, 97), (397, 603)):  # spans the tier boundary, ragged ends
            _write(t, layer, first, n, seed=7 + layer)
    torch.cuda.synchronize()
    for layer in (0, 1):
        vals = moe_synth.gen_kv(7 + layer, layer, 0, 1000, values)
        want = kvo.quantize_cells(vals)
        assert np.array_equal(_cells(t, layer, 0, 1000), want), layer
        for first, n in ((0, 1000), (330, 7), (999, 1)):
            assert np.array_equal(_read(t, layer, first, n), kvo.dequantize_cells(want[first:first + n], values))
    st = B.moe_kv_get_stats(t.kv)
    assert st["cells_written"] == 2000 and st["cells_read"] == 2 * 1008
    t.close()


def test_prefetch_slots_staged_writes_and_accounting():
    R, total, block = 256, 2048, 64
    t = KvTier(n_layers=1, cells_total=total, cells_resident=R, values=1024, block_cells=block, stage_cells=512)
    vals = _write(t, 0, 0, total, seed=11)
    torch.cuda.synchronize()
    want = kvo.quantize_cells(vals)
    staged = []
    expect = [0, 0, 0]  # block reads, VRAM block reads, host bytes

    def read_check(first, n):
        got = _read(t, 0, first, n)
        assert np.array_equal(got, kvo.dequantize_cells(want[first:first + n])), (first, n)
        # the oracle's accounting against each staged range the read can see
        b, v, h = _account(first, n)
        expect[0] += b
        expect[1] += v
        expect[2] += h

    def _account(first, n):
        # a cell is from VRAM if resident or inside either staged range
        blocks = vram = host = 0
        c = first
        while c < first + n:
            end = min(first + n, (c // block + 1) * block)
            fh = sum(1 for cc in range(c, end) if cc >= R and not any(a <= cc < a + m for a, m in staged))
            blocks, vram, host = blocks + 1, vram + (fh == 0), host + fh * t.cb
            c = end
        return blocks, vram, host

    read_check(200, 200)                      # resident + host, nothing staged
    for first in (300, 900):                  # fill both slots
        B.moe_kv_prefetch(t.kv, 0, first, 512)
        staged.append((first, 512))
    read_check(300, 1112)                     # both slots and the resident window
    B.moe_kv_prefetch(t.kv, 0, 1500, 300)     # replaces the older slot (300..811)
    staged[0] = (1500, 300)
    read_check(250, 1798)
    # single-slot accounting matches the oracle function itself
    assert kvo.read_accounting(1500, 300, R, block, (1500, 300), t.cb) == (6, 6, 0)  # blocks 23..28, all staged
    # a write into a staged range: the staged copy and host memory both change
    new = _write(t, 0, 1600, 50, seed=12)
    want[1600:1650] = kvo.quantize_cells(new)
    torch.cuda.synchronize()
    assert np.array_equal(_cells(t, 0, 1600, 50), want[1600:1650])
    read_check(1550, 200)
    st = B.moe_kv_get_stats(t.kv)
    assert [st["block_reads"], st["vram_block_reads"], st["host_bytes"]] == expect
    assert st["prefetch_bytes"] == (512 + 512 + 300) * t.cb
    t.close()


def test_pages_shape_sampled():
    wl = moe_synth.WORKLOADS["kv_tier"]
    total, R, chunk = wl["cells_total"], wl["cells_resident"], wl["chunk_cells"]
    say(f"  KV tier at the pages' shape: {total} cells, first {R} resident, written in {chunk}-cell chunks")
    t = KvTier(n_layers=1, cells_total=total, cells_resident=R, values=wl["values"], block_cells=wl["block_cells"],
               stage_cells=chunk)
    for first in range(0, total, chunk):
        _write(t, 0, first, chunk, seed=21)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    cells = sorted(set(rng.integers(0, total, 48).tolist()) | {0, R - 1, R, total - 1})
    for c in cells:
        want = kvo.quantize_cells(moe_synth.gen_kv(21, 0, c, 1))
        assert np.array_equal(_cells(t, 0, c, 1), want), c
        assert np.array_equal(_read(t, 0, c, 1), kvo.dequantize_cells(want)), c
    # a whole-context read: 128 of 512 blocks resident
    out = torch.empty((total, t.values), device="cuda")
    s0 = B.moe_kv_get_stats(t.kv)
    B.moe_kv_read(t.kv, 0, 0, total, out)
    torch.cuda.synchronize()
    s1 = B.moe_kv_get_stats(t.kv)
    assert (s1["block_reads"] - s0["block_reads"], s1["vram_block_reads"] - s0["vram_block_reads"]) == (512, 128)
    got = out[cells].cpu().numpy()
    for i, c in enumerate(cells):
        assert np.array_equal(got[i], kvo.dequantize_cells(kvo.quantize_cells(moe_synth.gen_kv(21, 0, c, 1)))[0])
    t.close()


def test_refusals():
    t = KvTier(n_layers=1, cells_total=100, cells_resident=40, values=1024, block_cells=16, stage_cells=32)
    v = torch.zeros((10, 1024), device="cuda")
    for fn, args in ((B.moe_kv_write, (t.kv, 0, 95, 10, v)), (B.moe_kv_read, (t.kv, 1, 0, 10, v)),
                     (B.moe_kv_prefetch, (t.kv, 0, 0, 33)), (B.moe_kv_read, (t.kv, 0, -1, 5, v))):
        with pytest.raises(B.MoeError) as ei:
            fn(*args)
        assert ei.value.status == B.MOE_ERR_INVALID
    assert B.moe_kv_get_stats(t.kv) == {k: 0 for k in B.moe_kv_get_stats(t.kv)}
    # a host store that is not pinned memory cannot be mapped
    host = torch.empty((1, 60, t.cb), dtype=torch.uint8)
    cfg = B.moe_kv_config(1, 1024, 100, 40, 16, 32, t.resident.data_ptr(), host.data_ptr())
    with pytest.raises(B.MoeError) as ei:
        B.moe_kv_create(cfg)
    assert ei.value.status == B.MOE_ERR_INVALID
    assert B.moe_kv_cell_bytes(1024) == 1056 and B.moe_kv_cell_bytes(1000) == 0
    t.close()
