"""CPU oracle for the KV tier -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

What the pages fix ("单卡5090跑125B 大模型 ...", section 2.2 and section 7.2;
"一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s", section 四个发现):

* the KV cache is stored as int8 at 1,056 bytes per cell;
* of a layer's 131,072 (or 262,144) cells only the first 32,768 stay in VRAM;
  the rest live in pinned host memory (1.55 GiB on the 131,072-cell box) and
  are streamed on demand, with an optional prefetch of the next blocks;
* the engine reports the share of KV block reads served from VRAM (98.8%).

Readings where the pages are silent (listed again in the design notes):

* a cell holds V = 1,024 values (one token's K and V of one layer) as int8
  codes in groups of G = 64, followed by one fp16 scale per group:
  1,024 + 2 * 16 = 1,056 bytes;
* a group's scale is s = fp16(absmax / 127) (the division in float32, the
  rounding to fp16 to nearest with ties to even); codes are
  q = clamp(rint(v / s), -127, 127) with the division in float32 and rint
  rounding ties to even; a group whose scale is 0 stores zero codes;
* a value reads back as q * s (exact in float32);
* cell c of a layer is in VRAM when c < resident, else at host index
  c - resident; a read of cells [first, first + n) touches the blocks
  floor(c / block) of its cells, and a block read is served from VRAM when
  every cell the read takes from that block comes from VRAM (the resident
  window, or a prefetched staging copy); the others read from host memory.

Every function is pinned in ``tests/test_oracle_kv.py`` (hand-worked codes and
scales, ties, zero groups, the error bound, the pages' byte counts).
"""
from __future__ import annotations

import numpy as np

KV_GROUP = 64
KV_VALUES = 1024


def cell_bytes(values: int = KV_VALUES, group: int = KV_GROUP) -> int:
    """int8 codes then one fp16 scale per group."""
    if values % group:
        raise ValueError("values must be a multiple of the group size")
    return values + 2 * (values // group)


def quantize_cells(vals: np.ndarray, group: int = KV_GROUP) -> np.ndarray:
    """float32 [n][V] -> uint8 [n][cell_bytes]: per group s = fp16(absmax / 127),
    q = clamp(rint(v / s), -127, 127) (float32 division, ties to even)."""
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    n, V = vals.shape
    g = vals.reshape(n, V // group, group)
    absmax = np.max(np.abs(g), axis=2)                              # exact in float32
    s16 = (absmax / np.float32(127.0)).astype(np.float32).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    q = np.rint(g / safe[:, :, None]).astype(np.float32)            # float32 division, rint = ties to even
    q = np.clip(q, -127, 127)
    q = np.where(s32[:, :, None] == 0, 0, q).astype(np.int8)
    out = np.empty((n, cell_bytes(V, group)), dtype=np.uint8)
    out[:, :V] = q.reshape(n, V).view(np.uint8)
    out[:, V:] = s16.view(np.uint8).reshape(n, -1)
    return out


def dequantize_cells(cells: np.ndarray, values: int = KV_VALUES, group: int = KV_GROUP) -> np.ndarray:
    """uint8 [n][cell_bytes] -> float32 [n][V]: q * s."""
    cells = np.ascontiguousarray(cells, dtype=np.uint8)
    n = cells.shape[0]
    q = cells[:, :values].view(np.int8).astype(np.float32).reshape(n, values // group, group)
    s = cells[:, values:].copy().view(np.float16).astype(np.float32).reshape(n, values // group)
    return (q * s[:, :, None]).reshape(n, values)


def tier_of(cell: int, resident: int):
    """('vram', slot) for the first `resident` cells, else ('host', index)."""
    return ("vram", cell) if cell < resident else ("host", cell - resident)


def read_accounting(first: int, n: int, resident: int, block: int, staged=None, cbytes: int = 0):
    """Blocks touched by a read of cells [first, first + n), how many are served
    from VRAM, and the bytes taken from host memory.  `staged` is a (first, n)
    range of cells held in VRAM by a prefetch, or None."""
    blocks, vram = 0, 0
    host_cells = 0
    c = first
    while c < first + n:
        b = c // block
        end = min(first + n, (b + 1) * block)
        from_host = 0
        for cc in range(c, end):
            in_stage = staged is not None and staged[0] <= cc < staged[0] + staged[1]
            if cc >= resident and not in_stage:
                from_host += 1
        blocks += 1
        vram += from_host == 0
        host_cells += from_host
        c = end
    return blocks, vram, host_cells * cbytes
