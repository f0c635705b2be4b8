"""Device plumbing around libmoe: pools and buffers in torch memory, one context.

torch provides the allocations (device memory, pinned host memory) and the
stream; every step of the layer runs in libmoe's kernels through ``binding``.
"""
from __future__ import annotations

import torch

from . import binding as B


class MoeContext:
    """Owns the slot pool, the shared pool, the optional pinned host store and a
    libmoe context sized for ``max_tokens``."""

    def __init__(self, d_model, d_ff, n_experts, top_k, n_layers, n_slots=None, max_tokens=16,
                 device="cuda:0", host_store=None, slot_pool=None, shared_pool=None):
        self.d_model, self.d_ff, self.E, self.k, self.L = d_model, d_ff, n_experts, top_k, n_layers
        self.ids = n_layers * n_experts
        self.n_slots = n_slots or self.ids
        self.resident = self.n_slots == self.ids
        self.max_tokens = max_tokens
        self.device = torch.device(device)
        self.stride = B.moe_expert_bytes(d_model, d_ff)
        if self.stride == 0:
            raise ValueError("invalid d_model / d_ff")
        self.slot_pool = slot_pool if slot_pool is not None else \
            torch.empty((self.n_slots, self.stride), dtype=torch.uint8, device=self.device)
        self.shared_pool = shared_pool if shared_pool is not None else \
            torch.empty((n_layers, self.stride), dtype=torch.uint8, device=self.device)
        if not self.resident and host_store is None:
            host_store = torch.empty((self.ids, self.stride), dtype=torch.uint8, pin_memory=True)
        self.host_store = host_store
        cfg = B.make_config(d_model, d_ff, n_experts, top_k, n_layers, self.n_slots, max_tokens,
                            self.slot_pool, self.shared_pool, host_store)
        self.ctx = B.moe_create(cfg)

    def close(self):
        if self.ctx:
            B.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def buffers(self, T):
        d, k, dev = self.d_model, self.k, self.device
        return dict(
            logits=torch.empty((T, self.E), dtype=torch.float32, device=dev),
            idx=torch.empty((T, k), dtype=torch.int32, device=dev),
            w=torch.empty((T, k), dtype=torch.float32, device=dev),
            slot=torch.empty((T, k), dtype=torch.int32, device=dev),
            y_pairs=torch.empty((T * k, d), dtype=torch.float32, device=dev),
            y_shared=torch.empty((T, d), dtype=torch.float32, device=dev),
            out=torch.empty((T, d), dtype=torch.float32, device=dev),
        )

    def layer(self, layer, x, w_router, bias, buf, path=B.MOE_PATH_AUTO, stream=None, logits=True, info=False,
              async_resolve=False):
        """route -> cache_resolve -> expert_ffn -> combine for one layer.  With
        ``async_resolve`` the slots come from moe_cache_resolve_async (no host
        round trip; misses filled by a kernel reading the pinned host store)."""
        T = x.shape[0]
        B.moe_route(self.ctx, layer, x, T, w_router, bias, buf["logits"] if logits else None, buf["idx"], buf["w"],
                    stream)
        slot = buf["slot"] if (not self.resident or logits) else None
        if async_resolve:
            B.moe_cache_resolve_async(self.ctx, layer, buf["idx"], T, slot, stream)
            ri = None
        else:
            ri = B.moe_cache_resolve(self.ctx, layer, buf["idx"], T, slot, info, stream)
        B.moe_expert_ffn(self.ctx, layer, x, T, buf["idx"], slot, buf["y_pairs"], buf["y_shared"], path, stream)
        B.moe_combine(self.ctx, buf["y_pairs"], buf["w"], buf["y_shared"], T, buf["out"], stream)
        return ri


class KvTier:
    """The stores of a moe_kv handle, allocated with torch: the resident window
    in device memory and the streamed cells in pinned host memory (torch's
    pinned allocations come from hipHostMalloc, so the library can map them)."""

    def __init__(self, n_layers, cells_total, cells_resident, values=1024, block_cells=256, stage_cells=4096,
                 device="cuda:0"):
        self.cb = B.moe_kv_cell_bytes(values)
        if self.cb == 0:
            raise ValueError("unsupported values per cell")
        self.values, self.cells_total, self.cells_resident = values, cells_total, cells_resident
        self.resident = torch.empty((n_layers, max(cells_resident, 1), self.cb), dtype=torch.uint8, device=device)
        self.host = torch.empty((n_layers, max(cells_total - cells_resident, 1), self.cb), dtype=torch.uint8,
                                pin_memory=True)
        cfg = B.moe_kv_config(n_layers, values, cells_total, cells_resident, block_cells, stage_cells,
                              self.resident.data_ptr(), self.host.data_ptr())
        self.kv = B.moe_kv_create(cfg)

    def close(self):
        if self.kv:
            B.moe_kv_destroy(self.kv)
            self.kv = None
