"""Synthetic workloads on the GPU: fill a libmoe context with generated experts
and run layers through the C ABI.  Used by the GPU tests, the smoke check and
the bench; the CPU oracle never imports this module.
"""
from __future__ import annotations

import numpy as np
import torch

from quantized_expert_ffn_softmax_amd import binding as B
from quantized_expert_ffn_softmax_amd.runtime import MoeContext

from . import fill_blobs, gen_bias, gen_blob, gen_router, gen_x, blob_stride


def _np(t):
    return t.detach().cpu().numpy()


def fill_pool(pool: torch.Tensor, ids, seed, d_model, d_ff, n_experts, chunk=256, threads=None):
    """Generate blobs for ``ids`` (identity ints or (layer, expert) tuples) into
    rows 0.. of ``pool`` (device or pinned host uint8 [n][stride])."""
    stride = blob_stride(d_model, d_ff)
    host = np.empty((min(chunk, len(ids)), stride), dtype=np.uint8)
    for i0 in range(0, len(ids), chunk):
        part = ids[i0:i0 + chunk]
        buf = host[:len(part)]
        fill_blobs(buf, part, seed, d_model, d_ff, n_experts, threads=threads)
        pool[i0:i0 + len(part)].copy_(torch.from_numpy(buf), non_blocking=False)


class SyntheticLayer:
    """One resident layer (layer index 0) with E experts, shared expert, router,
    optional Zipf bias and T tokens of x."""

    def __init__(self, seed, d_model, d_ff, n_experts, top_k, n_tokens, alpha=0.0, device="cuda:0", step=0,
                 max_tokens=None, x=None):
        self.seed, self.d_model, self.d_ff, self.E, self.k, self.T = seed, d_model, d_ff, n_experts, top_k, n_tokens
        self.ctx = MoeContext(d_model, d_ff, n_experts, top_k, 1, None, max_tokens or n_tokens, device)
        fill_pool(self.ctx.slot_pool, list(range(n_experts)), seed, d_model, d_ff, n_experts)
        fill_pool(self.ctx.shared_pool, [(0, n_experts)], seed, d_model, d_ff, n_experts)
        self.wr_np = gen_router(seed, 0, n_experts, d_model)
        self.bias_np = gen_bias(seed, 0, n_experts, alpha) if alpha else None
        self.x_np = gen_x(seed, step, n_tokens, d_model) if x is None else np.ascontiguousarray(x, dtype=np.float32)
        self.wr = torch.from_numpy(self.wr_np).to(device)
        self.bias = torch.from_numpy(self.bias_np).to(device) if self.bias_np is not None else None
        self.x = torch.from_numpy(self.x_np).to(device)
        self._blob_cache = {}

    def blob_np(self, e):
        if e not in self._blob_cache:
            self._blob_cache[e] = gen_blob(self.seed, 0, e, self.d_model, self.d_ff)
        return self._blob_cache[e]

    @property
    def shared_np(self):
        return self.blob_np(self.E)

    def forward_gpu(self, path=B.MOE_PATH_AUTO):
        buf = self.ctx.buffers(self.T)
        self.ctx.layer(0, self.x, self.wr, self.bias, buf, path)
        torch.cuda.synchronize()
        return {k: _np(v) for k, v in buf.items()}

    def close(self):
        self.ctx.close()
