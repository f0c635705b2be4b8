"""Routed MoE layer with 3-bit block-quantised experts for MI355X (gfx950).

The compute lives in ``libmoe.so`` (HIP kernels behind the C ABI of
``include/libmoe.h``); ``binding`` marshals arguments to it and ``runtime``
adds a small context/buffer helper on top of torch device memory.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
