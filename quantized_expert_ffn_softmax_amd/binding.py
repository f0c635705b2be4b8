"""ctypes binding of libmoe (include/libmoe.h): argument marshalling only.

Every function keeps the C name and order of arguments.  Tensor arguments may
be torch tensors (their ``data_ptr()`` is passed), integers (raw pointers) or
None (NULL).  ``stream`` may be a torch stream, an int handle or None (the
current torch stream when torch has a GPU, else NULL).  No computation happens
here: a missing or unloadable library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID = -1
MOE_ERR_ALIGN = -2
MOE_ERR_CAPACITY = -3
MOE_ERR_HIP = -4
MOE_ERR_OOM = -5

MOE_PATH_AUTO = 0
MOE_PATH_DECODE = 1
MOE_PATH_PREFILL = 2


class moe_config(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("n_slots", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("host_store", ctypes.c_void_p),
        ("slot_pool", ctypes.c_void_p),
        ("shared_pool", ctypes.c_void_p),
    ]


class moe_resolve_info(ctypes.Structure):
    _fields_ = [
        ("lookups", ctypes.c_int64),
        ("hits", ctypes.c_int64),
        ("misses", ctypes.c_int64),
        ("bytes_h2d", ctypes.c_uint64),
        ("resolve_calls", ctypes.c_int64),
        ("failed_calls", ctypes.c_int64),
    ]

    def as_dict(self):
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


class moe_kv_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("values", ctypes.c_int32),
        ("cells_total", ctypes.c_int32),
        ("cells_resident", ctypes.c_int32),
        ("block_cells", ctypes.c_int32),
        ("stage_cells", ctypes.c_int32),
        ("resident", ctypes.c_void_p),
        ("host", ctypes.c_void_p),
    ]


class moe_kv_stats(ctypes.Structure):
    _fields_ = [
        ("cells_written", ctypes.c_int64),
        ("cells_read", ctypes.c_int64),
        ("block_reads", ctypes.c_int64),
        ("vram_block_reads", ctypes.c_int64),
        ("host_bytes", ctypes.c_int64),
        ("prefetch_bytes", ctypes.c_int64),
    ]

    def as_dict(self):
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "moe_expert_bytes": (ctypes.c_size_t, [_I, _I]),
    "moe_create": (_I, [ctypes.POINTER(moe_config), ctypes.POINTER(_P)]),
    "moe_destroy": (_I, [_P]),
    "moe_route": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _P, _P]),
    "moe_cache_resolve": (_I, [_P, _I, _P, _I, _P, ctypes.POINTER(moe_resolve_info), _P]),
    "moe_cache_resolve_async": (_I, [_P, _I, _P, _I, _P, _P]),
    "moe_combine_norm": (_I, [_P, _P, _P, _P, _I, _P, _P, _P]),
    "moe_decode_layer": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _I, _P]),
    "moe_combine": (_I, [_P, _P, _P, _P, _I, _P, _P]),
    "moe_bucket": (_I, [_P, _P, _I, _P, _P, _P]),
    "moe_bucket_noalloc": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_cache_snapshot": (_I, [_P, _P, _P, _P]),
    "moe_cache_reset": (_I, [_P]),
    "moe_get_stats": (_I, [_P, ctypes.POINTER(moe_resolve_info)]),
    "moe_chain_norm": (_I, [_P, _P, _I, _P, _P]),
    "moe_peak_hbm_read": (_I, [_P, ctypes.c_uint64, _P, _I, _P]),
    "moe_peak_mfma_f16": (_I, [_I, _I, _P, _P]),
    "moe_kv_cell_bytes": (ctypes.c_size_t, [_I]),
    "moe_kv_create": (_I, [ctypes.POINTER(moe_kv_config), ctypes.POINTER(_P)]),
    "moe_kv_destroy": (_I, [_P]),
    "moe_kv_write": (_I, [_P, _I, _I, _I, _P, _P]),
    "moe_kv_read": (_I, [_P, _I, _I, _I, _P, _P]),
    "moe_kv_prefetch": (_I, [_P, _I, _I, _I, _P]),
    "moe_kv_get_stats": (_I, [_P, ctypes.POINTER(moe_kv_stats)]),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return list(_SIGS)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if isinstance(t, ctypes.Array) or isinstance(t, ctypes._Pointer):
        return ctypes.cast(t, ctypes.c_void_p).value
    raise TypeError(f"cannot pass {type(t)} as a pointer")


def _stream(s):
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:
            pass
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st: int, where: str):
    if st != MOE_OK:
        lib = load()
        raise MoeError(st, where, lib.moe_last_error().decode() or lib.moe_status_str(st).decode())


# --- the C calls, same names -------------------------------------------------

def moe_expert_bytes(d_model: int, d_ff: int) -> int:
    return int(load().moe_expert_bytes(d_model, d_ff))


def moe_create(cfg: moe_config) -> int:
    out = _P()
    _check(load().moe_create(ctypes.byref(cfg), ctypes.byref(out)), "moe_create")
    return out.value


def moe_destroy(ctx: int) -> None:
    _check(load().moe_destroy(ctx), "moe_destroy")


def moe_route(ctx, layer, x, T, w_router, bias, logits, idx, w, stream=None):
    _check(load().moe_route(ctx, layer, _ptr(x), T, _ptr(w_router), _ptr(bias), _ptr(logits), _ptr(idx),
                            _ptr(w), _stream(stream)), "moe_route")


def moe_cache_resolve(ctx, layer, idx, T, slot_of_pair, info=None, stream=None):
    """Returns the call's moe_resolve_info (as a dict) when ``info`` is True."""
    ri = moe_resolve_info() if info else None
    _check(load().moe_cache_resolve(ctx, layer, _ptr(idx), T, _ptr(slot_of_pair),
                                    ctypes.byref(ri) if ri is not None else None, _stream(stream)),
           "moe_cache_resolve")
    return ri.as_dict() if ri is not None else None


def moe_cache_resolve_async(ctx, layer, idx, T, slot_of_pair, stream=None):
    _check(load().moe_cache_resolve_async(ctx, layer, _ptr(idx), T, _ptr(slot_of_pair), _stream(stream)),
           "moe_cache_resolve_async")


def moe_expert_ffn(ctx, layer, x, T, idx, slot_of_pair, y_pairs, y_shared, path=MOE_PATH_AUTO, stream=None):
    _check(load().moe_expert_ffn(ctx, layer, _ptr(x), T, _ptr(idx), _ptr(slot_of_pair), _ptr(y_pairs),
                                 _ptr(y_shared), path, _stream(stream)), "moe_expert_ffn")


def moe_combine(ctx, y_pairs, w, y_shared, T, out, stream=None):
    _check(load().moe_combine(ctx, _ptr(y_pairs), _ptr(w), _ptr(y_shared), T, _ptr(out), _stream(stream)),
           "moe_combine")


def moe_bucket(ctx, idx, T, offsets, perm, stream=None):
    _check(load().moe_bucket(ctx, _ptr(idx), T, _ptr(offsets), _ptr(perm), _stream(stream)), "moe_bucket")


def moe_bucket_noalloc(idx, T, top_k, n_experts, offsets, perm, stream=None):
    _check(load().moe_bucket_noalloc(_ptr(idx), T, top_k, n_experts, _ptr(offsets), _ptr(perm), _stream(stream)),
           "moe_bucket_noalloc")


def moe_cache_snapshot(ctx, slot_of=None, id_of=None, stamp=None):
    """Host numpy arrays (or None) are filled in place."""
    def hp(a):
        return None if a is None else a.ctypes.data
    _check(load().moe_cache_snapshot(ctx, hp(slot_of), hp(id_of), hp(stamp)), "moe_cache_snapshot")


def moe_cache_reset(ctx) -> None:
    _check(load().moe_cache_reset(ctx), "moe_cache_reset")


def moe_get_stats(ctx) -> dict:
    ri = moe_resolve_info()
    _check(load().moe_get_stats(ctx, ctypes.byref(ri)), "moe_get_stats")
    return ri.as_dict()


def moe_combine_norm(ctx, y_pairs, w, y_shared, T, out, x_next, stream=None):
    _check(load().moe_combine_norm(ctx, _ptr(y_pairs), _ptr(w), _ptr(y_shared), T, _ptr(out), _ptr(x_next),
                                   _stream(stream)), "moe_combine_norm")


def moe_decode_layer(ctx, layer, x, T, w_router, bias, logits, idx, w, y_pairs, y_shared, out, x_next=None,
                     stream=None):
    _check(load().moe_decode_layer(ctx, layer, _ptr(x), T, _ptr(w_router), _ptr(bias), _ptr(logits), _ptr(idx),
                                   _ptr(w), _ptr(y_pairs), _ptr(y_shared), _ptr(out), _ptr(x_next), _stream(stream)),
           "moe_decode_layer")


def moe_chain_norm(ctx, out, T, x_next, stream=None):
    _check(load().moe_chain_norm(ctx, _ptr(out), T, _ptr(x_next), _stream(stream)), "moe_chain_norm")


def moe_status_str(s: int) -> str:
    return load().moe_status_str(s).decode()


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def make_config(d_model, d_ff, n_experts, top_k, n_layers, n_slots, max_tokens, slot_pool, shared_pool,
                host_store=None) -> moe_config:
    return moe_config(d_model, d_ff, n_experts, top_k, n_layers, n_slots, max_tokens, _ptr(host_store),
                      _ptr(slot_pool), _ptr(shared_pool))


def moe_peak_hbm_read(buf, nbytes, sink, n_blocks, stream=None):
    _check(load().moe_peak_hbm_read(_ptr(buf), nbytes, _ptr(sink), n_blocks, _stream(stream)), "moe_peak_hbm_read")


def moe_peak_mfma_f16(iters, n_blocks, sink, stream=None):
    _check(load().moe_peak_mfma_f16(iters, n_blocks, _ptr(sink), _stream(stream)), "moe_peak_mfma_f16")


# --- KV tier ------------------------------------------------------------------

def moe_kv_cell_bytes(values: int) -> int:
    return int(load().moe_kv_cell_bytes(values))


def moe_kv_create(cfg: moe_kv_config) -> int:
    out = _P()
    _check(load().moe_kv_create(ctypes.byref(cfg), ctypes.byref(out)), "moe_kv_create")
    return out.value


def moe_kv_destroy(kv: int) -> None:
    _check(load().moe_kv_destroy(kv), "moe_kv_destroy")


def moe_kv_write(kv, layer, first, n, vals, stream=None):
    _check(load().moe_kv_write(kv, layer, first, n, _ptr(vals), _stream(stream)), "moe_kv_write")


def moe_kv_read(kv, layer, first, n, out, stream=None):
    _check(load().moe_kv_read(kv, layer, first, n, _ptr(out), _stream(stream)), "moe_kv_read")


def moe_kv_prefetch(kv, layer, first, n, stream=None):
    _check(load().moe_kv_prefetch(kv, layer, first, n, _stream(stream)), "moe_kv_prefetch")


def moe_kv_get_stats(kv) -> dict:
    st = moe_kv_stats()
    _check(load().moe_kv_get_stats(kv, ctypes.byref(st)), "moe_kv_get_stats")
    return st.as_dict()
