"""The C-ABI library loads and exports what include/libmoe.h declares (CPU only:
no call here reaches a GPU -- only argument validation and pure host helpers)."""
import ctypes
import os
import re

import pytest

from quantized_expert_ffn_softmax_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return B.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.exported_symbols()) == names


def test_expert_bytes(lib):
    assert B.moe_expert_bytes(2048, 768) == 2228224
    assert B.moe_expert_bytes(256, 128) == 51200
    assert B.moe_expert_bytes(33, 128) == 0
    assert B.moe_expert_bytes(0, 0) == 0
    assert B.moe_expert_bytes(2048, 768) % 256 == 0


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert B.moe_status_str(s)
    assert B.moe_status_str(-99) == "unknown status"


def _cfg(**kw):
    base = dict(d_model=256, d_ff=128, n_experts=16, top_k=2, n_layers=1, n_slots=16, max_tokens=8,
                slot_pool=4096, shared_pool=8192, host_store=None)
    base.update(kw)
    return B.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=33), B.MOE_ERR_INVALID),
    (dict(d_model=96), B.MOE_ERR_INVALID),   # a valid blob shape, but rows of an odd number of scale blocks
    (dict(d_ff=8200), B.MOE_ERR_INVALID),
    (dict(n_experts=0), B.MOE_ERR_INVALID),
    (dict(n_experts=2000), B.MOE_ERR_INVALID),
    (dict(top_k=17), B.MOE_ERR_INVALID),
    (dict(top_k=0), B.MOE_ERR_INVALID),
    (dict(n_slots=17), B.MOE_ERR_INVALID),
    (dict(n_slots=0), B.MOE_ERR_INVALID),
    (dict(max_tokens=0), B.MOE_ERR_INVALID),
    (dict(slot_pool=None), B.MOE_ERR_INVALID),
    (dict(slot_pool=4100), B.MOE_ERR_ALIGN),
    (dict(shared_pool=8200), B.MOE_ERR_ALIGN),
    (dict(n_slots=8), B.MOE_ERR_INVALID),   # capped without host_store
])
def test_create_validation(lib, kw, code):
    out = ctypes.c_void_p()
    st = lib.moe_create(ctypes.byref(_cfg(**kw)), ctypes.byref(out))
    assert st == code
    assert out.value is None
    assert B.moe_last_error()


def test_null_context_calls(lib):
    assert lib.moe_route(None, 0, None, 1, None, None, None, None, None, None) == B.MOE_ERR_INVALID
    assert lib.moe_cache_resolve(None, 0, None, 1, None, None, None) == B.MOE_ERR_INVALID
    assert lib.moe_expert_ffn(None, 0, None, 1, None, None, None, None, 0, None) == B.MOE_ERR_INVALID
    assert lib.moe_combine(None, None, None, None, 1, None, None) == B.MOE_ERR_INVALID
    assert lib.moe_bucket(None, None, 1, None, None, None) == B.MOE_ERR_INVALID
    assert lib.moe_destroy(None) == B.MOE_ERR_INVALID
    assert lib.moe_get_stats(None, None) == B.MOE_ERR_INVALID
    assert lib.moe_cache_reset(None) == B.MOE_ERR_INVALID
    assert lib.moe_chain_norm(None, None, 1, None, None) == B.MOE_ERR_INVALID
    assert lib.moe_cache_resolve_async(None, 0, None, 1, None, None) == B.MOE_ERR_INVALID
    assert lib.moe_combine_norm(None, None, None, None, 1, None, None, None) == B.MOE_ERR_INVALID
    with pytest.raises(B.MoeError):
        B.moe_destroy(None)


def test_noalloc_bucket_validation(lib):
    # refused before any HIP call: null pointers, sizes past the static scratch
    p = 4096
    assert lib.moe_bucket_noalloc(None, 1, 1, 1, p, p, None) == B.MOE_ERR_INVALID
    assert lib.moe_bucket_noalloc(p, 13108, 10, 512, p, p, None) == B.MOE_ERR_INVALID  # 131,080 pairs
    assert lib.moe_bucket_noalloc(p, 8, 2, 1025, p, p, None) == B.MOE_ERR_INVALID
    assert lib.moe_bucket_noalloc(p, 0, 2, 16, p, p, None) == B.MOE_ERR_INVALID
    assert lib.moe_bucket_noalloc(p, 8, 33, 64, p, p, None) == B.MOE_ERR_INVALID
    assert "131,072" in B.moe_last_error() or B.moe_last_error()
