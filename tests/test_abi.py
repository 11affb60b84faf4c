"""The C ABI library loads and exports every function include/paged_attn.h
declares, and rejects bad configurations on the host before any GPU work
(runs without a GPU)."""
import ctypes
import os

import pytest

import paged_attention_long_amd as pal
from paged_attention_long_amd import binding as B


def test_library_is_built():
    assert os.path.exists(B.LIB_PATH), "run python -m paged_attention_long_amd.build"


def test_exports_every_declared_function():
    lib = pal.load_library()
    names = pal.header_functions()
    assert {"paged_attn_create", "paged_attn_forward", "paged_attn_destroy"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_version():
    assert pal.paged_attn_version() == "0.2.0"


def _cfg(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16", max_num_seqs=4,
                max_q_len=8, max_num_tokens=32)
    base.update(kw)
    return pal.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=30), B.PA_ERR_INVALID_ARGUMENT),      # Hq % Hkv
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(q_dtype="fp8_e4m3"), B.PA_ERR_UNSUPPORTED),
    (dict(q_dtype="f16", kv_dtype="bf16"), B.PA_ERR_UNSUPPORTED),
    (dict(max_num_seqs=0), B.PA_ERR_INVALID_ARGUMENT),
    (dict(max_num_seqs=5000), B.PA_ERR_INVALID_ARGUMENT),
    (dict(max_q_len=0), B.PA_ERR_INVALID_ARGUMENT),
    (dict(max_num_tokens=0), B.PA_ERR_INVALID_ARGUMENT),
    (dict(num_q_heads=64, num_kv_heads=2), B.PA_ERR_UNSUPPORTED),   # group 32
    (dict(head_dim=512), B.PA_ERR_UNSUPPORTED),
    (dict(head_dim=64, max_q_len=17), B.PA_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_config_on_host(kw, code):
    cfg = _cfg(**kw)
    with pytest.raises(pal.PagedAttnError) as e:
        pal.paged_attn_create(cfg)
    assert e.value.code == code
    assert pal.paged_attn_last_error(None) != ""


@pytest.mark.parametrize("page_size", [0, 8, 24, 40, 65552])
def test_page_size_not_a_multiple_of_16_rejected(page_size):
    cfg = _cfg()
    cfg.page_size = page_size
    with pytest.raises(pal.PagedAttnError) as e:
        pal.paged_attn_create(cfg)
    assert e.value.code == B.PA_ERR_UNSUPPORTED
    assert "page_size" in pal.paged_attn_last_error(None)


def test_page_chunk_division_by_multiply_high():
    """The kernels find a 16-token chunk's page as umulhi(c, magic) >> shift
    with the host's magic number for d = page_size / 16: exact for every
    c < 2^24 (checked here on all of them for the pages' block sizes and a
    few others)."""
    import numpy as np

    c = np.arange(1 << 24, dtype=np.uint64)
    for d in (2, 3, 4, 5, 7, 64, 66, 99, 100, 127, 128, 129, 4095, 4096):
        s = 0
        while (1 << (s + 1)) < d:
            s += 1
        magic = ((1 << (32 + s)) + d - 1) // d
        assert magic < (1 << 32)
        q = ((c * np.uint64(magic)) >> np.uint64(32)) >> np.uint64(s)
        assert np.array_equal(q, c // np.uint64(d)), d


def test_unknown_flags_rejected():
    cfg = _cfg()
    cfg.flags = 2
    with pytest.raises(pal.PagedAttnError) as e:
        pal.paged_attn_create(cfg)
    assert e.value.code == B.PA_ERR_INVALID_ARGUMENT
    assert "flags" in pal.paged_attn_last_error(None)


def test_null_handle_calls_fail_cleanly():
    lib = pal.load_library()
    rc = lib.paged_attn_forward(None, None, 1, None, None, None, None, 1, 1, None, None, 0, 1.0, None, None, None,
                                None)
    assert rc == B.PA_ERR_INVALID_ARGUMENT
    assert lib.paged_attn_set_tuning(None, None) == B.PA_ERR_INVALID_ARGUMENT
    lib.paged_attn_destroy(None)
    out = ctypes.c_void_p()
    assert lib.paged_attn_create(None, ctypes.byref(out)) == B.PA_ERR_INVALID_ARGUMENT
    assert out.value is None
