"""ctypes binding of libpaged_attn.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does
nothing but turn torch tensors into pointers and sizes; all of the work runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpaged_attn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "paged_attn.h")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_OUT_OF_MEMORY = 3
PA_ERR_HIP = 4

PA_DTYPE_F16 = 1
PA_DTYPE_BF16 = 2
PA_DTYPE_FP8_E4M3 = 3
PA_DTYPE_INT8 = 4

PA_DEBUG_CHECKS = 1
PA_CHECK_LENGTHS = 1
PA_CHECK_TABLE = 2
PA_CHECK_PAGE = 4
PA_CHECK_TOKENS = 8

PA_PATH_AUTO = 0
PA_PATH_VALU = 1
PA_PATH_MFMA = 2

DTYPE_CODES = {"f16": PA_DTYPE_F16, "bf16": PA_DTYPE_BF16, "fp8_e4m3": PA_DTYPE_FP8_E4M3, "int8": PA_DTYPE_INT8}
ELEM_BYTES = {PA_DTYPE_F16: 2, PA_DTYPE_BF16: 2, PA_DTYPE_FP8_E4M3: 1, PA_DTYPE_INT8: 1}


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"paged_attn error {code}: {msg}")
        self.code = code


class pa_config_t(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("max_num_seqs", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("min_q_len", ctypes.c_int32),
        ("max_num_tokens", ctypes.c_int64),
        ("device", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class pa_cache_layout_t(ctypes.Structure):
    _fields_ = [
        ("num_pages", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
    ]


class pa_tuning_t(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32),
        ("kv_tiles_per_split", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("split_mode", ctypes.c_int32),
    ]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m paged_attention_long_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.paged_attn_create.argtypes = [ctypes.POINTER(pa_config_t), ctypes.POINTER(vp)]
    lib.paged_attn_create.restype = ctypes.c_int
    lib.paged_attn_forward.argtypes = [
        vp, vp, i64, vp, vp, ctypes.POINTER(pa_cache_layout_t), vp, i32, i32, vp, vp, i32, f32, vp, vp, vp, vp]
    lib.paged_attn_forward.restype = ctypes.c_int
    lib.paged_attn_destroy.argtypes = [vp]
    lib.paged_attn_destroy.restype = None
    lib.paged_attn_last_error.argtypes = [vp]
    lib.paged_attn_last_error.restype = ctypes.c_char_p
    lib.paged_attn_set_tuning.argtypes = [vp, ctypes.POINTER(pa_tuning_t)]
    lib.paged_attn_set_tuning.restype = ctypes.c_int
    lib.paged_attn_debug_gather.argtypes = [
        vp, vp, ctypes.POINTER(pa_cache_layout_t), vp, i32, i32, vp, vp, i32, vp, vp, i64, vp]
    lib.paged_attn_debug_gather.restype = ctypes.c_int
    lib.paged_attn_append.argtypes = [
        vp, vp, vp, ctypes.c_int64, vp, vp, ctypes.POINTER(pa_cache_layout_t), vp, ctypes.c_int32, ctypes.c_int32,
        vp, vp, vp, vp]
    lib.paged_attn_append.restype = ctypes.c_int
    lib.paged_attn_forward_noalloc.argtypes = [
        ctypes.POINTER(pa_config_t), vp, i64, vp, vp, ctypes.POINTER(pa_cache_layout_t), vp, i32, i32, vp, vp, i32,
        f32, vp, vp, vp, vp]
    lib.paged_attn_forward_noalloc.restype = ctypes.c_int
    lib.paged_attn_debug_status.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
    lib.paged_attn_debug_status.restype = ctypes.c_int
    lib.paged_attn_version.argtypes = []
    lib.paged_attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions include/paged_attn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_attn_\w+)\s*\(", text)))


def _check(rc: int, handle=None):
    if rc != PA_OK:
        msg = load_library().paged_attn_last_error(handle).decode()
        raise PagedAttnError(rc, msg)


class Handle:
    """Owns a pa_handle_t*; destroyed by paged_attn_destroy()."""

    def __init__(self, ptr: int, cfg: pa_config_t):
        self.ptr = ptr
        self.cfg = cfg

    @property
    def value(self):
        return self.ptr


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(num_q_heads: int, num_kv_heads: int, head_dim: int, q_dtype: str, kv_dtype: str,
                max_num_seqs: int, max_q_len: int, max_num_tokens: int, page_size: int = 16,
                device: int = 0, min_q_len: int = 1, flags: int = 0) -> pa_config_t:
    return pa_config_t(num_q_heads, num_kv_heads, head_dim, page_size, DTYPE_CODES[q_dtype],
                       DTYPE_CODES[kv_dtype], max_num_seqs, max_q_len, min_q_len, max_num_tokens, device, flags)


def paged_attn_create(cfg: pa_config_t) -> Handle:
    lib = load_library()
    out = ctypes.c_void_p()
    _check(lib.paged_attn_create(ctypes.byref(cfg), ctypes.byref(out)))
    return Handle(out.value, cfg)


def paged_attn_destroy(h: Optional[Handle]) -> None:
    if h is None or h.ptr is None:
        return
    load_library().paged_attn_destroy(h.ptr)
    h.ptr = None


def paged_attn_last_error(h: Optional[Handle]) -> str:
    return load_library().paged_attn_last_error(h.ptr if h else None).decode()


def paged_attn_set_tuning(h: Handle, path: int = 0, pages_per_split: int = 0, kv_tiles_per_split: int = 0,
                          grid: int = 0, split_mode: int = 0) -> None:
    t = pa_tuning_t(path, pages_per_split, kv_tiles_per_split, grid, split_mode)
    _check(load_library().paged_attn_set_tuning(h.ptr, ctypes.byref(t)), h.ptr)


def cache_layout(k_cache) -> pa_cache_layout_t:
    """Layout of a [num_pages, Hkv, P, D] tensor view (any strides, D contiguous)."""
    if k_cache.dim() != 4 or k_cache.stride(3) != 1:
        raise ValueError("cache must be a 4-d [num_pages, Hkv, P, D] view with D contiguous")
    return pa_cache_layout_t(k_cache.shape[0], k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))


_FLOAT16_NAMES = {PA_DTYPE_F16: "float16", PA_DTYPE_BF16: "bfloat16"}


def _check_16bit(name: str, t, q_dtype: int):
    """A 16-bit input must be raw 16-bit storage (int16/uint16 bits) or the
    handle's own floating type: f16 rows given to a bf16 handle (or the
    reverse) would be reinterpreted, so they are refused."""
    if t.element_size() != 2:
        raise ValueError(f"{name} must have 2-byte elements")
    kind = str(t.dtype).replace("torch.", "")
    if kind in ("float16", "bfloat16") and kind != _FLOAT16_NAMES[q_dtype]:
        raise ValueError(f"{name} is {kind} but the handle's q_dtype is {_FLOAT16_NAMES[q_dtype]}")


def _check_cache(h: Handle, k_cache):
    c = h.cfg
    if k_cache.element_size() != ELEM_BYTES[c.kv_dtype]:
        raise ValueError("cache element size does not match the handle's kv dtype")
    if tuple(k_cache.shape[1:]) != (c.num_kv_heads, c.page_size, c.head_dim):
        raise ValueError(f"cache shape {tuple(k_cache.shape)} is not [pages, {c.num_kv_heads}, "
                         f"{c.page_size}, {c.head_dim}]")


def _check_row_scales(h, k_cache, kv_scale):
    """An int8 cache's kv_scale is its row-scale pool: fp32, contiguous, one
    scale per cached row of K and of V (laid out like the cache with rows of
    one element)."""
    c = h.cfg
    if c.kv_dtype != PA_DTYPE_INT8 or kv_scale is None:
        return
    need = 2 * k_cache.shape[0] * k_cache.stride(0) // c.head_dim
    if kv_scale.element_size() != 4 or not kv_scale.is_contiguous() or kv_scale.numel() != need:
        raise ValueError(f"an int8 cache needs kv_scale as {need} contiguous fp32 row scales "
                         "(K rows then V rows, laid out like the cache)")


def _check_forward_args(h, q, k_cache, v_cache, block_table, out, lse):
    c = h.cfg
    if q.dim() != 3 or tuple(q.shape[1:]) != (c.num_q_heads, c.head_dim) or not q.is_contiguous():
        raise ValueError("q must be a contiguous [T, Hq, D] tensor")
    _check_16bit("q", q, c.q_dtype)
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous() or out.element_size() != 4:
        raise ValueError("out must be a contiguous fp32 [T, Hq, D] tensor")
    if lse is not None and (tuple(lse.shape) != tuple(q.shape[:2]) or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [T, Hq] tensor")
    _check_cache(h, k_cache)
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("v_cache must match k_cache in shape and strides")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.element_size() != 4:
        raise ValueError("block_table must be int32 [num_seqs, width] with unit column stride")


def paged_attn_forward(h: Handle, q, k_cache, v_cache, block_table, seq_lens, q_lens, window: int, scale: float,
                       kv_scale, out, lse=None, stream=None) -> None:
    """Enqueue paged attention; see include/paged_attn.h for the contract."""
    _check_forward_args(h, q, k_cache, v_cache, block_table, out, lse)
    _check_row_scales(h, k_cache, kv_scale)
    layout = cache_layout(k_cache)
    rc = load_library().paged_attn_forward(
        h.ptr, _ptr(q), q.shape[0], _ptr(k_cache), _ptr(v_cache), ctypes.byref(layout), _ptr(block_table),
        seq_lens.shape[0], block_table.stride(0), _ptr(seq_lens), _ptr(q_lens), int(window), float(scale),
        _ptr(kv_scale), _ptr(out), _ptr(lse), _stream_ptr(stream))
    _check(rc, h.ptr)


class _CfgView:
    """What the argument checks read from a handle: its configuration."""

    def __init__(self, cfg: pa_config_t):
        self.cfg = cfg
        self.ptr = None


def paged_attn_forward_noalloc(cfg: pa_config_t, q, k_cache, v_cache, block_table, seq_lens, q_lens, window: int,
                               scale: float, kv_scale, out, lse=None, stream=None) -> None:
    """Enqueue the forward that allocates nothing (fixed device array); see
    include/paged_attn.h.  Errors come from paged_attn_last_error(None)."""
    _check_forward_args(_CfgView(cfg), q, k_cache, v_cache, block_table, out, lse)
    _check_row_scales(_CfgView(cfg), k_cache, kv_scale)
    layout = cache_layout(k_cache)
    rc = load_library().paged_attn_forward_noalloc(
        ctypes.byref(cfg), _ptr(q), q.shape[0], _ptr(k_cache), _ptr(v_cache), ctypes.byref(layout),
        _ptr(block_table), seq_lens.shape[0], block_table.stride(0), _ptr(seq_lens), _ptr(q_lens), int(window),
        float(scale), _ptr(kv_scale), _ptr(out), _ptr(lse), _stream_ptr(stream))
    _check(rc, None)


def paged_attn_debug_gather(h: Handle, k_cache, block_table, seq_lens, q_lens, window: int, slots_out, rows_out,
                            stream=None) -> None:
    _check_cache(h, k_cache)
    layout = cache_layout(k_cache)
    rc = load_library().paged_attn_debug_gather(
        h.ptr, _ptr(k_cache), ctypes.byref(layout), _ptr(block_table), seq_lens.shape[0], block_table.stride(0),
        _ptr(seq_lens), _ptr(q_lens), int(window), _ptr(slots_out), _ptr(rows_out), slots_out.shape[0],
        _stream_ptr(stream))
    _check(rc, h.ptr)


def paged_attn_append(h: Handle, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_lens, kv_scale=None,
                      stream=None) -> None:
    """Enqueue the cache append; see include/paged_attn.h for the contract."""
    c = h.cfg
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dim() != 3 or tuple(t.shape[1:]) != (c.num_kv_heads, c.head_dim) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T, Hkv, D] tensor")
        _check_16bit(name, t, c.q_dtype)
    if v_new.shape != k_new.shape:
        raise ValueError("v_new must match k_new")
    _check_cache(h, k_cache)
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("v_cache must match k_cache in shape and strides")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.element_size() != 4:
        raise ValueError("block_table must be int32 [num_seqs, width] with unit column stride")
    _check_row_scales(h, k_cache, kv_scale)
    layout = cache_layout(k_cache)
    rc = load_library().paged_attn_append(
        h.ptr, _ptr(k_new), _ptr(v_new), k_new.shape[0], _ptr(k_cache), _ptr(v_cache), ctypes.byref(layout),
        _ptr(block_table), seq_lens.shape[0], block_table.stride(0), _ptr(seq_lens), _ptr(q_lens), _ptr(kv_scale),
        _stream_ptr(stream))
    _check(rc, h.ptr)


def paged_attn_debug_status(h: Handle):
    """(PA_CHECK_* bits, message) of a PA_DEBUG_CHECKS handle's device error
    word, which the call clears; the caller synchronises its stream first."""
    bits = ctypes.c_int32(0)
    rc = load_library().paged_attn_debug_status(h.ptr, ctypes.byref(bits))
    if rc not in (PA_OK, PA_ERR_INVALID_ARGUMENT):
        _check(rc, h.ptr)
    return bits.value, load_library().paged_attn_last_error(h.ptr).decode() if rc != PA_OK else ""


def paged_attn_version() -> str:
    return load_library().paged_attn_version().decode()
