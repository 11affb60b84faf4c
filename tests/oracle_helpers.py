"""Helpers for oracle self-tests: an independent logical (dense) view of the
generated cache, decoded with torch's own dtype conversions.

The dense view indexes the generator's live pages in their (sequence,
logical page) order, which never goes through the block table, so it is an
independent path to the same logical cache that the oracle de-pages.
"""
from __future__ import annotations

import numpy as np
import torch

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn, "int8": torch.int8}
_VIEW = {"f16": torch.int16, "bf16": torch.int16, "fp8_e4m3": torch.uint8, "int8": torch.uint8}


def torch_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    arr = np.ascontiguousarray(bits)
    if dtype in ("f16", "bf16"):
        t = torch.from_numpy(arr.view(np.int16))
    else:
        t = torch.from_numpy(arr.view(np.uint8))
    return t.view(_TORCH[dtype]).to(torch.float64).numpy()


def dense_view(inp, b: int):
    """(q [q_len][Hq][D], k [Hkv][seq_len][D], v ...) of sequence b as lists."""
    P = inp.page_size
    s, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
    o0 = int(inp.page_offsets[b])
    kk = torch_decode(inp.k_live[o0:o0 + (s + P - 1) // P], inp.kv_dtype)
    vv = torch_decode(inp.v_live[o0:o0 + (s + P - 1) // P], inp.kv_dtype)
    # [pages, Hkv, P, D] -> [Hkv, pages*P, D]
    kk = kk.transpose(1, 0, 2, 3).reshape(inp.num_kv_heads, -1, inp.head_dim)[:, :s]
    vv = vv.transpose(1, 0, 2, 3).reshape(inp.num_kv_heads, -1, inp.head_dim)[:, :s]
    if inp.kv_dtype == "fp8_e4m3":
        kk = kk * inp.kv_scale[0][:, None, None].astype(np.float64)
        vv = vv * inp.kv_scale[1][:, None, None].astype(np.float64)
    if inp.kv_dtype == "int8":
        # the generator's own per-row scales, in (logical page, slot) order
        n = (s + P - 1) // P
        for w, arr in ((0, "kk"), (1, "vv")):
            rs = inp.row_scale[w, o0:o0 + n].astype(np.float64)          # [pages, Hkv, P]
            rs = rs.transpose(1, 0, 2).reshape(inp.num_kv_heads, -1)[:, :s]
            if w == 0:
                kk = kk * rs[:, :, None]
            else:
                vv = vv * rs[:, :, None]
    t0 = int(np.sum(inp.q_lens[:b]))
    qq = torch_decode(inp.q[t0:t0 + ql], inp.q_dtype)
    return qq.tolist(), kk.tolist(), vv.tolist()
