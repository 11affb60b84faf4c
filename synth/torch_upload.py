"""Place generated batches in device memory (torch), as raw storage bits.

The K and V pools are filled with the NaN pattern first, then every batch's
live pages are scattered to their physical ids, so any page no batch owns
(and the block table's padding page) holds NaN.  Marshalling only.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np
import torch

from .gen import PagedInputs


def _bits_tensor(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a))
    raise TypeError(a.dtype)


def _fill_value(inp: PagedInputs) -> int:
    if inp.kv_dtype in ("fp8_e4m3", "int8"):
        return int(inp.fill_bits)
    return int(np.array(inp.fill_bits, dtype=np.uint16).view(np.int16))


def upload_pool(batches: List[PagedInputs], device="cuda", layout: str = "hnd") -> Dict[str, torch.Tensor]:
    """K/V pools holding every batch's live pages.

    layout "hnd": [pages, Hkv, P, D] contiguous; "nhd": storage is
    [pages, P, Hkv, D] and the returned tensors are [pages, Hkv, P, D] views.
    int8 caches also get "row_scale": the contiguous fp32 row-scale storage
    (K scales, then V scales), the kv_scale argument of an int8 forward.
    """
    f = batches[0]
    sdtype = torch.int16 if f.kv_dtype in ("f16", "bf16") else torch.uint8
    shape = (f.num_pages, f.num_kv_heads, f.page_size, f.head_dim)
    if layout == "nhd":
        store = (f.num_pages, f.page_size, f.num_kv_heads, f.head_dim)
    else:
        store = shape
    pools = {}
    if f.row_scale is not None:
        # one fp32 scale per cached row, laid out like the cache with rows of
        # one element: [2][pages][Hkv][P] (HND) or [2][pages][P][Hkv] (NHD);
        # rows of pages no batch owns hold NaN
        sstore = (2, f.num_pages, f.page_size, f.num_kv_heads) if layout == "nhd" else (2,) + shape[:3]
        rs = torch.full(sstore, float("nan"), dtype=torch.float32, device=device)
        rview = rs.permute(0, 1, 3, 2) if layout == "nhd" else rs
        for inp in batches:
            idx = torch.from_numpy(inp.live_pages.astype(np.int64)).to(device)
            rview[:, idx] = torch.from_numpy(np.ascontiguousarray(inp.row_scale)).to(device)
        pools["row_scale"] = rs
    for name, attr in (("k", "k_live"), ("v", "v_live")):
        pool = torch.full(store, _fill_value(f), dtype=sdtype, device=device)
        view = pool.permute(0, 2, 1, 3) if layout == "nhd" else pool
        on_device = {}   # batches that share one host array (relocated copies) upload it once
        for inp in batches:
            arr = getattr(inp, attr)
            src = on_device.get(id(arr))
            if src is None:
                src = _bits_tensor(arr).to(device)
                on_device[id(arr)] = src
            idx = torch.from_numpy(inp.live_pages.astype(np.int64)).to(device)
            view[idx] = src
        pools[name] = view
        del on_device
    return pools


def upload_batch(inp: PagedInputs, device="cuda") -> Dict[str, torch.Tensor]:
    """Per-batch device tensors: q, block_table, seq_lens, q_lens, kv_scale."""
    d = {
        "q": _bits_tensor(inp.q).to(device),
        "block_table": torch.from_numpy(inp.block_table.astype(np.int32)).to(device),
        "seq_lens": torch.from_numpy(inp.seq_lens.astype(np.int32)).to(device),
        "q_lens": torch.from_numpy(inp.q_lens.astype(np.int32)).to(device),
        "kv_scale": None,
    }
    if inp.kv_scale is not None:
        d["kv_scale"] = torch.from_numpy(np.ascontiguousarray(inp.kv_scale, dtype=np.float32)).to(device)
    return d
