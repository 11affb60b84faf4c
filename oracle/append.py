"""Writing a step's new K/V rows into the paged cache (oracle, test only).

Where a row goes: sequence b's new tokens are its last q_len_b positions
(seq_len_b already counts them, the same reading the attention oracle uses),
so token i of the sequence's block of new rows is logical position
p = seq_len_b - q_len_b + i, stored in page block_table[b][p // P], slot
p % P, for every KV head.  Growing the cache one step at a time this way is
the loop the pages' decode and speculative-verify kernels run inside
("Dual MI50, part 2", sections "Bug 2: the drafter read freed memory" and
"Decode: a new kernel for the shape MTP actually runs").

What is stored: a 16-bit cache keeps the input bits unchanged.  An fp8
E4M3FN cache stores the code whose value is nearest to x / s, where x is
the input value and s the KV head's fp32 scale (K scales first, then V
scales, as in the attention call), the quotient taken in fp32.  A tie goes
to the code with an even mantissa; magnitudes past the largest finite value
(448) store 448; NaN stores the NaN code; the sign is kept in every case.
The pages' own cache was quantised on write with per-row int8 scales
("Dual MI50, part 2", section "Prefill: teach the fork's fast kernel to
read the int8 cache"); here the format is the fp8 one the attention path
reads.  Each function follows that definition directly: a nearest-value
search over the 256-code table, no bit tricks.
"""
from __future__ import annotations

import numpy as np

from .codec import decode_bits, fp8_e4m3_table

_TABLE = fp8_e4m3_table()
_POS = _TABLE[:0x7F]            # codes 0x00..0x7E: the non-negative finite values, ascending
assert np.all(np.diff(_POS) > 0)


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN codes of fp32 values: nearest finite value after clamping the
    magnitude to 448, ties to the even code, sign kept, NaN to 0x7F | sign."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.minimum(np.where(nan, 0.0, a), 448.0)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return (code | sign).astype(np.uint8)


def new_row_positions(seq_len: int, q_len: int) -> np.ndarray:
    """Logical positions of a sequence's new rows."""
    return np.arange(seq_len - q_len, seq_len, dtype=np.int64)


def int8_encode_row(x) -> tuple:
    """int8 codes (as uint8 bits) and fp32 scale of one row of fp32 values:
    scale = amax / 127 with amax the largest |x| of the row (NaN if the row
    holds a NaN, infinity if it holds an infinity), code = x / scale rounded
    to the nearest integer, ties to even, limited to [-127, 127], both the
    division and amax / 127 in fp32; a NaN quotient (a zero or non-finite
    row) stores code 0.  This is the per-row quantisation of the pages' int8
    cache ("Dual MI50, part 2", section "Prefill: teach the fork's fast kernel
    to read the int8 cache"), in the plainest reading: symmetric, absolute
    maximum, round to nearest."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x)
    amax = np.float32(np.nan) if np.isnan(a).any() else a.max()
    scale = np.float32(amax / np.float32(127.0))
    codes = np.zeros(x.shape, dtype=np.int8)
    for i, v in enumerate(x.tolist()):
        with np.errstate(divide="ignore", invalid="ignore"):
            q = float(np.float32(v) / scale)        # one fp32 rounding
        if q != q:
            continue
        q = min(max(q, -127.0), 127.0)
        n = int(np.floor(q))
        frac = q - n
        if frac > 0.5 or (frac == 0.5 and n % 2 != 0):
            n += 1
        codes[i] = n
    return codes.view(np.uint8), scale


def append_kv(k_new: np.ndarray, v_new: np.ndarray, in_dtype: str, k_pool: np.ndarray, v_pool: np.ndarray,
              cache_dtype: str, block_table: np.ndarray, seq_lens, q_lens, kv_scale=None, page_size: int = 16,
              row_scale=None):
    """Pools (storage bits, [num_pages][Hkv][P][D]) after writing the new rows.

    k_new, v_new: storage bits [T][Hkv][D] of dtype in_dtype ("f16"/"bf16"),
    rows of sequence 0 first.  kv_scale: fp32 [2][Hkv] (fp8 caches only).
    row_scale: fp32 [2][num_pages][Hkv][P] row scales (int8 caches only).
    Returns new arrays (k, v, and for int8 the row scales); the inputs are
    not modified."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    rs_out = None if row_scale is None else np.array(row_scale, dtype=np.float32, copy=True)
    hkv = k_new.shape[1]
    t = 0
    for b, (sl, ql) in enumerate(zip(np.asarray(seq_lens).tolist(), np.asarray(q_lens).tolist())):
        for i, p in enumerate(new_row_positions(sl, ql).tolist()):
            page = int(block_table[b, p // page_size])
            slot = p % page_size
            for which, src, dst in ((0, k_new, k_out), (1, v_new, v_out)):
                for g in range(hkv):
                    bits = src[t + i, g, :]
                    if cache_dtype == in_dtype:
                        dst[page, g, slot, :] = bits
                    elif cache_dtype == "fp8_e4m3":
                        x = decode_bits(bits, in_dtype).astype(np.float32)      # exact: 16-bit values fit fp32
                        s = np.float32(np.asarray(kv_scale, dtype=np.float32).reshape(2, hkv)[which, g])
                        dst[page, g, slot, :] = e4m3_encode(x / s)               # fp32 quotient
                    elif cache_dtype == "int8":
                        x = decode_bits(bits, in_dtype).astype(np.float32)
                        dst[page, g, slot, :], rs_out[which, page, g, slot] = int8_encode_row(x)
                    else:
                        raise ValueError(f"cannot store {in_dtype} rows in a {cache_dtype} cache")
        t += ql
    if cache_dtype == "int8":
        return k_out, v_out, rs_out
    return k_out, v_out
