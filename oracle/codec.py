"""Decoding of cache / query storage bits to float64 (oracle, test only).

* fp16: IEEE binary16, decoded by numpy's own float16 type.
* bf16: the upper 16 bits of an IEEE binary32; widening is a 16-bit left
  shift of the bit pattern, so the value is exact.
* fp8 E4M3FN (the OCP 8-bit format used for the cache): 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
  (value = m * 2^-9); there is no infinity, and S.1111.111 is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448.  The table below is built
  from that definition, one code at a time.

* int8: two's-complement signed bytes; the value is the integer itself.

Scales are applied by the caller after decoding: one fp32 scale per KV head
for fp8 caches, one fp32 scale per cached row (token and KV head) for int8
caches, the pages' own format ("Dual MI50, part 2", section "Prefill: teach
the fork's fast kernel to read the int8 cache").
"""
from __future__ import annotations

import numpy as np


def _fp8_e4m3_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9          # (m / 8) * 2^(1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_FP8_TABLE = np.array([_fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def fp8_e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3FN codes."""
    return _FP8_TABLE.copy()


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of storage bits of the given dtype."""
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):     # NaN payloads widen to NaN
            return u32.view(np.float32).astype(np.float64)
    if dtype == "fp8_e4m3":
        return _FP8_TABLE[np.asarray(bits, dtype=np.uint8)]
    if dtype == "int8":
        return np.asarray(bits, dtype=np.uint8).view(np.int8).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
