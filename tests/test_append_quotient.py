"""The append's fast quotient (CPU): x * fl(1/s), with the exact quotient
fl(x / s) taken wherever the product lies within 3 units in its last place of
a rounding boundary (a point half-way between two fp8 E4M3 codes from 2^-6 up,
every magnitude below 2^-6, or a half-integer for the int8 codes), rounds to
the same code as fl(x / s) itself.  The product is within 2.5 ulp of the
once-rounded quotient when s and 1/s are normal (two roundings of relative
size 2^-24 each, plus the quotient's own half ulp); this checks the claim on
random and adversarial inputs with numpy's IEEE float32 arithmetic, and that a
window of 0 ulp does not suffice (so the check can fail)."""
import numpy as np
import pytest

import oracle

f32 = np.float32


def _e4m3(q: np.ndarray) -> np.ndarray:
    """E4M3FN codes of fp32 values through the oracle's encoder."""
    return oracle.e4m3_encode(q.astype(np.float32))


def _fp8_near(q: np.ndarray, w: int) -> np.ndarray:
    a = q.view(np.uint32).astype(np.int64) & 0x7fffffff
    return (a < 0x3c800000) | (np.abs((a & 0xfffff) - 0x80000) <= w)


def _int_near(q: np.ndarray, w: int) -> np.ndarray:
    d = np.abs(np.abs(q - np.rint(q)) - f32(0.5))
    eb = (q.view(np.uint32).astype(np.int64) & 0x7f800000) - (23 << 23)
    ulp = np.maximum(eb, 0).astype(np.uint32).view(np.float32)
    return d <= w * ulp


def _fp8_inputs(rng, n, adversarial):
    s = (rng.uniform(0.001, 0.1, n) * (10.0 ** rng.integers(-3, 4, n))).astype(f32)
    if adversarial:
        table = oracle.fp8_e4m3_table()[:0x7F].astype(np.float64)
        mids = (table[:-1] + table[1:]) / 2
        x = (rng.choice(mids, n) * s.astype(np.float64)).astype(f32)
        x = (x.view(np.int32) + rng.integers(-4, 5, n).astype(np.int32)).view(f32)
        x = np.where(rng.random(n) < 0.5, -x, x).astype(f32)
    else:
        x = (rng.standard_normal(n) * (2.0 ** rng.integers(-140, 20, n))).astype(f32)
        x = (x.view(np.uint32) & 0xffff0000).view(f32)          # bf16 values
    return x, s


def _fp8_mismatches(x, s, w):
    with np.errstate(all="ignore"):
        q_rn = (x / s).astype(f32)
        q1 = (x * (f32(1) / s).astype(f32)).astype(f32)
    exact = _e4m3(q_rn)
    fast = np.where(_fp8_near(q1, w), exact, _e4m3(q1))
    return int(np.sum(fast != exact))


@pytest.mark.parametrize("adversarial", [False, True])
def test_fp8_fast_quotient_matches_the_exact_code(adversarial):
    rng = np.random.default_rng(11 + adversarial)
    x, s = _fp8_inputs(rng, 1_000_000, adversarial)
    assert _fp8_mismatches(x, s, 3) == 0


def test_fp8_window_of_zero_ulp_is_not_enough():
    rng = np.random.default_rng(13)
    x, s = _fp8_inputs(rng, 200_000, True)
    assert _fp8_mismatches(x, s, 0) > 0


def _int8_case(rng, rows):
    x = (rng.standard_normal((rows, 16)) * (2.0 ** rng.integers(-20, 10, (rows, 1)))).astype(f32)
    x = (x.view(np.uint32) & 0xffff0000).view(f32)
    amax = np.max(np.abs(x), axis=1, keepdims=True).astype(f32)
    s = (amax / f32(127)).astype(f32)
    k = rng.integers(-126, 126, (rows, 16)) + 0.5                  # planted half-integer quotients
    x2 = (k * s.astype(np.float64)).astype(f32)
    x2 = (x2.view(np.int32) + rng.integers(-3, 4, (rows, 16)).astype(np.int32)).view(f32)
    x2 = (x2.view(np.uint32) & 0xffff0000).view(f32)
    x = np.where(rng.random((rows, 16)) < 0.7, x2, x).astype(f32)
    amax = np.max(np.abs(x), axis=1, keepdims=True).astype(f32)
    return x, (amax / f32(127)).astype(f32)


def _int8_mismatches(x, s, w):
    ok = np.broadcast_to(s > 0, x.shape)
    with np.errstate(all="ignore"):
        q_rn = (x / s).astype(f32)
        q1 = (x * (f32(1) / s).astype(f32)).astype(f32)
    code = lambda q: np.rint(np.clip(q, -127, 127))
    fast = np.where(_int_near(q1, w), code(q_rn), code(q1))
    return int(np.sum(ok & (fast != code(q_rn))))


def test_int8_fast_quotient_matches_the_exact_code():
    x, s = _int8_case(np.random.default_rng(17), 60_000)
    assert _int8_mismatches(x, s, 3) == 0


def test_int8_window_of_zero_ulp_is_not_enough():
    x, s = _int8_case(np.random.default_rng(19), 60_000)
    assert _int8_mismatches(x, s, 0) > 0
