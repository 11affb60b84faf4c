"""Pins of the oracle's cache append and its E4M3FN encoder (CPU).

The encoder is checked against what fixes it from outside: torch's own
float8_e4m3fn cast (round to nearest even) on in-range values and on every
midpoint between neighbouring codes, the exact round trip of every finite
code, the format's saturation and NaN rules, and a brute-force nearest-value
search.  The append is checked by brute force on small caches."""
import numpy as np
import pytest
import torch

import oracle
from oracle.append import append_kv, e4m3_encode

TABLE = oracle.fp8_e4m3_table()


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_matches_torch_cast_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (1e-3, 0.1, 1.0, 30.0, 150.0)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(e4m3_encode(x), _torch_codes(x))


def test_midpoints_round_to_even_code():
    pos = TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)   # exact in fp32
    codes = e4m3_encode(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0, 0x7E)) | (codes == np.arange(1, 0x7F)))
    assert np.array_equal(codes, _torch_codes(mids))
    assert np.array_equal(e4m3_encode(-mids), codes | 0x80)


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if not np.isnan(TABLE[c])], dtype=np.uint8)
    vals = TABLE[codes].astype(np.float32)
    got = e4m3_encode(vals)
    # +0 and -0 keep their sign bits
    assert np.array_equal(got, codes)


def test_saturation_nan_and_sign():
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e30, np.inf, -500.0, -np.inf, np.nan, -np.nan, 0.0, -0.0],
                 dtype=np.float32)
    assert e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0xFF, 0x00, 0x80]


def test_brute_force_nearest():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(2000) * rng.choice([1e-3, 1.0, 100.0], 2000)).astype(np.float32)
    codes = e4m3_encode(x)
    finite = TABLE[~np.isnan(TABLE)]
    for xi, ci in zip(x.tolist(), codes.tolist()):
        best = np.min(np.abs(finite - xi))
        assert abs(TABLE[ci] - xi) == best


@pytest.mark.parametrize("cache_dtype", ["f16", "fp8_e4m3"])
def test_append_brute_force(cache_dtype):
    rng = np.random.default_rng(3)
    P, hkv, D, pages = 16, 2, 8, 12
    seq_lens, q_lens = np.array([20, 5, 16, 33]), np.array([3, 5, 0, 17])
    bt = rng.permutation(pages)[:12].reshape(4, 3).astype(np.int32)     # distinct pages per sequence
    T = int(q_lens.sum())
    k_new = rng.standard_normal((T, hkv, D)).astype(np.float16).view(np.uint16)
    v_new = rng.standard_normal((T, hkv, D)).astype(np.float16).view(np.uint16)
    st = np.uint16 if cache_dtype == "f16" else np.uint8
    k_pool = rng.integers(0, 255, (pages, hkv, P, D)).astype(st)
    v_pool = rng.integers(0, 255, (pages, hkv, P, D)).astype(st)
    scale = np.array([[0.5, 2.0], [0.25, 3.0]], dtype=np.float32)
    k_out, v_out = append_kv(k_new, v_new, "f16", k_pool, v_pool, cache_dtype, bt, seq_lens, q_lens, scale, P)
    touched = np.zeros((pages, P), dtype=bool)
    t = 0
    for b in range(4):
        for i in range(int(q_lens[b])):
            p = int(seq_lens[b] - q_lens[b] + i)
            pg, sl = int(bt[b, p // P]), p % P
            touched[pg, sl] = True
            for g in range(hkv):
                for which, new, out in ((0, k_new, k_out), (1, v_new, v_out)):
                    if cache_dtype == "f16":
                        assert np.array_equal(out[pg, g, sl], new[t + i, g])
                    else:
                        x = new[t + i, g].view(np.float16).astype(np.float64)
                        vals = TABLE[out[pg, g, sl]] * scale[which, g]
                        # nearest representable after scaling (fp32 quotient: within half a step)
                        step = np.abs(TABLE[out[pg, g, sl] ^ 1] - TABLE[out[pg, g, sl]]) * scale[which, g]
                        assert np.all(np.abs(vals - x) <= step / 2 * (1 + 1e-6))
        t += int(q_lens[b])
    # nothing else changed
    for pg in range(pages):
        for sl in range(P):
            if not touched[pg, sl]:
                assert np.array_equal(k_out[pg, :, sl], k_pool[pg, :, sl])
                assert np.array_equal(v_out[pg, :, sl], v_pool[pg, :, sl])


# ------------------------------------------------------------------ int8 rows with their own scale

def _torch_int8_row(x):
    """The same definition through torch's ops: fp32 amax / 127, fp32
    quotient, torch.round (half to even), clamp; NaN quotients to 0."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    s = t.abs().max() / torch.tensor(127.0, dtype=torch.float32)
    q = torch.round(t / s).clamp(-127, 127)
    q = torch.where(torch.isnan(q), torch.zeros_like(q), q)
    return q.to(torch.int8).view(torch.uint8).numpy(), np.float32(s.item())


def test_int8_rows_match_torch_ops():
    rng = np.random.default_rng(11)
    for scale in (1e-3, 0.3, 1.0, 50.0, 3e4):
        for _ in range(200):
            x = (rng.standard_normal(128) * scale).astype(np.float32)
            c, s = oracle.int8_encode_row(x)
            tc, ts = _torch_int8_row(x)
            assert s == ts
            assert np.array_equal(c, tc)


def test_int8_row_closed_forms():
    # exact multiples of a power-of-two scale: the codes are the integers
    k = np.arange(-127, 128, dtype=np.float32)
    c, s = oracle.int8_encode_row(k * np.float32(0.125))
    assert s == np.float32(0.125 * 127 / 127)
    assert np.array_equal(c.view(np.int8), k.astype(np.int8))
    # halfway between integers (exact in fp32): to the even integer
    x = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], dtype=np.float32)
    c, s = oracle.int8_encode_row(x)
    assert s == np.float32(1.0)
    assert c.view(np.int8).tolist() == [127, 0, 2, 2, 0, -2, -2, 126]
    # the largest magnitude maps to +-127, a zero row to zeros with scale 0
    c, s = oracle.int8_encode_row(np.array([-3.0, 1.0, 2.0], np.float32))
    assert c.view(np.int8)[0] == -127
    c, s = oracle.int8_encode_row(np.zeros(16, np.float32))
    assert s == 0 and not c.any()
    # a NaN in the row: NaN scale, codes 0
    c, s = oracle.int8_encode_row(np.array([1.0, np.nan, 2.0], np.float32))
    assert np.isnan(s) and not c.any()


def test_int8_append_places_rows_and_scales():
    """append_kv with an int8 cache writes each new row's codes and its scale
    to the row's own page and slot (brute force over a small pool)."""
    rng = np.random.default_rng(12)
    hkv, D, P, pages = 2, 16, 16, 9
    seq_lens, q_lens = np.array([20, 5, 33]), np.array([4, 0, 3])
    T = int(q_lens.sum())
    new = rng.standard_normal((2, T, hkv, D)).astype(np.float32)
    bits = torch.from_numpy(new).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pool = rng.integers(0, 256, (2, pages, hkv, P, D)).astype(np.uint8)
    rs = rng.uniform(0, 1, (2, pages, hkv, P)).astype(np.float32)
    bt = np.array([[3, 5, 0], [1, 0, 0], [7, 2, 8]], dtype=np.int32)
    k2, v2, rs2 = append_kv(bits[0], bits[1], "bf16", pool[0], pool[1], "int8", bt, seq_lens, q_lens,
                            page_size=P, row_scale=rs)
    want_k, want_v, want_rs = pool[0].copy(), pool[1].copy(), rs.copy()
    t = 0
    for b in range(3):
        for i in range(int(q_lens[b])):
            p = int(seq_lens[b] - q_lens[b] + i)
            pg, sl = int(bt[b, p // P]), p % P
            for g in range(hkv):
                for w, dst in ((0, want_k), (1, want_v)):
                    x = oracle.decode_bits(bits[w, t + i, g], "bf16").astype(np.float32)
                    dst[pg, g, sl], want_rs[w, pg, g, sl] = _torch_int8_row(x)
        t += int(q_lens[b])
    assert np.array_equal(k2, want_k) and np.array_equal(v2, want_v)
    assert np.array_equal(rs2, want_rs)
