"""Pins of the fp64 oracle against facts fixed by the mathematics and by the
source pages -- not against itself.

* fp8 / bf16 / fp16 decoding against torch's conversions (library routines)
  and against hand-known codes;
* closed forms: one cached token gives out = V and lse = s; identical keys
  give the mean of V and lse = s + ln n; with Q = 0 and a position-probe V
  the output is the midpoint of the visible range and lse = ln(count), which
  fixes both mask bounds exactly; W = 1 gives V at the row's own position;
* invariants: probabilities sum to 1; output is bitwise invariant under a
  physical-page permutation; GQA equals MHA with replicated KV heads;
  (scale*c, Q/c) invariance; LSE merge of disjoint key splits equals the
  whole;
* brute force: a dense pure-Python implementation on the logical cache
  (math.fsum sums, explicit mask matrix) agrees to 1e-12;
* the sliding-window NaN test of "Dual MI50, part 2", section "Bug 2: the
  drafter read freed memory": with every out-of-window page NaN the output is
  finite and unchanged.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import Spec, generate
from synth.gen import permute_pool
from tests.oracle_helpers import dense_view, torch_decode


# ------------------------------------------------------------------ codecs

def test_fp8_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_bits(codes, "fp8_e4m3")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])


def test_fp8_known_codes():
    t = oracle.fp8_e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0      # largest finite
    assert t[0x38] == 1.0 and t[0xB8] == -1.0          # exponent field 7 = bias
    assert t[0x08] == 2.0 ** -6                        # smallest normal
    assert t[0x01] == 2.0 ** -9                        # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                    # largest subnormal
    assert t[0x00] == 0.0 and math.copysign(1, t[0x80]) == -1


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_16bit_decode_matches_torch(dtype):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ours = oracle.decode_bits(bits, dtype)
    ref = torch_decode(bits, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ------------------------------------------------------------------ helpers

def _spec(**kw):
    base = dict(name="t", num_q_heads=4, num_kv_heads=2, head_dim=8, seq_lens=(37,), q_lens=(1,),
                q_dtype="f16", kv_dtype="f16", page_size=4, seed=7)
    base.update(kw)
    return Spec(**base)


def _one(**kw):
    return generate(_spec(**kw))[0]


def _set_f16(arr_bits, idx, val):
    arr_bits[idx] = np.array(val, dtype=np.float16).view(np.uint16)


# ------------------------------------------------------------------ closed forms

def test_single_cached_token():
    inp = _one(seq_lens=(1,), q_lens=(1,), num_q_heads=2, num_kv_heads=1, head_dim=16)
    out, lse = oracle.attention(inp)
    k = torch_decode(inp.k_live[0, 0, 0], "f16")
    v = torch_decode(inp.v_live[0, 0, 0], "f16")
    for h in range(2):
        q = torch_decode(inp.q[0, h], "f16")
        s = float(np.float32(inp.scale)) * math.fsum(q * k)
        assert np.array_equal(out[0, h], v)
        assert abs(lse[0, h] - s) < 1e-12


def test_identical_keys_give_mean_of_values():
    inp = _one(seq_lens=(23,), q_lens=(1,), num_q_heads=3, num_kv_heads=1, head_dim=8)
    # every live key of head 0 := key at token 0
    k0 = inp.k_live[0, 0, 0].copy()
    inp.k_live[:, 0, :, :] = k0
    out, lse = oracle.attention(inp)
    n = 23
    P = inp.page_size
    v = torch_decode(inp.v_live, "f16")[:, 0].reshape(-1, 8)[:n]   # logical order (single seq)
    k = torch_decode(k0, "f16")
    for h in range(3):
        q = torch_decode(inp.q[0, h], "f16")
        s = float(np.float32(inp.scale)) * math.fsum(q * k)
        np.testing.assert_allclose(out[0, h], v.mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[0, h] - (s + math.log(n))) < 1e-12


@pytest.mark.parametrize("window", [0, 1, 2, 5, 16, 200])
@pytest.mark.parametrize("q_len", [1, 3, 8])
def test_mask_bounds_position_probe(window, q_len):
    """Q = 0 makes every visible score equal; V[j][0] = j then puts the mean
    position of the visible set in out[..., 0] and its size in lse."""
    s = 150
    inp = _one(seq_lens=(s,), q_lens=(q_len,), num_q_heads=2, num_kv_heads=1, window=window)
    inp.q[:] = 0
    P = inp.page_size
    for j in range(s):
        _set_f16(inp.v_live, (j // P, 0, j % P, 0), float(j))
    out, lse = oracle.attention(inp)
    for i in range(q_len):
        p = s - q_len + i
        lo = max(0, p - window + 1) if window > 0 else 0
        for h in range(2):
            assert out[i, h, 0] == pytest.approx((lo + p) / 2, abs=1e-12)
            assert lse[i, h] == pytest.approx(math.log(p - lo + 1), abs=1e-12)
            if window == 1:
                assert out[i, h, 0] == p


def test_window_wider_than_context_equals_no_window():
    a = _one(seq_lens=(50,), q_lens=(4,), window=0)
    b = _one(seq_lens=(50,), q_lens=(4,), window=50)
    oa, la = oracle.attention(a)
    ob, lb = oracle.attention(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


# ------------------------------------------------------------------ invariants

def test_probabilities_sum_to_one():
    inp = _one(seq_lens=(40, 9), q_lens=(3, 2), window=6)
    _, _, probs = oracle.attention(inp, return_probs=True)
    assert len(probs) == 5 * 4
    for (lo, p) in probs.values():
        assert abs(p.sum() - 1.0) < 1e-14
        assert np.all(p >= 0)


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8_e4m3", "int8"])
def test_block_table_permutation_is_bitwise_invariant(kv):
    inp = _one(seq_lens=(61, 17, 4), q_lens=(2, 1, 4), kv_dtype=kv, pool_pages=80)
    o1, l1 = oracle.attention(inp)
    o2, l2 = oracle.attention(permute_pool(inp, 3))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_block_table_permutation_invariant_with_48_token_pages():
    inp = _one(seq_lens=(200, 47), q_lens=(4, 2), page_size=48, pool_pages=20)
    o1, l1 = oracle.attention(inp)
    o2, l2 = oracle.attention(permute_pool(inp, 5))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_equals_mha_with_replicated_heads():
    inp = _one(seq_lens=(33,), q_lens=(2,), num_q_heads=6, num_kv_heads=2)
    out, lse = oracle.attention(inp)
    mha = _one(seq_lens=(33,), q_lens=(2,), num_q_heads=6, num_kv_heads=6)
    mha.q = inp.q.copy()
    mha.k_live = np.repeat(inp.k_live, 3, axis=1)
    mha.v_live = np.repeat(inp.v_live, 3, axis=1)
    mha.block_table = inp.block_table.copy()
    mha.live_pages = inp.live_pages.copy()
    mha.num_pages = inp.num_pages
    out2, lse2 = oracle.attention(mha)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-14)


def test_scale_q_invariance():
    a = _one(seq_lens=(29,), q_lens=(3,), scale=0.25)
    b = _one(seq_lens=(29,), q_lens=(3,), scale=0.5)
    # q/2 is exact in fp16 for these magnitudes (no subnormals at |q| >= 2^-13)
    qf = torch_decode(a.q, "f16")
    assert np.all((qf == 0) | (np.abs(qf) >= 2.0 ** -13))
    b.q = (qf / 2).astype(np.float16).view(np.uint16)
    oa, la = oracle.attention(a)
    ob, lb = oracle.attention(b)
    np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("cut", [0, 1, 20, 35, 41])
def test_lse_merge_of_disjoint_splits(cut):
    inp = _one(seq_lens=(42,), q_lens=(3,), window=30)
    out, lse = oracle.attention(inp)
    for t in range(3):
        for h in range(4):
            a = oracle.row_partial(inp, t, h, 0, cut)
            b = oracle.row_partial(inp, t, h, cut, 10 ** 9)
            o, l = oracle.merge_partials([a, b])
            np.testing.assert_allclose(o, out[t, h], rtol=0, atol=1e-13)
            assert abs(l - lse[t, h]) < 1e-13


# ------------------------------------------------------------------ brute force

BRUTE = [
    dict(seq_lens=(37,), q_lens=(1,)),
    dict(seq_lens=(9, 30, 4), q_lens=(1, 3, 4), num_q_heads=6, num_kv_heads=2),
    dict(seq_lens=(45,), q_lens=(8,), window=7),
    dict(seq_lens=(20, 33), q_lens=(0, 5), window=1),
    dict(seq_lens=(50,), q_lens=(5,), kv_dtype="bf16", q_dtype="bf16", num_q_heads=4, num_kv_heads=4),
    dict(seq_lens=(70, 12), q_lens=(4, 1), kv_dtype="fp8_e4m3", q_dtype="bf16", window=13),
    dict(seq_lens=(26,), q_lens=(2,), page_size=16, k_outlier_frac=0.1),
    # pages of 48 and of 1,056 tokens (the pages' hybrid-model block size,
    # "tps-maxxing on amd gpu", section "Baseline"): a token's page and slot
    # come from a division by a page size that is no power of two
    dict(seq_lens=(100, 49), q_lens=(3, 1), page_size=48, window=30),
    dict(seq_lens=(1100,), q_lens=(2,), page_size=1056, kv_dtype="fp8_e4m3", q_dtype="bf16"),
    # int8 codes with a scale per cached row
    dict(seq_lens=(60, 9), q_lens=(4, 1), kv_dtype="int8", q_dtype="bf16", window=21, k_outlier_frac=0.1),
    dict(seq_lens=(100,), q_lens=(2,), kv_dtype="int8", q_dtype="f16", page_size=48),
]


@pytest.mark.parametrize("kw", BRUTE)
def test_agrees_with_bruteforce(kw):
    inp = _one(**kw)
    out, lse = oracle.attention(inp)
    t0 = 0
    for b in range(inp.num_seqs):
        s, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
        q, k, v = dense_view(inp, b)
        bo, bl = oracle.dense_attention_bruteforce(q, k, v, s, ql, inp.window,
                                                   float(np.float32(inp.scale)), inp.group)
        if ql:
            np.testing.assert_allclose(out[t0:t0 + ql], np.array(bo), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[t0:t0 + ql], np.array(bl), rtol=0, atol=1e-12)
        t0 += ql
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_sampled_rows_match_full():
    inp = _one(seq_lens=(77, 31), q_lens=(6, 2), window=20, kv_dtype="bf16", q_dtype="bf16")
    out, lse = oracle.attention(inp)
    rows = [(0, 0), (3, 2), (5, 3), (6, 1), (7, 0)]
    got = oracle.attention_rows(inp, rows)
    for (t, h) in rows:
        o, l = got[(t, h)]
        np.testing.assert_allclose(o, out[t, h], rtol=0, atol=1e-13)
        assert abs(l - lse[t, h]) < 1e-13


def test_fp8_dequantisation_recovers_data():
    """code * scale must reproduce the float data within e4m3 rounding
    (half an ulp: 2^-4 relative for normals, 2^-10 * scale absolute below)."""
    inp = _one(seq_lens=(40,), q_lens=(1,), kv_dtype="fp8_e4m3", q_dtype="bf16", keep_float=True)
    for which, key in (("k", "k_float"), ("v", "v_float")):
        ref = inp.extra[key]
        for g in range(inp.num_kv_heads):
            got = oracle.depage(inp, which, 0, g, 0, 40)
            want = ref[:, g].reshape(-1, inp.head_dim)[:40].astype(np.float64)
            s = float(inp.kv_scale[0 if which == "k" else 1][g])
            err = np.abs(got - want)
            assert np.all(err <= np.abs(want) * 2.0 ** -4 + 2.0 ** -10 * s + 1e-12)


# ------------------------------------------------------------------ NaN poison (window)

def test_window_nan_poison_finite_and_unchanged():
    clean = _one(seq_lens=(130,), q_lens=(8,), window=20, pool_pages=64)
    dirty = _one(seq_lens=(130,), q_lens=(8,), window=20, pool_pages=64, poison_out_of_window=True)
    assert dirty.extra["poisoned_pages"], "nothing was poisoned"
    n_dead = dirty.extra["poisoned_pages"][0][1]
    assert np.all(np.isnan(torch_decode(dirty.k_live[:n_dead], "f16")))
    o1, l1 = oracle.attention(clean)
    o2, l2 = oracle.attention(dirty)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------ int8 with per-row scales

def test_int8_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch_decode(codes, "int8")
    assert np.array_equal(oracle.decode_bits(codes, "int8"), ref)
    assert oracle.decode_bits(np.array([0x80, 0x7F, 0xFF], np.uint8), "int8").tolist() == [-128.0, 127.0, -1.0]


@pytest.mark.parametrize("window", [0, 7])
def test_int8_row_scale_position_probe(window):
    """Q = 0 makes every visible score equal; V codes of 1 with row scale
    j + 1 (token j's own scale, set through its page and slot in the
    generator's live order) put the mean of j + 1 over the visible keys in
    every output column.  A scale taken from another page, slot or head
    breaks it."""
    s, ql, P = 100, 3, 16
    inp = _one(seq_lens=(s, 40), q_lens=(ql, 2), num_q_heads=4, num_kv_heads=2, kv_dtype="int8", q_dtype="bf16",
               page_size=P, window=window, pool_pages=30)
    inp.q[:] = 0
    inp.v_live[:] = 1
    n0 = (s + P - 1) // P
    for b, (sl, o0) in enumerate(((s, 0), (40, n0))):
        for j in range(sl):
            for g in range(2):
                inp.row_scale[1, o0 + j // P, g, j % P] = np.float32(j + 1 + 1000 * g + 500 * b)
    out, lse = oracle.attention(inp)
    t = 0
    for b, (sl, q) in enumerate(((s, ql), (40, 2))):
        for i in range(q):
            p = sl - q + i
            lo = max(0, p - window + 1) if window > 0 else 0
            for h in range(4):
                g = h // 2
                want = (lo + p) / 2 + 1 + 1000 * g + 500 * b
                np.testing.assert_allclose(out[t + i, h], want, rtol=0, atol=1e-10)
                assert lse[t + i, h] == pytest.approx(math.log(p - lo + 1), abs=1e-12)
        t += q


def test_int8_identical_rows_scale_the_score():
    """Every key the same int8 row c but with its own scale s_j: the scores
    are scale * s_j * (q . c), so the oracle's lse is the closed form
    log sum_j exp(scale * s_j * (q . c))."""
    n = 37
    inp = _one(seq_lens=(n,), q_lens=(1,), num_q_heads=2, num_kv_heads=1, kv_dtype="int8", q_dtype="bf16",
               head_dim=8)
    c = inp.k_live[0, 0, 0].copy()
    inp.k_live[:, 0, :, :] = c
    rng = np.random.default_rng(5)
    P = inp.page_size
    sj = rng.uniform(0.01, 0.3, n).astype(np.float32)
    for j in range(n):
        inp.row_scale[0, j // P, 0, j % P] = sj[j]
    _, lse = oracle.attention(inp)
    cv = oracle.decode_bits(c, "int8")
    for h in range(2):
        qv = torch_decode(inp.q[0, h], "bf16")
        dot = math.fsum(qv * cv)
        sc = [float(np.float32(inp.scale)) * float(x) * dot for x in sj]
        m = max(sc)
        want = m + math.log(math.fsum(math.exp(x - m) for x in sc))
        assert abs(lse[0, h] - want) < 1e-12


def test_int8_window_nan_poison_finite_and_unchanged():
    clean = _one(seq_lens=(130,), q_lens=(8,), window=20, pool_pages=64, kv_dtype="int8", q_dtype="bf16")
    dirty = _one(seq_lens=(130,), q_lens=(8,), window=20, pool_pages=64, kv_dtype="int8", q_dtype="bf16",
                 poison_out_of_window=True)
    n_dead = dirty.extra["poisoned_pages"][0][1]
    assert np.all(np.isnan(dirty.row_scale[:, :n_dead]))
    o1, l1 = oracle.attention(clean)
    o2, l2 = oracle.attention(dirty)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_int8_dequantisation_recovers_data():
    """code * row scale reproduces the float data within half a code step
    (scale / 2) on every live row."""
    inp = _one(seq_lens=(40,), q_lens=(1,), kv_dtype="int8", q_dtype="bf16", keep_float=True)
    for which, key in (("k", "k_float"), ("v", "v_float")):
        ref = inp.extra[key]
        for g in range(inp.num_kv_heads):
            got = oracle.depage(inp, which, 0, g, 0, 40)
            want = ref[:, g].reshape(-1, inp.head_dim)[:40].astype(np.float64)
            rs = inp.row_scale[0 if which == "k" else 1][:, g].reshape(-1)[:40].astype(np.float64)
            assert np.all(np.abs(got - want) <= rs[:, None] * 0.5 * (1 + 1e-6))
