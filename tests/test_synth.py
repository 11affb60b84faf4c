"""Seeded generator: determinism, page bookkeeping, poison placement, and the
algorithmic byte / flop counts of the named workloads."""
import numpy as np
import pytest

from synth import NAMED_SPECS, Spec, generate
from tests.oracle_helpers import torch_decode


def _small(**kw):
    base = dict(name="s", num_q_heads=4, num_kv_heads=2, head_dim=8, seq_lens=(37, 5), q_lens=(2, 1),
                page_size=4, seed=11)
    base.update(kw)
    return Spec(**base)


def test_same_seed_same_bytes():
    a = generate(_small())[0]
    b = generate(_small())[0]
    for f in ("k_live", "v_live", "q", "block_table", "live_pages"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = generate(_small(seed=12))[0]
    assert not np.array_equal(a.k_live, c.k_live)


def test_batches_use_disjoint_pages():
    bs = generate(_small(), batches=3)
    seen = set()
    for x in bs:
        s = set(x.live_pages.tolist())
        assert not (s & seen)
        seen |= s
        assert x.nan_page not in seen
    assert bs[0].nan_page == bs[1].nan_page


def test_tail_slots_and_padding_are_nan():
    x = generate(_small(seq_lens=(10, 3), q_lens=(1, 1), kv_dtype="bf16"))[0]
    k = torch_decode(x.k_live, "bf16")
    # seq 0: 10 tokens over 3 pages of 4 -> slots 2, 3 of page 2 dead
    assert np.all(np.isnan(k[2, :, 2:])) and np.all(np.isfinite(k[2, :, :2]))
    # seq 1: 3 tokens in its one page -> slot 3 dead
    assert np.all(np.isnan(k[3, :, 3:])) and np.all(np.isfinite(k[3, :, :3]))
    assert x.block_table[1, 1] == x.nan_page and x.block_table[1, 2] == x.nan_page


def test_window_poison_pages():
    x = generate(_small(seq_lens=(40,), q_lens=(3,), window=10, poison_out_of_window=True))[0]
    lo = 40 - 3 - 10 + 1     # 28 -> pages 0..6 fully before lo
    assert x.extra["poisoned_pages"] == [(0, lo // 4)]
    k = torch_decode(x.k_live, "f16")
    assert np.all(np.isnan(k[:7])) and np.all(np.isfinite(k[7:10]))


def test_fp8_codes_in_range():
    x = generate(_small(kv_dtype="fp8_e4m3", q_dtype="bf16"))[0]
    assert x.kv_scale.shape == (2, 2) and np.all(x.kv_scale > 0)
    vals = torch_decode(x.k_live, "fp8_e4m3")
    fin = vals[np.isfinite(vals)]
    assert np.abs(fin).max() == 448.0     # amax maps to the largest code


def test_int8_codes_and_row_scales():
    x = generate(_small(seq_lens=(37, 5), q_lens=(2, 1), kv_dtype="int8", q_dtype="bf16", window=10,
                        poison_out_of_window=True, keep_float=True))[0]
    assert x.kv_scale is None and x.row_scale.shape == (2,) + x.k_live.shape[:3]
    codes = x.k_live.view(np.int8)
    live = np.isfinite(x.row_scale[0])
    # live rows: codes in [-127, 127] and the row's largest |x| at +-127
    assert np.abs(codes[live].astype(int)).max() <= 127
    assert np.all(np.abs(codes[live].astype(int)).max(axis=-1) == 127)
    # dead rows (tail slots, the poisoned page): code -128 and a NaN scale
    assert np.all(codes[~live] == -128)
    n_dead = x.extra["poisoned_pages"][0][1]
    assert np.all(np.isnan(x.row_scale[:, :n_dead]))
    assert np.isnan(x.row_scale[0, 2, :, 37 % 4:]).all()   # sequence 0 ends inside its last page


def test_outlier_positions():
    x = generate(_small(seq_lens=(200,), q_lens=(1,), k_outlier_frac=0.01, keep_float=True))[0]
    pos = x.extra["outliers"][0]
    assert len(pos) == 2 and len(set(pos.tolist())) == 2


# Algorithmic sizes of the named workloads, worked by hand:
#   decode: 4,097 tokens x 8 KV heads x 128 x 2 B x (K+V) = 16,781,312 B
#   verify: 61,448 tokens, same shape, fp16            = 251,691,008 B
#   verify_window: tokens 59,393..61,447 (2,055)        =   8,417,280 B
#   prefill: 67,584 x 4 x 128 x 2 x 2                   = 138,412,032 B
#   mixed_fp8: 367,950 x 8 x 128 x 1 x 2                = 753,561,600 B
#   mixed_int8: 367,950 x 8 x (128 x 1 + 4) x 2         = 777,110,400 B (codes + row scales)
@pytest.mark.parametrize("name,kv_bytes", [
    ("tiny_decode", 257 * 1 * 64 * 2 * 2),
    ("decode", 16_781_312),
    ("verify", 251_691_008),
    ("verify_window", 8_417_280),
    ("prefill", 138_412_032),
    ("mixed_fp8", 753_561_600),
    ("mixed_int8", 777_110_400),
    ("prefill_d256", 138_412_032),
    ("prefill_int8", 2 * 67_584 * 4 * (128 + 4)),
])
def test_named_kv_bytes(name, kv_bytes):
    spec = NAMED_SPECS[name]

    class Meta:  # metadata only: avoids drawing the big arrays
        pass

    from synth.gen import PagedInputs
    m = PagedInputs.__new__(PagedInputs)
    m.seq_lens = np.array(spec.seq_lens)
    m.q_lens = np.array(spec.q_lens)
    m.window = spec.window
    m.num_kv_heads = spec.num_kv_heads
    m.num_q_heads = spec.num_q_heads
    m.head_dim = spec.head_dim
    m.kv_dtype = spec.kv_dtype
    assert m.kv_bytes() == kv_bytes


def test_prefill_flops():
    from synth.gen import PagedInputs
    spec = NAMED_SPECS["prefill"]
    m = PagedInputs.__new__(PagedInputs)
    m.seq_lens = np.array(spec.seq_lens)
    m.q_lens = np.array(spec.q_lens)
    m.window = 0
    m.num_q_heads, m.head_dim = 24, 128
    # pairs: sum over i of (65,536 + i + 1) for i < 2048 = 2048*65,536 + 2048*2049/2
    pairs = 2048 * 65536 + 2048 * 2049 // 2
    assert m.pair_count() == pairs
    assert m.flops() == 4 * 128 * 24 * pairs       # 1,675.05 GF
    assert abs(m.flops() / 1e9 - 1675.05) < 0.01


def test_prefill_d256_flops():
    from synth.gen import PagedInputs
    spec = NAMED_SPECS["prefill_d256"]
    m = PagedInputs.__new__(PagedInputs)
    m.seq_lens = np.array(spec.seq_lens)
    m.q_lens = np.array(spec.q_lens)
    m.window = 0
    m.num_q_heads, m.head_dim = 16, 256
    pairs = 2048 * 65536 + 2048 * 2049 // 2
    assert m.pair_count() == pairs
    assert m.flops() == 4 * 256 * 16 * pairs       # 2,233.4 GF
