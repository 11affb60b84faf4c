"""GPU parity of the MFMA tile path (chunked prefill and verification-width
rows) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from synth import Spec, generate, named
from tests.gpu_helpers import GpuCase, compare, progress

pytestmark = pytest.mark.gpu


def _spec(**kw):
    base = dict(name="pf", num_q_heads=24, num_kv_heads=4, head_dim=128, seq_lens=(1000,), q_lens=(200,),
                q_dtype="bf16", kv_dtype="bf16", seed=17)
    base.update(kw)
    return Spec(**base)


PREFILL = {
    "bf16_g6_chunk200": dict(),
    "bf16_all_new_130": dict(seq_lens=(130,), q_lens=(130,)),
    "f16_window50": dict(seq_lens=(777,), q_lens=(64,), q_dtype="f16", kv_dtype="f16", window=50,
                         poison_out_of_window=True),
    "fp8_prefill": dict(seq_lens=(1500, 300), q_lens=(40, 25), kv_dtype="fp8_e4m3"),
    "bf16_outliers": dict(seq_lens=(2000,), q_lens=(96,), k_outlier_frac=0.01),
    "f16_outliers_g4": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(3000,), q_lens=(48,), q_dtype="f16",
                            kv_dtype="f16", k_outlier_frac=0.01),
    "mixed_lengths": dict(seq_lens=(513, 70, 2049), q_lens=(33, 70, 5), num_q_heads=8, num_kv_heads=2),
    # head_dim 64 (VALU kernel only) at its limit of 64 rows per KV head
    "f16_d64_max_rows": dict(num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=(700, 16), q_lens=(16, 16),
                             q_dtype="f16", kv_dtype="f16"),
    "fp8_d64_window": dict(num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=(900,), q_lens=(16,),
                           kv_dtype="fp8_e4m3", window=120, poison_out_of_window=True, k_outlier_frac=0.01),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_small_parity(name):
    inp = generate(_spec(name=name, **PREFILL[name]))[0]
    progress(f"prefill {name}: seqs={inp.seq_lens.tolist()} q={inp.q_lens.tolist()} kv={inp.kv_dtype} "
             f"G={inp.group} W={inp.window}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(name, inp.kv_dtype, out, lse, ref_o, ref_l)


def test_prefill_named_sampled_rows():
    """The 2,048-token chunk on 65,536 cached tokens, checked on sampled rows
    (first, last and random tokens; every head of a few tokens)."""
    inp = named("prefill")[0]
    progress("prefill named sampled rows")
    rng = np.random.default_rng(3)
    toks = sorted(set([0, 1, 127, 128, 1023, 2046, 2047] + rng.choice(2048, 9, replace=False).tolist()))
    rows = []
    for t in toks:
        for h in rng.choice(inp.num_q_heads, size=4, replace=False):
            rows.append((int(t), int(h)))
    rows += [(2047, h) for h in range(inp.num_q_heads)]
    ref = oracle.attention_rows(inp, sorted(set(rows)))
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    compare("prefill", inp.kv_dtype, out, lse, None, None, rows=ref)


VERIFY = {
    "f16_q8": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(5000,), q_lens=(8,), q_dtype="f16", kv_dtype="f16",
                   k_outlier_frac=0.01),
    "f16_q8_window": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(5000,), q_lens=(8,), q_dtype="f16",
                          kv_dtype="f16", window=300, poison_out_of_window=True),
    "fp8_q4_q8": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(3000, 999), q_lens=(4, 8), kv_dtype="fp8_e4m3"),
    "bf16_q3_g6": dict(seq_lens=(1234,), q_lens=(3,)),
    # fp8 verification widths on the tile kernel: a poisoned window (dead
    # rows zeroed in the widened V buffer) and sequences of one and two tiles
    "fp8_q8_window": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(4000,), q_lens=(8,), kv_dtype="fp8_e4m3",
                          window=200, poison_out_of_window=True, k_outlier_frac=0.01),
    "fp8_short": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(20, 50, 33), q_lens=(8, 2, 4), kv_dtype="fp8_e4m3"),
}


@pytest.mark.parametrize("path", [pal.PA_PATH_AUTO, pal.PA_PATH_VALU, pal.PA_PATH_MFMA])
@pytest.mark.parametrize("name", list(VERIFY))
def test_paths_agree_with_oracle(name, path):
    inp = generate(_spec(name=name, **VERIFY[name]))[0]
    progress(f"verify {name} path={path}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], path=path)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"{name}/path{path}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("tps", [1, 3, 1000])
def test_tile_split_invariance(tps):
    inp = generate(_spec(seq_lens=(2500,), q_lens=(150,)))[0]
    progress(f"tile split tps={tps}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], kv_tiles_per_split=tps)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"tps={tps}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("tps", [1, 2, 3, 5])
def test_f16_verify_tile_split_invariance(tps):
    # verification widths on 16-bit caches (register-staged tiles): 1 .. 5
    # tiles per item give each wave zero, one or two tiles; outliers and a
    # window edge put dead rows and large scores inside the items
    inp = generate(_spec(num_q_heads=32, num_kv_heads=8, seq_lens=(2100, 700), q_lens=(8, 4), q_dtype="f16",
                         kv_dtype="f16", window=600, poison_out_of_window=True, k_outlier_frac=0.01))[0]
    progress(f"f16 verify tile split tps={tps}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], kv_tiles_per_split=tps, path=pal.PA_PATH_MFMA)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"f16 tps={tps}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("tps", [1, 2, 3, 5])
def test_fp8_tile_split_invariance(tps):
    # 1 .. 5 tiles per item: a wave gets zero, one or two tiles, so each of the
    # fp8 pipeline's endings (one step, an even and an odd count) is taken
    inp = generate(_spec(num_q_heads=32, num_kv_heads=8, seq_lens=(2100, 700), q_lens=(8, 4),
                         kv_dtype="fp8_e4m3"))[0]
    progress(f"fp8 tile split tps={tps}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], kv_tiles_per_split=tps, path=pal.PA_PATH_MFMA)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"fp8 tps={tps}", inp.kv_dtype, out, lse, ref_o, ref_l)


def test_mfma_deterministic():
    inp = generate(_spec(seq_lens=(3000,), q_lens=(100,)))[0]
    c = GpuCase([inp])
    try:
        o1, l1 = c.run()
        o2, l2 = c.run()
    finally:
        c.close()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
