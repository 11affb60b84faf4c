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
    # the largest group (16 query heads per KV head) in 256-row items
    "bf16_g16_chunk": dict(num_q_heads=32, num_kv_heads=2, seq_lens=(1400,), q_lens=(100,)),
    "fp8_g16_chunk": dict(num_q_heads=16, num_kv_heads=1, seq_lens=(900, 300), q_lens=(50, 20),
                          kv_dtype="fp8_e4m3"),
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


def test_prefill_named_dense_rows():
    """The 2,048-token chunk on 65,536 cached tokens: every 16th token and the
    last, with all 24 query heads (3,096 rows).  A 256-row item spans about
    43 tokens, so every item, and within it every split of the key range,
    reaches the comparison."""
    inp = named("prefill")[0]
    progress("prefill named dense rows")
    toks = sorted(set(list(range(0, 2048, 16)) + [1, 2047]))
    rows = [(t, h) for t in toks for h in range(inp.num_q_heads)]
    ref = oracle.attention_rows(inp, rows)
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    compare("prefill", inp.kv_dtype, out, lse, None, None, rows=ref)


def test_prefill_int8_named_dense_rows():
    """The same chunk on the int8 cache with per-row scales (the pipelined
    256-row loop on register-staged, widened tiles): every 16th token and the
    last, all 24 heads."""
    inp = named("prefill_int8")[0]
    progress("prefill int8 named dense rows")
    toks = sorted(set(list(range(0, 2048, 16)) + [1, 2047]))
    rows = [(t, h) for t in toks for h in range(inp.num_q_heads)]
    ref = oracle.attention_rows(inp, rows)
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    compare("prefill int8", inp.kv_dtype, out, lse, None, None, rows=ref)


def test_prefill_fp8_named_dense_rows():
    """The same chunk on an fp8 cache (per-head scales; tiles widened through
    registers into the pipelined ring): every 16th token and the last, all 24
    heads."""
    inp = named("prefill", kv_dtype="fp8_e4m3", seed=1009)[0]
    progress("prefill fp8 named dense rows")
    toks = sorted(set(list(range(0, 2048, 16)) + [1, 2047]))
    rows = [(t, h) for t in toks for h in range(inp.num_q_heads)]
    ref = oracle.attention_rows(inp, rows)
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    compare("prefill fp8", inp.kv_dtype, out, lse, None, None, rows=ref)


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
    # 9..16 new tokens at four query heads per KV head: 33..64 rows, two
    # 32-row tiles per (sequence, KV head) on the tile kernel (the 15 drafts
    # + 1 verification width of "tps-maxxing on amd gpu", section
    # "Speculative decoding: native MTP vs. DFlash")
    "f16_q16_window_outliers": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(5000,), q_lens=(16,), q_dtype="f16",
                                    kv_dtype="f16", window=700, poison_out_of_window=True, k_outlier_frac=0.01),
    "f16_q9_q16_outliers": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(7001, 2500), q_lens=(9, 16),
                                q_dtype="f16", kv_dtype="f16", k_outlier_frac=0.01),
    "bf16_q12_q16_window": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(6100, 900), q_lens=(12, 16),
                                window=1000, poison_out_of_window=True, k_outlier_frac=0.01),
    "bf16_q16_long": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(20011,), q_lens=(16,), k_outlier_frac=0.01),
    "fp8_q16_window_outliers": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(4500,), q_lens=(16,),
                                    kv_dtype="fp8_e4m3", window=900, poison_out_of_window=True, k_outlier_frac=0.01),
    "fp8_q9_q13_q16": dict(num_q_heads=32, num_kv_heads=8, seq_lens=(3000, 1200, 16), q_lens=(9, 13, 16),
                           kv_dtype="fp8_e4m3", k_outlier_frac=0.01),
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


def test_verify_named_on_valu_path():
    """The 61,448-token verification batch in full on the vector-ALU path
    (every sequence through the split-KV decode kernel)."""
    inp = named("verify")[0]
    progress("named verify full oracle, VALU path")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], path=pal.PA_PATH_VALU)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare("verify/valu", inp.kv_dtype, out, lse, ref_o, ref_l)


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


ROW_MERGE = {
    # head_dim 128 on the tile kernel: 128 tiles, two per split -> 64 splits
    "d128_tile_64_splits": (dict(num_q_heads=32, num_kv_heads=8, seq_lens=(4096,), q_lens=(8,), q_dtype="f16",
                                 kv_dtype="f16", k_outlier_frac=0.01), dict(kv_tiles_per_split=1)),
    # head_dim 64 and 256 on the VALU kernel with the device plan and small splits
    "d64_valu_planned": (dict(num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=(2000, 900), q_lens=(4, 16),
                              q_dtype="f16", kv_dtype="f16"), dict(split_mode=2, pages_per_split=2)),
    "d256_valu_planned": (dict(num_q_heads=16, num_kv_heads=2, head_dim=256, seq_lens=(1500, 60), q_lens=(2, 1),
                               kv_dtype="fp8_e4m3"), dict(split_mode=2, pages_per_split=2)),
    # many groups: every unit of a wide grid loops over several rows
    "d128_many_groups": (dict(num_q_heads=40, num_kv_heads=40, seq_lens=(3000, 2000, 900), q_lens=(8, 4, 2),
                              q_dtype="f16", kv_dtype="f16"), dict(path=pal.PA_PATH_MFMA, kv_tiles_per_split=2)),
}


@pytest.mark.parametrize("name", list(ROW_MERGE))
def test_row_merge_parity(name):
    """The one-row-per-unit merge launch (each row's splits spread over the
    workgroup's thread groups) at the 64-split limit, at head_dim 64 / 128 /
    256, and over a grid whose workgroups take several rows."""
    spec, tuning = ROW_MERGE[name]
    inp = generate(_spec(name=name, **spec))[0]
    progress(f"row merge {name}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], **tuning)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(name, inp.kv_dtype, out, lse, ref_o, ref_l)


def test_prefill_pipeline_unstaged_page_ids():
    """A prefill item longer than the page-id staging area (more than 2,041
    tiles of 32 keys in one split): the pipelined loop takes each tile's page
    ids from the block table directly, a step ahead of its loads."""
    inp = generate(_spec(num_q_heads=24, num_kv_heads=4, seq_lens=(70000,), q_lens=(64,), seed=23))[0]
    progress("prefill, one split of ~2,190 tiles (page ids not staged)")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], kv_tiles_per_split=100000)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare("unstaged page ids", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
def test_verify_item_unstaged_page_ids(kv):
    """A 32-row item longer than its page-id staging area (more than 511
    tiles in one split): the register-staged (16-bit) and raw-staged
    (one-byte) loops read each tile's page ids from the block table."""
    inp = generate(_spec(num_q_heads=32, num_kv_heads=8, seq_lens=(20000,), q_lens=(8,), q_dtype="f16",
                         kv_dtype=kv, k_outlier_frac=0.01, seed=29))[0]
    progress(f"verify width, one split of 625 tiles (page ids not staged), {kv}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], kv_tiles_per_split=100000, path=pal.PA_PATH_MFMA)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"unstaged verify {kv}", inp.kv_dtype, out, lse, ref_o, ref_l)
