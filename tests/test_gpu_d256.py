"""GPU parity at head_dim 256 through the C ABI, against the fp64 oracle.

The dense models of the pages' prefill measurements use 256-wide heads
("Strix Halo dense cliff patch attribution", section "Which patch, and how I
know").  At this width the library runs decode and verification widths (up
to 64 query rows per KV head) on the VALU kernel: a token row is 32 lanes of
8 elements, two tokens per wavefront load round.  Past 64 rows (chunked
prefill) a tile kernel on the matrix cores with 128-row items takes the
sequences of more than 8 rows.  Every KV format, page size and split mode of
both kernels runs here."""
import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from synth import Spec, generate
from tests.gpu_helpers import GpuCase, compare, progress

pytestmark = pytest.mark.gpu


def _spec(**kw):
    base = dict(name="d256", num_q_heads=16, num_kv_heads=2, head_dim=256, seq_lens=(1000,), q_lens=(1,),
                q_dtype="bf16", kv_dtype="bf16", seed=71)
    base.update(kw)
    return Spec(**base)


CASES = {
    # decode rows of a batch (8 query heads per KV head), one 3-row sequence
    "bf16_decode_batch": dict(seq_lens=(5000, 333, 20011, 17), q_lens=(1, 1, 1, 3), k_outlier_frac=0.01),
    # 8 tokens x 8 heads = 64 rows per KV head, causal, poisoned window
    "f16_verify8_window": dict(seq_lens=(7000, 600), q_lens=(8, 8), q_dtype="f16", kv_dtype="f16", window=900,
                               poison_out_of_window=True, k_outlier_frac=0.01),
    # 16 tokens x 4 heads (the 15-draft + 1 verification width)
    "bf16_verify16_g4": dict(num_q_heads=16, num_kv_heads=4, seq_lens=(4000, 1200, 16), q_lens=(16, 9, 16)),
    "fp8_mixed": dict(seq_lens=(20001, 3000, 100), q_lens=(1, 4, 8), kv_dtype="fp8_e4m3", k_outlier_frac=0.01),
    "int8_mixed": dict(seq_lens=(20001, 3000, 100), q_lens=(1, 4, 8), kv_dtype="int8", k_outlier_frac=0.01),
    "int8_f16q_window": dict(seq_lens=(9000,), q_lens=(4,), q_dtype="f16", kv_dtype="int8", window=2000,
                             poison_out_of_window=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_d256_parity(name):
    inp = generate(_spec(name=name, **CASES[name]))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"d256 {name}: seqs={inp.seq_lens.tolist()} q={inp.q_lens.tolist()} W={inp.window}")
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"d256 {name}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("page_size,layout", [(48, "hnd"), (1056, "nhd"), (1584, "hnd")])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_d256_page_sizes(page_size, layout, kv):
    inp = generate(_spec(page_size=page_size, kv_dtype=kv, seq_lens=(6000, 800), q_lens=(1, 8), k_outlier_frac=0.01,
                         window=2500, poison_out_of_window=True))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"d256 P{page_size} {layout} {kv}")
    c = GpuCase([inp], layout=layout)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"d256 P{page_size} {layout} {kv}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("split_mode,pps", [(1, 4), (1, 12), (1, 64), (2, 0), (2, 4), (2, 40)])
def test_d256_split_invariance(split_mode, pps):
    """Static splits (one sequence: with the in-kernel merge of small grids or
    fixed merge slots) and planned splits, several split sizes: all within
    tolerance of the oracle."""
    inp = generate(_spec(seq_lens=(12000,), q_lens=(4,), kv_dtype="fp8_e4m3", k_outlier_frac=0.01))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"d256 split_mode {split_mode} pages_per_split {pps}")
    c = GpuCase([inp], split_mode=split_mode, pages_per_split=pps)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"d256 mode{split_mode} pps{pps}", inp.kv_dtype, out, lse, ref_o, ref_l)


def test_d256_page_permutation_bit_identical():
    from synth.gen import permute_pool

    inp = generate(_spec(seq_lens=(5000, 1200), q_lens=(8, 4), kv_dtype="int8", pool_pages=800))[0]
    progress("d256 permutation")
    c1, c2 = GpuCase([inp]), GpuCase([permute_pool(inp, 9)])
    try:
        o1, l1 = c1.run()
        o2, l2 = c2.run()
    finally:
        c1.close()
        c2.close()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


PREFILL = {
    # 300 tokens x 8 heads = 2,400 rows per KV head: 19 row blocks, the last ragged
    "bf16_prefill": dict(seq_lens=(3000,), q_lens=(300,), k_outlier_frac=0.01),
    "f16_prefill_window": dict(seq_lens=(2500, 900), q_lens=(100, 40), q_dtype="f16", kv_dtype="f16", window=500,
                               poison_out_of_window=True),
    "fp8_prefill_g4": dict(num_q_heads=16, num_kv_heads=4, seq_lens=(2000, 700), q_lens=(100, 40),
                           kv_dtype="fp8_e4m3", k_outlier_frac=0.01),
    "int8_prefill": dict(seq_lens=(1800,), q_lens=(130,), kv_dtype="int8", k_outlier_frac=0.01),
    "int8_f16q_prefill_window": dict(seq_lens=(2200,), q_lens=(64,), q_dtype="f16", kv_dtype="int8", window=300,
                                     poison_out_of_window=True),
    # prefill rows next to decode and verification rows: both kernels in one forward
    "bf16_mixed_batch": dict(seq_lens=(4000, 1500, 333, 70), q_lens=(1, 200, 8, 70), k_outlier_frac=0.01),
    "fp8_mixed_batch": dict(seq_lens=(20001, 3000, 100), q_lens=(1, 40, 9), kv_dtype="fp8_e4m3"),
    # a window narrower than one 32-key tile
    "bf16_window_16": dict(seq_lens=(1000,), q_lens=(90,), window=16, poison_out_of_window=True),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_d256_prefill_parity(name):
    inp = generate(_spec(name=name, **PREFILL[name]))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"d256 prefill {name}: seqs={inp.seq_lens.tolist()} q={inp.q_lens.tolist()} W={inp.window}")
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"d256 prefill {name}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8_e4m3", "int8"])
def test_d256_tile_kernel_at_few_rows(kv):
    """PA_PATH_MFMA sends decode and verification rows through the tile
    kernel as well (one 128-row item with 1 to 64 live rows)."""
    q = "f16" if kv == "f16" else "bf16"
    inp = generate(_spec(seq_lens=(5000, 333, 17), q_lens=(1, 8, 3), q_dtype=q, kv_dtype=kv, window=1200,
                         poison_out_of_window=True, k_outlier_frac=0.01))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"d256 tile kernel few rows {kv}")
    c = GpuCase([inp], path=pal.PA_PATH_MFMA)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"d256 tile few rows {kv}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("tps", [1, 2, 3, 7])
def test_d256_tile_split_invariance(tps):
    inp = generate(_spec(seq_lens=(2100, 700), q_lens=(80, 20), kv_dtype="bf16", k_outlier_frac=0.01))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"d256 tile split tps={tps}")
    c = GpuCase([inp], kv_tiles_per_split=tps)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"d256 tile tps={tps}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("page_size,layout", [(48, "nhd"), (1056, "hnd")])
def test_d256_prefill_page_sizes(page_size, layout):
    inp = generate(_spec(page_size=page_size, seq_lens=(3000, 500), q_lens=(120, 9), kv_dtype="fp8_e4m3",
                         k_outlier_frac=0.01))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"d256 prefill P{page_size} {layout}")
    c = GpuCase([inp], layout=layout)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"d256 prefill P{page_size} {layout}", inp.kv_dtype, out, lse, ref_o, ref_l)


def test_d256_prefill_long_context():
    """512 new tokens after 7,680 cached ones, 16 query heads over 2 KV heads
    (4,096 rows per KV head, 32 row blocks): every row against the oracle."""
    inp = generate(_spec(seq_lens=(8192,), q_lens=(512,), k_outlier_frac=0.01, seed=72))[0]
    progress("d256 prefill long context (oracle)")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare("d256 prefill long", inp.kv_dtype, out, lse, ref_o, ref_l)
