"""GPU parity of the int8 cache with one fp32 scale per cached row (the
pages' own cache format, "Dual MI50, part 2", section "Prefill: teach the
fork's fast kernel to read the int8 cache"), through the C ABI, against the
fp64 oracle that de-pages every row with its own scale."""
import dataclasses
import zlib

import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from synth import Spec, generate, named
from tests.gpu_helpers import GpuCase, compare, progress

pytestmark = pytest.mark.gpu


def _spec(**kw):
    base = dict(name="i8", num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=(1000,), q_lens=(1,),
                q_dtype="bf16", kv_dtype="int8", seed=61)
    base.update(kw)
    return Spec(**base)


CASES = {
    # decode rows (VALU kernel), a long one (tile kernel), a 3-row sequence
    "decode_batch": dict(seq_lens=(5000, 333, 20011, 17), q_lens=(1, 1, 1, 3), k_outlier_frac=0.01),
    "f16q_decode": dict(seq_lens=(3001,), q_lens=(2,), q_dtype="f16"),
    # verification widths (32-row tiles, raw staging) with a poisoned window
    "verify8_window": dict(seq_lens=(7000,), q_lens=(8,), window=900, poison_out_of_window=True, k_outlier_frac=0.01),
    "verify16_mixed": dict(seq_lens=(4000, 1200, 16), q_lens=(16, 9, 16), k_outlier_frac=0.01),
    "f16q_verify": dict(seq_lens=(2500, 50), q_lens=(8, 4), q_dtype="f16", window=300, poison_out_of_window=True),
    # prefill widths (256-row items, tiles widened into the pipelined ring)
    "prefill_g6": dict(num_q_heads=24, num_kv_heads=4, seq_lens=(3000,), q_lens=(300,), k_outlier_frac=0.01),
    "prefill_window_f16q": dict(num_q_heads=24, num_kv_heads=4, seq_lens=(2000, 700), q_lens=(100, 40),
                                q_dtype="f16", window=500, poison_out_of_window=True),
    # head_dim 64 (VALU kernel)
    "d64": dict(num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=(900, 31), q_lens=(4, 1)),
}

PATHS = {"auto": pal.PA_PATH_AUTO, "valu": pal.PA_PATH_VALU, "mfma": pal.PA_PATH_MFMA}


def _paths(name):
    if name.startswith("prefill"):
        return ["auto"]
    if name == "d64":
        return ["auto"]
    return ["auto", "valu", "mfma"]


@pytest.mark.parametrize("name", list(CASES))
def test_int8_parity(name):
    inp = generate(_spec(name=name, **CASES[name]))[0]
    ref_o, ref_l = oracle.attention(inp)
    for path in _paths(name):
        progress(f"int8 {name} path {path}: seqs={inp.seq_lens.tolist()} q={inp.q_lens.tolist()} W={inp.window}")
        c = GpuCase([inp], path=PATHS[path])
        try:
            out, lse = c.run()
        finally:
            c.close()
        compare(f"int8 {name}/{path}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("page_size", [48, 1584])
@pytest.mark.parametrize("layout", ["hnd", "nhd"])
def test_int8_page_sizes_and_layouts(page_size, layout):
    inp = generate(_spec(page_size=page_size, seq_lens=(6000, 800, 100), q_lens=(1, 8, 40), num_q_heads=16,
                         num_kv_heads=4, window=2000, poison_out_of_window=True, k_outlier_frac=0.01))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"int8 P{page_size} {layout}")
    c = GpuCase([inp], layout=layout)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"int8 P{page_size} {layout}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("tps", [1, 2, 3, 5])
def test_int8_tile_split_invariance(tps):
    inp = generate(_spec(seq_lens=(2100, 700), q_lens=(8, 4), k_outlier_frac=0.01))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"int8 tile split tps={tps}")
    c = GpuCase([inp], kv_tiles_per_split=tps, path=pal.PA_PATH_MFMA)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"int8 tps={tps}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("path", [pal.PA_PATH_AUTO, pal.PA_PATH_VALU])
def test_mixed_int8_full(path):
    """The 200k / 131k / 33k / 4k batch on an int8 cache: all 448 rows."""
    inp = named("mixed_int8")[0]
    progress(f"mixed_int8 full oracle, path {path}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], path=path)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"mixed_int8/path{path}", inp.kv_dtype, out, lse, ref_o, ref_l)


def test_int8_nan_scale_poison_bit_identical():
    """Out-of-window rows with NaN scales (and code -128) change nothing."""
    clean = generate(_spec(seq_lens=(9000,), q_lens=(8,), window=2048))[0]
    dirty = generate(_spec(seq_lens=(9000,), q_lens=(8,), window=2048, poison_out_of_window=True))[0]
    assert dirty.extra["poisoned_pages"]
    c1, c2 = GpuCase([clean]), GpuCase([dirty])
    try:
        o1, l1 = c1.run()
        o2, l2 = c2.run()
    finally:
        c1.close()
        c2.close()
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("in_dtype,page_size,D", [("bf16", 16, 128), ("f16", 48, 128), ("bf16", 16, 64),
                                                   ("bf16", 48, 256), ("f16", 16, 256)])
def test_int8_append_bit_exact_then_forward(in_dtype, page_size, D):
    """The append quantises each new row (scale amax/127, nearest integer,
    ties to even) bit for bit as the oracle does, codes and scales, over the
    whole pools; the forward over the appended rows matches the oracle.
    Rows include zeros, exact ties, a NaN and an infinity."""
    import torch

    from synth.torch_upload import upload_batch, upload_pool

    hq, hkv = {128: (32, 8), 64: (8, 2), 256: (16, 2)}[D]
    inp = generate(_spec(page_size=page_size, head_dim=D, num_q_heads=hq, num_kv_heads=hkv, q_dtype=in_dtype,
                         seq_lens=(2500, 97, 33), q_lens=(8, 4, 1), seed=62))[0]
    T, P = inp.num_tokens, inp.page_size
    rng = np.random.default_rng(zlib.crc32(f"{in_dtype}{page_size}{D}".encode()))
    x = (rng.standard_normal((2, T, hkv, D)) * rng.uniform(0.1, 30.0, (2, T, hkv, 1))).astype(np.float32)
    x[0, 0, 0, :] = 0.0                                         # a zero row
    x[1, 1, 0, :4] = [127.0, 0.5, 1.5, -2.5]                     # amax 127: scale 1, exact ties
    x[1, 1, 0, 4:] = 0.25
    x[0, 2, 1, 3] = np.nan                                      # rows with a non-finite value
    x[1, 3, 0, 5] = np.inf
    tt = getattr(torch, {"bf16": "bfloat16", "f16": "float16"}[in_dtype])
    new_bits = torch.from_numpy(x).to(tt).view(torch.int16).numpy().view(np.uint16)
    pools_before, scales_before = [], None
    for attr in ("k_live", "v_live"):
        arr = getattr(inp, attr)
        pool = np.full((inp.num_pages,) + arr.shape[1:], inp.fill_bits, dtype=arr.dtype)
        pool[inp.live_pages] = arr
        pools_before.append(pool)
    rs = np.full((2, inp.num_pages, hkv, P), np.nan, dtype=np.float32)
    rs[:, inp.live_pages] = inp.row_scale
    for b in range(inp.num_seqs):
        sl, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
        for p in range(sl - ql, sl):
            for w in range(2):
                pools_before[w][inp.block_table[b, p // P], :, p % P, :] = inp.fill_bits
            rs[:, inp.block_table[b, p // P], :, p % P] = np.nan
    ref_k, ref_v, ref_rs = oracle.append_kv(new_bits[0], new_bits[1], in_dtype, pools_before[0], pools_before[1],
                                            "int8", inp.block_table, inp.seq_lens, inp.q_lens, None, P, row_scale=rs)
    before = dataclasses.replace(inp, k_live=pools_before[0][inp.live_pages], v_live=pools_before[1][inp.live_pages],
                                 row_scale=rs[:, inp.live_pages])
    after = dataclasses.replace(inp, k_live=ref_k[inp.live_pages], v_live=ref_v[inp.live_pages],
                                row_scale=ref_rs[:, inp.live_pages])
    progress(f"int8 append {in_dtype} P{page_size} D{D}")
    pools = upload_pool([before])
    d = upload_batch(before)
    kn = torch.from_numpy(new_bits[0].view(np.int16)).cuda().view(tt).contiguous()
    vn = torch.from_numpy(new_bits[1].view(np.int16)).cuda().view(tt).contiguous()
    cfg = pal.make_config(hq, hkv, D, in_dtype, "int8", inp.num_seqs, int(inp.q_lens.max()), T, page_size=P)
    h = pal.paged_attn_create(cfg)
    try:
        pal.paged_attn_append(h, kn, vn, pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                              pools["row_scale"])
        torch.cuda.synchronize()
        got_k, got_v = pools["k"].cpu().numpy(), pools["v"].cpu().numpy()
        got_rs = pools["row_scale"].cpu().numpy()
    finally:
        pal.paged_attn_destroy(h)
    assert np.array_equal(got_k, ref_k), f"K codes differ at {np.argwhere(got_k != ref_k)[:5].tolist()}"
    assert np.array_equal(got_v, ref_v), f"V codes differ at {np.argwhere(got_v != ref_v)[:5].tolist()}"
    same = (got_rs == ref_rs) | (np.isnan(got_rs) & np.isnan(ref_rs))
    assert same.all(), f"row scales differ at {np.argwhere(~same)[:5].tolist()}"
    # The forward reads appended rows of the workloads' N(0,1) magnitude (the
    # out bound is absolute: the wide rows above, |V| up to ~100, are for the
    # quantiser), all finite (a NaN row scale makes its key NaN).
    x2 = rng.standard_normal((2, T, hkv, D)).astype(np.float32)
    x2[0, 0, 0, :] = 0.0
    nb2 = torch.from_numpy(x2).to(tt).view(torch.int16).numpy().view(np.uint16)
    ref_k2, ref_v2, ref_rs2 = oracle.append_kv(nb2[0], nb2[1], in_dtype, pools_before[0], pools_before[1], "int8",
                                               inp.block_table, inp.seq_lens, inp.q_lens, None, P, row_scale=rs)
    after = dataclasses.replace(inp, k_live=ref_k2[inp.live_pages], v_live=ref_v2[inp.live_pages],
                                row_scale=ref_rs2[:, inp.live_pages])
    pools = upload_pool([before])
    kn = torch.from_numpy(nb2[0].view(np.int16)).cuda().view(tt).contiguous()
    vn = torch.from_numpy(nb2[1].view(np.int16)).cuda().view(tt).contiguous()
    h = pal.paged_attn_create(cfg)
    try:
        out = torch.full((T, hq, D), float("nan"), device="cuda")
        lse = torch.full((T, hq), float("nan"), device="cuda")
        pal.paged_attn_append(h, kn, vn, pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                              pools["row_scale"])
        pal.paged_attn_forward(h, d["q"], pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                               inp.window, inp.scale, pools["row_scale"], out, lse)
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
    finally:
        pal.paged_attn_destroy(h)
    ref_o, ref_l = oracle.attention(after)
    compare(f"int8 append then forward {in_dtype} P{page_size} D{D}", "int8", o, l, ref_o, ref_l)
