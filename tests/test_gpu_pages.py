"""GPU parity at page sizes other than 16 tokens, through the C ABI.

The cache is read in place at any block size ("Dual MI50, part 2", section
"Prefill: teach the fork's fast kernel to read the int8 cache"); the pages'
own caches use 1,056-token pages ("tps-maxxing on amd gpu", section
"Baseline": a 4096-token prompt ran as 3168 + 928 tokens) and 1,584-token
blocks ("Dual MI50, part 2", section "Agent turns: stop re-reading what's
already cached").  Every kernel path runs at 32, 48, 64, 1,056 and 1,584
tokens per page against the fp64 oracle, which de-pages with its own
division by the page size."""
import dataclasses

import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from synth import Spec, generate
from tests.gpu_helpers import GpuCase, compare, progress

pytestmark = pytest.mark.gpu

PAGE_SIZES = [32, 48, 64, 1056, 1584]


def _spec(**kw):
    base = dict(name="pg", num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=(1000,), q_lens=(1,),
                q_dtype="bf16", kv_dtype="bf16", seed=91)
    base.update(kw)
    return Spec(**base)


CASES = {
    # decode rows: short contexts on the VALU kernel, the long one on the tile kernel
    "bf16_decode": (dict(seq_lens=(5000, 333, 20000), q_lens=(1, 1, 1)), [pal.PA_PATH_AUTO, pal.PA_PATH_VALU]),
    # verification widths, 16-bit tiles staged through registers; poisoned window
    "f16_verify_window": (dict(seq_lens=(7000,), q_lens=(8,), q_dtype="f16", kv_dtype="f16", window=900,
                               poison_out_of_window=True, k_outlier_frac=0.01),
                          [pal.PA_PATH_AUTO, pal.PA_PATH_VALU]),
    # fp8 tiles staged raw by asynchronous loads
    "fp8_mixed": (dict(seq_lens=(20001, 3000, 100), q_lens=(1, 4, 8), kv_dtype="fp8_e4m3", k_outlier_frac=0.01),
                  [pal.PA_PATH_AUTO, pal.PA_PATH_VALU]),
    # 256-row prefill items (the pipelined ring)
    "bf16_prefill": (dict(num_q_heads=24, num_kv_heads=4, seq_lens=(3000,), q_lens=(300,)), [pal.PA_PATH_AUTO]),
    # fp8 prefill on the 256-row pipelined ring (register-staged tiles)
    "fp8_prefill": (dict(num_q_heads=24, num_kv_heads=4, seq_lens=(2000, 700), q_lens=(100, 40),
                         kv_dtype="fp8_e4m3"), [pal.PA_PATH_AUTO]),
}


@pytest.mark.parametrize("page_size", PAGE_SIZES)
@pytest.mark.parametrize("name", list(CASES))
def test_page_size_parity(name, page_size):
    kw, paths = CASES[name]
    inp = generate(_spec(name=name, page_size=page_size, **kw))[0]
    ref_o, ref_l = oracle.attention(inp)
    for path in paths:
        progress(f"pages {page_size} {name} path {path}: seqs={inp.seq_lens.tolist()} q={inp.q_lens.tolist()}")
        c = GpuCase([inp], path=path)
        try:
            out, lse = c.run()
        finally:
            c.close()
        compare(f"P{page_size} {name}/path{path}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("page_size", [65520, 65536])
def test_largest_page_sizes(page_size):
    """The largest pages the ABI takes (65,536 tokens, and 65,520: 4,095
    16-token chunks, the largest divisor the kernels' multiply-high division
    covers): a sequence across two pages and a short one, decode and
    verification rows, on the default and the VALU-only paths."""
    inp = generate(_spec(page_size=page_size, num_q_heads=8, num_kv_heads=2, seq_lens=(70000, 3000), q_lens=(1, 8),
                         q_dtype="f16", kv_dtype="f16", seed=93))[0]
    ref_o, ref_l = oracle.attention(inp)
    for path in (pal.PA_PATH_AUTO, pal.PA_PATH_VALU):
        progress(f"pages {page_size} largest, path {path}")
        c = GpuCase([inp], path=path)
        try:
            out, lse = c.run()
        finally:
            c.close()
        compare(f"P{page_size} largest/path{path}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("page_size", [48, 1056])
def test_page_size_nhd_layout(page_size):
    """[pages][P][Hkv][D] storage seen through strides: the page stride is
    P * Hkv * D, a multiple of 16 token rows."""
    inp = generate(_spec(page_size=page_size, seq_lens=(4000, 600), q_lens=(8, 1), q_dtype="f16", kv_dtype="f16",
                         k_outlier_frac=0.01))[0]
    ref_o, ref_l = oracle.attention(inp)
    progress(f"pages {page_size} NHD")
    c = GpuCase([inp], layout="nhd")
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"P{page_size} nhd", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("page_size", [48, 1584])
def test_page_permutation_bit_identical(page_size):
    from synth.gen import permute_pool

    n_live = sum((s + page_size - 1) // page_size for s in (5000, 1200))
    inp = generate(_spec(page_size=page_size, seq_lens=(5000, 1200), q_lens=(8, 4), kv_dtype="fp8_e4m3",
                         pool_pages=2 * n_live + 3))[0]
    progress(f"pages {page_size} permutation")
    c1, c2 = GpuCase([inp]), GpuCase([permute_pool(inp, 9)])
    try:
        o1, l1 = c1.run()
        o2, l2 = c2.run()
    finally:
        c1.close()
        c2.close()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("page_size", [48, 1056])
def test_debug_gather_bit_exact(page_size):
    import torch

    inp = generate(_spec(page_size=page_size, seq_lens=(3000, 200), q_lens=(4, 1), window=1100,
                         poison_out_of_window=True))[0]
    c = GpuCase([inp])
    try:
        d = c.dev[0]
        n = sum(hi - lo for lo, hi in (inp.visible_range(b) for b in range(inp.num_seqs)))
        slots = torch.full((n,), -1, dtype=torch.int64, device="cuda")
        rows = torch.zeros((n, inp.num_kv_heads, inp.head_dim * 2), dtype=torch.uint8, device="cuda")
        pal.paged_attn_debug_gather(c.h, c.pools["k"], d["block_table"], d["seq_lens"], d["q_lens"], inp.window,
                                    slots, rows)
        torch.cuda.synchronize()
        got_slots, got_rows = slots.cpu().numpy(), rows.cpu().numpy()
    finally:
        c.close()
    P = inp.page_size
    k = 0
    for b in range(inp.num_seqs):
        lo, hi = inp.visible_range(b)
        for j in range(lo, hi):
            assert got_slots[k + j - lo] == int(inp.block_table[b, j // P]) * P + j % P
        for g in range(inp.num_kv_heads):
            raw = np.ascontiguousarray(got_rows[k:k + hi - lo, g]).view(np.uint16)
            assert np.array_equal(oracle.decode_bits(raw, inp.kv_dtype), oracle.depage(inp, "k", b, g, lo, hi))
        k += hi - lo


@pytest.mark.parametrize("page_size", [48, 1056])
def test_append_then_forward(page_size):
    """New rows written by the append at a page size of 48 or 1,056 tokens
    land where the oracle's append puts them (bit for bit over the pools)
    and the forward over them matches the oracle."""
    import torch

    from synth.torch_upload import upload_batch, upload_pool

    inp = generate(_spec(page_size=page_size, seq_lens=(2500, 97, 1057), q_lens=(8, 4, 1), kv_dtype="fp8_e4m3",
                         seed=92))[0]
    T, hkv, D, P = inp.num_tokens, inp.num_kv_heads, inp.head_dim, inp.page_size
    rng = np.random.default_rng(93)
    x = rng.standard_normal((2, T, hkv, D)).astype(np.float32)
    new_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pools_before = []
    for attr in ("k_live", "v_live"):
        arr = getattr(inp, attr)
        pool = np.full((inp.num_pages,) + arr.shape[1:], inp.fill_bits, dtype=arr.dtype)
        pool[inp.live_pages] = arr
        for b in range(inp.num_seqs):
            sl, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
            for p in range(sl - ql, sl):
                pool[inp.block_table[b, p // P], :, p % P, :] = inp.fill_bits
        pools_before.append(pool)
    ref_k, ref_v = oracle.append_kv(new_bits[0], new_bits[1], "bf16", pools_before[0], pools_before[1],
                                    inp.kv_dtype, inp.block_table, inp.seq_lens, inp.q_lens, inp.kv_scale, P)
    before = dataclasses.replace(inp, k_live=pools_before[0][inp.live_pages], v_live=pools_before[1][inp.live_pages])
    after = dataclasses.replace(inp, k_live=ref_k[inp.live_pages], v_live=ref_v[inp.live_pages])
    progress(f"pages {page_size} append then forward")
    pools = upload_pool([before])
    d = upload_batch(before)
    kn = torch.from_numpy(new_bits[0].view(np.int16)).cuda().view(torch.bfloat16).contiguous()
    vn = torch.from_numpy(new_bits[1].view(np.int16)).cuda().view(torch.bfloat16).contiguous()
    cfg = pal.make_config(inp.num_q_heads, hkv, D, "bf16", inp.kv_dtype, inp.num_seqs, int(inp.q_lens.max()), T,
                          page_size=P)
    h = pal.paged_attn_create(cfg)
    try:
        out = torch.full((T, inp.num_q_heads, D), float("nan"), device="cuda")
        lse = torch.full((T, inp.num_q_heads), float("nan"), device="cuda")
        pal.paged_attn_append(h, kn, vn, pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                              d["kv_scale"])
        pal.paged_attn_forward(h, d["q"], pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                               inp.window, inp.scale, d["kv_scale"], out, lse)
        torch.cuda.synchronize()
        got = [pools[w].cpu().numpy() for w in "kv"]
        o, l = out.cpu().numpy(), lse.cpu().numpy()
    finally:
        pal.paged_attn_destroy(h)
    assert np.array_equal(got[0], ref_k) and np.array_equal(got[1], ref_v)
    ref_o, ref_l = oracle.attention(after)
    compare(f"P{page_size} append then forward", inp.kv_dtype, o, l, ref_o, ref_l)
