"""GPU parity of the decode / verify path against the fp64 oracle, through
the C ABI (libpaged_attn.so).  Every input is seeded and synthetic."""
import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from synth import Spec, generate, named
from synth.gen import permute_pool
from tests.gpu_helpers import GpuCase, compare, progress

pytestmark = pytest.mark.gpu


def _spec(**kw):
    base = dict(name="case", num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=(1000,), q_lens=(1,),
                q_dtype="bf16", kv_dtype="bf16", seed=5)
    base.update(kw)
    return Spec(**base)


SMALL = {
    "bf16_g4_ragged": dict(seq_lens=(1000,), q_lens=(1,)),
    "f16_verify8_causal": dict(seq_lens=(777,), q_lens=(8,), q_dtype="f16", kv_dtype="f16"),
    "f16_verify8_window_poison": dict(seq_lens=(3000,), q_lens=(8,), q_dtype="f16", kv_dtype="f16", window=100,
                                      poison_out_of_window=True, k_outlier_frac=0.01),
    "f16_d64_multi": dict(num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=(257, 31, 600), q_lens=(1, 2, 1),
                          q_dtype="f16", kv_dtype="f16"),
    "fp8_mixed": dict(seq_lens=(2001, 1313, 333, 41), q_lens=(1, 4, 8, 1), kv_dtype="fp8_e4m3"),
    "fp8_f16q": dict(seq_lens=(999,), q_lens=(2,), q_dtype="f16", kv_dtype="fp8_e4m3"),
    "bf16_g6": dict(num_q_heads=24, num_kv_heads=4, seq_lens=(1234,), q_lens=(3,)),
    "f16_mha": dict(num_q_heads=4, num_kv_heads=4, seq_lens=(517,), q_lens=(1,), q_dtype="f16", kv_dtype="f16"),
    "bf16_g8": dict(num_q_heads=32, num_kv_heads=4, seq_lens=(2500,), q_lens=(1,)),
    # the largest group (16 query heads per KV head): 16 rows per token, so a
    # decode row set already takes the tile kernel and 4 new tokens fill its 64 rows
    "bf16_g16_decode": dict(num_q_heads=32, num_kv_heads=2, seq_lens=(3001, 40), q_lens=(1, 1)),
    "f16_g16_verify4": dict(num_q_heads=16, num_kv_heads=1, seq_lens=(2222,), q_lens=(4,), q_dtype="f16",
                            kv_dtype="f16", k_outlier_frac=0.01),
    "fp8_g16_mixed": dict(num_q_heads=32, num_kv_heads=2, seq_lens=(1800, 600), q_lens=(3, 1),
                          kv_dtype="fp8_e4m3"),
    "f16_d64_g16_max_rows": dict(num_q_heads=16, num_kv_heads=1, head_dim=64, seq_lens=(500, 90), q_lens=(4, 2),
                                 q_dtype="f16", kv_dtype="f16"),
    "bf16_d256_g16": dict(num_q_heads=16, num_kv_heads=1, head_dim=256, seq_lens=(1300,), q_lens=(2,)),
    # many KV heads, not a power of two, one query head each
    "f16_mha40": dict(num_q_heads=40, num_kv_heads=40, seq_lens=(900, 64), q_lens=(1, 8), q_dtype="f16",
                      kv_dtype="f16"),
    "qlen0_in_batch": dict(seq_lens=(300, 50, 129), q_lens=(2, 0, 1)),
    "all_new_rows": dict(seq_lens=(8, 5), q_lens=(8, 5), q_dtype="f16", kv_dtype="f16"),
    "single_token": dict(seq_lens=(1,), q_lens=(1,)),
    "window_1": dict(seq_lens=(400,), q_lens=(4,), window=1, poison_out_of_window=True),
    "window_wide": dict(seq_lens=(400,), q_lens=(4,), window=5000),
    "bf16_long_ragged_split": dict(seq_lens=(20007,), q_lens=(1,), num_kv_heads=2, num_q_heads=8),
    # a 4-row sequence past the VALU kernel's key limit (tile kernel) beside a short one (VALU kernel)
    "bf16_long_4row_and_short": dict(seq_lens=(17011, 300), q_lens=(1, 1), num_kv_heads=2, num_q_heads=8),
    # wide block table (both kernels launched) while every sequence is short (all on the VALU kernel)
    "wide_table_short_seqs": dict(seq_lens=(90, 17, 260), q_lens=(1, 1, 2), block_table_width=1500),
}

# More sequences than a workgroup has threads (the device plans loop over
# them), every row class, some with no new rows.
_rng = np.random.default_rng(77)
_MANY_Q = _rng.choice([0, 1, 1, 2, 4, 8], size=300)
_MANY_S = np.maximum(_MANY_Q, _rng.integers(1, 180, size=300))
SMALL["many_seqs_mixed_classes"] = dict(num_q_heads=8, num_kv_heads=2, seq_lens=tuple(int(x) for x in _MANY_S),
                                        q_lens=tuple(int(x) for x in _MANY_Q), q_dtype="f16", kv_dtype="f16")


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(name, mode):
    """mode: VALU-kernel split mode (0 automatic, 1 static, 2 device plan)."""
    inp = generate(_spec(name=name, **SMALL[name]))[0]
    progress(f"small parity {name} mode {mode}: seqs={inp.seq_lens.tolist()} q_lens={inp.q_lens.tolist()} "
             f"kv={inp.kv_dtype} D={inp.head_dim} G={inp.group} W={inp.window}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], split_mode=mode)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(name, inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("name", ["tiny_decode", "decode", "verify", "verify_window"])
def test_named_full(name):
    inp = named(name)[0]
    progress(f"named {name} full oracle")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp])
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(name, inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("path", [pal.PA_PATH_AUTO, pal.PA_PATH_VALU])
def test_mixed_fp8_full(path):
    """The 200k / 131k / 33k / 4k fp8 batch: all 14 tokens x 32 heads (448
    rows) element by element, on the automatic (tile kernel) and the VALU
    path."""
    inp = named("mixed_fp8")[0]
    progress(f"mixed_fp8 full oracle, path {path}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], path=path)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"mixed_fp8/path{path}", inp.kv_dtype, out, lse, ref_o, ref_l)


def test_window_nan_poison_bit_identical():
    """Every out-of-window page NaN: output finite and bit-identical to the
    same windowed run over clean pages ("Dual MI50, part 2", section "Bug 2")."""
    clean = named("verify_window", poison_out_of_window=False)[0]
    dirty = named("verify_window")[0]
    assert dirty.extra["poisoned_pages"] == [(0, 3712)]
    progress("window poison bit-identity")
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


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_page_permutation_bit_identical(kv):
    inp = generate(_spec(seq_lens=(3001, 77), q_lens=(1, 4), kv_dtype=kv, pool_pages=1000))[0]
    perm = permute_pool(inp, 9)
    progress(f"permutation bit-identity {kv}")
    c1, c2 = GpuCase([inp]), GpuCase([perm])
    try:
        o1, l1 = c1.run()
        o2, l2 = c2.run()
    finally:
        c1.close()
        c2.close()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


def test_deterministic_and_reusable():
    inp = generate(_spec(seq_lens=(5000, 123), q_lens=(2, 1)))[0]
    c = GpuCase([inp])
    try:
        o1, l1 = c.run()
        o2, l2 = c.run()
    finally:
        c.close()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("pps", [1, 4, 7, 100000])
def test_split_count_invariance(pps, mode):
    """Forcing the split size changes only the summation order."""
    inp = generate(_spec(seq_lens=(4097, 900), q_lens=(1, 3), q_dtype="f16", kv_dtype="f16"))[0]
    progress(f"split invariance pps={pps} mode={mode}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], path=pal.PA_PATH_VALU, pages_per_split=pps, split_mode=mode)
    try:
        out, lse = c.run()
    finally:
        c.close()
    compare(f"pps={pps}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("mode", [1, 2])
def test_rotating_batches_share_a_pool(mode):
    """Consecutive calls on different batches (split counters must reset)."""
    bs = generate(_spec(seq_lens=(2049,), q_lens=(1,)), batches=3)
    c = GpuCase(bs, path=pal.PA_PATH_VALU, split_mode=mode)
    try:
        for i, b in enumerate(bs):
            ref_o, ref_l = oracle.attention(b)
            out, lse = c.run(i)
            compare(f"batch{i}", b.kv_dtype, out, lse, ref_o, ref_l)
    finally:
        c.close()


def test_nhd_layout_through_strides():
    inp = generate(_spec(seq_lens=(1500,), q_lens=(2,)))[0]
    c1 = GpuCase([inp])
    c2 = GpuCase([inp], layout="nhd")
    try:
        assert c2.pools["k"].stride(2) == inp.num_kv_heads * inp.head_dim
        o1, l1 = c1.run()
        o2, l2 = c2.run()
    finally:
        c1.close()
        c2.close()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


GRAPH_CASES = {
    # static splits on 176 workgroups (VALU path): fixed merge slots
    "decode_merge_slots": dict(seq_lens=(4097,), q_lens=(1,)),
    # a single long decode sequence on the tile kernel, merged one row per unit
    "decode_tile_row_merge": dict(seq_lens=(4097,), q_lens=(1,)),
    # static splits on a small grid: merged inside the attention kernel
    "decode_in_kernel_merge": dict(seq_lens=(1003,), q_lens=(1,)),
    # verification width: tile kernel, published groups, merge launch
    "verify_merge_launch": dict(seq_lens=(3000,), q_lens=(8,), q_dtype="f16", kv_dtype="f16"),
    # a mixed fp8 batch: the one-round split plan, a merge grid past 64
    # workgroups (two-level arrival counters)
    "mixed_two_level_arrival": dict(seq_lens=(40001, 9004, 3000, 257), q_lens=(1, 4, 8, 1), kv_dtype="fp8_e4m3"),
    # prefill rows: ~1,000 merge workgroups on the two-level counters
    "prefill_merge_launch": dict(num_q_heads=24, num_kv_heads=4, seq_lens=(3000,), q_lens=(300,)),
    # head_dim 256 prefill on its tile kernel
    "d256_prefill": dict(num_q_heads=16, num_kv_heads=2, head_dim=256, seq_lens=(2500, 700), q_lens=(200, 9)),
}


GRAPH_TUNING = {"decode_merge_slots": dict(path=pal.PA_PATH_VALU)}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_graph_replay_matches_eager(name):
    """A captured forward replayed several times (eager work in between)
    equals the eager forward bit for bit: every counter and merge slot the
    forward uses is back at zero when it ends."""
    import torch

    inp = generate(_spec(**GRAPH_CASES[name]))[0]
    progress(f"graph replay {name}")
    c = GpuCase([inp], **GRAPH_TUNING.get(name, {}))
    try:
        eager_o, eager_l = c.run()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            c.forward(0, stream=s)          # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c.forward(0, stream=torch.cuda.current_stream())
        for rep in range(4):
            c.out[0].fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            o = c.out[0].cpu().numpy()
            l = c.lse[0].cpu().numpy()
            assert np.array_equal(o.view(np.uint32), eager_o.view(np.uint32)), f"replay {rep}"
            assert np.array_equal(l.view(np.uint32), eager_l.view(np.uint32)), f"replay {rep}"
    finally:
        c.close()


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3"])
def test_debug_gather_bit_exact(kv):
    import torch

    inp = generate(_spec(seq_lens=(333, 20, 1000), q_lens=(2, 1, 8), kv_dtype=kv, window=300,
                         q_dtype="f16", pool_pages=200))[0]
    c = GpuCase([inp])
    try:
        d = c.dev[0]
        P = inp.page_size
        n = sum(hi - lo for lo, hi in (inp.visible_range(b) for b in range(inp.num_seqs)))
        eb = 1 if kv == "fp8_e4m3" else 2
        slots = torch.full((n,), -1, dtype=torch.int64, device="cuda")
        rows = torch.zeros((n, inp.num_kv_heads, inp.head_dim * eb), dtype=torch.uint8, device="cuda")
        pal.paged_attn_debug_gather(c.h, c.pools["k"], d["block_table"], d["seq_lens"], d["q_lens"], inp.window,
                                    slots, rows)
        torch.cuda.synchronize()
        slots = slots.cpu().numpy()
        rows = rows.cpu().numpy()
    finally:
        c.close()
    # expected: generator's logical order (never through the block table)
    k = 0
    for b in range(inp.num_seqs):
        lo, hi = inp.visible_range(b)
        o0 = int(inp.page_offsets[b])
        for j in range(lo, hi):
            pg = o0 + j // P
            assert slots[k] == int(inp.live_pages[pg]) * P + j % P
            want = np.ascontiguousarray(inp.k_live[pg, :, j % P, :]).view(np.uint8).reshape(inp.num_kv_heads, -1)
            assert np.array_equal(rows[k], want), (b, j)
            k += 1
    assert k == n
    # the oracle's de-paging of sequence 0 decodes exactly these bytes
    lo, hi = inp.visible_range(0)
    for g in range(inp.num_kv_heads):
        raw = np.ascontiguousarray(rows[:hi - lo, g]).view(np.uint16 if eb == 2 else np.uint8)
        dec = oracle.decode_bits(raw, kv)
        if kv == "fp8_e4m3":
            dec = dec * float(inp.kv_scale[0][g])
        assert np.array_equal(dec, oracle.depage(inp, "k", 0, g, lo, hi))


def test_host_argument_errors():
    import torch

    inp = generate(_spec(seq_lens=(64,), q_lens=(1,)))[0]
    c = GpuCase([inp])
    try:
        d = c.dev[0]
        with pytest.raises(pal.PagedAttnError) as e:
            pal.paged_attn_forward(c.h, d["q"], c.pools["k"], c.pools["v"], d["block_table"], d["seq_lens"],
                                   d["q_lens"], 0, float("nan"), None, c.out[0], c.lse[0])
        assert e.value.code == 1
        with pytest.raises(pal.PagedAttnError):
            scale = torch.ones(2, 8, device="cuda")
            pal.paged_attn_forward(c.h, d["q"], c.pools["k"], c.pools["v"], d["block_table"], d["seq_lens"],
                                   d["q_lens"], 0, 0.1, scale, c.out[0], c.lse[0])
        with pytest.raises(pal.PagedAttnError):
            pal.paged_attn_set_tuning(c.h, grid=10 ** 7)
    finally:
        c.close()


def test_fixed_merge_slots_do_not_leak_between_forwards():
    """Static splits publish to fixed merge slots.  A (sequence, KV head) group
    merged from several splits, then the same group short enough for a single
    split on the same handle: the slot must have been emptied by the first
    merge, or the second forward's direct output would be overwritten."""
    long = generate(_spec(seq_lens=(4097,), q_lens=(1,)))[0]
    short = generate(_spec(seq_lens=(40,), q_lens=(1,), seed=9))[0]
    a = GpuCase([long], path=pal.PA_PATH_VALU, split_mode=1)
    b = GpuCase([short], handle=a.h)
    try:
        for i, (inp, case) in enumerate(((long, a), (short, b), (long, a), (short, b))):
            progress(f"fixed merge slots, forward {i}: seq_len {int(inp.seq_lens[0])}")
            ref_o, ref_l = oracle.attention(inp)
            out, lse = case.run()
            compare(f"forward{i}", inp.kv_dtype, out, lse, ref_o, ref_l)
    finally:
        b.close()
        a.close()


def test_static_splits_merged_in_kernel_and_through_slots():
    """Static splits of a small grid are merged inside the attention kernel by
    the last workgroup of each group to arrive; a larger grid goes through the
    fixed merge slots.  Both alternate on one handle, so the arrival counters
    and the slots must each be left clear by the forward that used them."""
    big = generate(_spec(seq_lens=(1000, 977, 1003, 640, 999, 1001, 850, 1003), q_lens=(1,) * 8))[0]
    small = generate(_spec(seq_lens=(1003,), q_lens=(1,), seed=9))[0]
    a = GpuCase([big], path=pal.PA_PATH_VALU, split_mode=1, pages_per_split=4)
    b = GpuCase([small], handle=a.h)
    try:
        for i, (inp, case) in enumerate(((big, a), (small, b), (small, b), (big, a), (small, b))):
            progress(f"static merges, forward {i}: {inp.num_seqs} sequences")
            ref_o, ref_l = oracle.attention(inp)
            out, lse = case.run()
            compare(f"forward{i}", inp.kv_dtype, out, lse, ref_o, ref_l)
    finally:
        b.close()
        a.close()


@pytest.mark.parametrize("q_len", [1, 3])
def test_in_kernel_merge_at_split_limit(q_len):
    """64 static splits per group (the most one merge reads) merged inside
    the attention kernel, rows spanning more than one merge pass; run twice
    on one handle, bit-identical."""
    inp = generate(_spec(num_q_heads=8, num_kv_heads=2, seq_lens=(4090,), q_lens=(q_len,), q_dtype="f16",
                         kv_dtype="f16", window=0))[0]
    progress(f"in-kernel merge at 64 splits, q_len {q_len}")
    ref_o, ref_l = oracle.attention(inp)
    c = GpuCase([inp], path=pal.PA_PATH_VALU, split_mode=1, pages_per_split=4)
    try:
        o1, l1 = c.run()
        o2, l2 = c.run()
    finally:
        c.close()
    compare("splits64", inp.kv_dtype, o1, l1, ref_o, ref_l)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
