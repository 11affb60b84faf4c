"""GPU parity of the cache append (paged_attn_append) against the oracle's
append, bit for bit over the whole K and V pools, through the C ABI."""
import zlib

import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from tests.gpu_helpers import progress

pytestmark = pytest.mark.gpu

P = 16
TORCH_16 = {"f16": "float16", "bf16": "bfloat16"}


def _bits16(x: np.ndarray, dtype: str) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(getattr(torch, TORCH_16[dtype]))
    return t.view(torch.int16).numpy().view(np.uint16)


def _case(rng, kv_dtype, in_dtype, hkv, D, seq_lens, q_lens, pages, width, scales="pow2"):
    T = int(np.sum(q_lens))
    x = rng.standard_normal((2, T, hkv, D)).astype(np.float32)
    scale = None
    if kv_dtype == "fp8_e4m3" and scales == "arbitrary":
        # scales as a quantiser derives them (any fp32 value): the quotient
        # x / s is inexact, so its single fp32 rounding decides many codes
        scale = rng.uniform(0.004, 0.05, (2, hkv)).astype(np.float32)
        x *= rng.uniform(0.5, 40.0, (1, 1, hkv, 1)).astype(np.float32)
    elif kv_dtype == "fp8_e4m3":
        # power-of-two scales keep the planted ties exact through the 16-bit
        # input and the fp32 quotient
        scale = rng.choice([0.125, 0.25, 0.5, 1.0, 2.0], (2, hkv)).astype(np.float32)
        # exact ties between neighbouring codes, values past 448 and NaN, after the scale
        table = oracle.fp8_e4m3_table()[:0x7F]
        mids = (table[:-1] + table[1:]) / 2
        flat = x.reshape(2, -1, hkv, D)
        for w in range(2):
            for g in range(hkv):
                sel = rng.random((flat.shape[1], D)) < 0.05
                pick = rng.choice(mids, size=int(sel.sum())) * rng.choice([-1, 1], size=int(sel.sum()))
                flat[w, :, g, :][sel] = pick * scale[w, g]
        x.reshape(-1)[rng.choice(x.size, 20, replace=False)] = 900.0
        x.reshape(-1)[rng.choice(x.size, 5, replace=False)] = np.nan
    bits = _bits16(x, in_dtype)                                   # [2][T][Hkv][D]
    st = np.uint8 if kv_dtype == "fp8_e4m3" else np.uint16
    pools = rng.integers(0, 1 << (8 * np.dtype(st).itemsize), (2, pages, hkv, P, D)).astype(st)
    bt = np.full((len(seq_lens), width), -7, dtype=np.int32)
    perm = rng.permutation(pages)
    k = 0
    for b, sl in enumerate(seq_lens):
        n = min(width, (int(sl) + P - 1) // P)
        bt[b, :n] = perm[k:k + n]
        k += n
    return bits, scale, pools, bt


CASES = {
    # decode rows of several sequences, one crossing into a new page, one empty
    "bf16_decode_batch": dict(kv="bf16", q="bf16", hkv=8, D=128, seq_lens=(17, 1, 4097, 33, 16), q_lens=(1, 1, 1, 0, 1)),
    "f16_verify_rows": dict(kv="f16", q="f16", hkv=8, D=128, seq_lens=(61, 9), q_lens=(8, 8)),
    "bf16_prefill_chunk": dict(kv="bf16", q="bf16", hkv=4, D=128, seq_lens=(700,), q_lens=(300,)),
    "fp8_from_bf16": dict(kv="fp8_e4m3", q="bf16", hkv=8, D=128, seq_lens=(40, 300, 5), q_lens=(8, 130, 5)),
    "fp8_from_f16_d64": dict(kv="fp8_e4m3", q="f16", hkv=2, D=64, seq_lens=(100, 31), q_lens=(16, 16)),
    # arbitrary fp32 scales and plain data (no planted ties)
    "fp8_from_bf16_any_scale": dict(kv="fp8_e4m3", q="bf16", hkv=8, D=128, seq_lens=(77, 1000, 16),
                                    q_lens=(8, 200, 16), scales="arbitrary"),
    "fp8_from_f16_any_scale": dict(kv="fp8_e4m3", q="f16", hkv=4, D=128, seq_lens=(500, 3), q_lens=(64, 3),
                                   scales="arbitrary"),
    # head_dim 256
    "bf16_d256": dict(kv="bf16", q="bf16", hkv=2, D=256, seq_lens=(33, 4097, 8), q_lens=(8, 1, 8)),
    "fp8_from_bf16_d256": dict(kv="fp8_e4m3", q="bf16", hkv=2, D=256, seq_lens=(70, 16), q_lens=(8, 16)),
    "fp8_from_f16_d256_any_scale": dict(kv="fp8_e4m3", q="f16", hkv=4, D=256, seq_lens=(300, 9), q_lens=(16, 9),
                                        scales="arbitrary"),
    # 40 KV heads: a row's 1,280 chunks take several passes of a workgroup
    "fp8_from_bf16_40_heads": dict(kv="fp8_e4m3", q="bf16", hkv=40, D=128, seq_lens=(300, 20), q_lens=(9, 3),
                                   scales="arbitrary"),
    "bf16_40_heads": dict(kv="bf16", q="bf16", hkv=40, D=128, seq_lens=(35, 70), q_lens=(5, 6)),
}


@pytest.mark.parametrize("layout", ["hnd", "nhd"])
@pytest.mark.parametrize("name", list(CASES))
def test_append_bit_exact(name, layout):
    import torch

    cs = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    seq_lens, q_lens = np.array(cs["seq_lens"], np.int32), np.array(cs["q_lens"], np.int32)
    pages = int(sum((s + P - 1) // P for s in seq_lens)) + 5
    width = max((int(s) + P - 1) // P for s in seq_lens) + 1
    bits, scale, pools, bt = _case(rng, cs["kv"], cs["q"], cs["hkv"], cs["D"], seq_lens, q_lens, pages, width,
                                   cs.get("scales", "pow2"))
    progress(f"append {name} {layout}: seqs={seq_lens.tolist()} q={q_lens.tolist()}")
    T = int(q_lens.sum())
    cfg = pal.make_config(cs["hkv"] * 4, cs["hkv"], cs["D"], cs["q"], cs["kv"], len(seq_lens), int(q_lens.max()),
                          max(T, 1))
    h = pal.paged_attn_create(cfg)
    try:
        dev = torch.device("cuda")
        tdt = torch.uint8 if cs["kv"] == "fp8_e4m3" else getattr(torch, TORCH_16[cs["kv"]])
        def pool(a):
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
            if tdt != torch.uint8:
                t = t.view(tdt)
            if layout == "nhd":
                t = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
            return t
        kc, vc = pool(pools[0]), pool(pools[1])
        qt = getattr(torch, TORCH_16[cs["q"]])
        kn = torch.from_numpy(bits[0].view(np.int16)).to(dev).view(qt).contiguous()
        vn = torch.from_numpy(bits[1].view(np.int16)).to(dev).view(qt).contiguous()
        ks = None if scale is None else torch.from_numpy(scale.reshape(-1)).to(dev)
        pal.paged_attn_append(h, kn, vn, kc, vc, torch.from_numpy(bt).to(dev), torch.from_numpy(seq_lens).to(dev),
                              torch.from_numpy(q_lens).to(dev), ks)
        torch.cuda.synchronize()
        def back(t):
            t = t.contiguous() if layout == "hnd" else t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3).contiguous()
            a = t.cpu()
            a = a.view(torch.int16).numpy().view(np.uint16) if tdt != torch.uint8 else a.numpy()
            return a
        got_k, got_v = back(kc), back(vc)
    finally:
        pal.paged_attn_destroy(h)
    bt_o = np.where(bt < 0, 0, bt)       # rows never reach the unset entries
    ref_k, ref_v = oracle.append_kv(bits[0], bits[1], cs["q"], pools[0], pools[1], cs["kv"], bt_o, seq_lens, q_lens,
                                    scale, P)
    assert np.array_equal(got_k, ref_k), f"K differs at {np.argwhere(got_k != ref_k)[:5].tolist()}"
    assert np.array_equal(got_v, ref_v), f"V differs at {np.argwhere(got_v != ref_v)[:5].tolist()}"


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast:RuntimeWarning")
@pytest.mark.parametrize("in_dtype,page_size", [("bf16", 16), ("f16", 48), ("bf16", 65520)])
def test_append_fp8_every_16bit_input(in_dtype, page_size):
    """Every 16-bit input value (all 65,536 bit patterns: zeros, subnormals,
    infinities, NaN of both signs) quantised to fp8 under scales from 2^-9 to
    17.3, bit for bit against the oracle: the fast quotient, its fallback to
    the exact one and the saturating conversion together reproduce the code of
    the once-rounded quotient for every value the input type can hold."""
    import torch

    hkv, D, T = 4, 128, 128
    rng = np.random.default_rng(zlib.crc32(f"every16{in_dtype}{page_size}".encode()))
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = np.stack([rng.permutation(allbits), rng.permutation(allbits)]).reshape(2, T, hkv, D)
    scale = np.array([[1.0, 0.0371, 2.0 ** -9, 17.3], [0.0071, 0.5, 3.3, 2.0 ** -5]], np.float32)
    seq_lens, q_lens = np.array([T + 37], np.int32), np.array([T], np.int32)
    pages = (int(seq_lens[0]) + page_size - 1) // page_size + 3
    width = pages
    bt = np.ascontiguousarray(rng.permutation(pages).astype(np.int32)[:width].reshape(1, width))
    pools = rng.integers(0, 256, (2, pages, hkv, page_size, D)).astype(np.uint8)
    progress(f"append every 16-bit {in_dtype} P{page_size}")
    cfg = pal.make_config(hkv * 4, hkv, D, in_dtype, "fp8_e4m3", 1, T, T, page_size=page_size)
    h = pal.paged_attn_create(cfg)
    try:
        dev = torch.device("cuda")
        kc, vc = (torch.from_numpy(pools[w]).to(dev) for w in range(2))
        qt = getattr(torch, TORCH_16[in_dtype])
        kn, vn = (torch.from_numpy(bits[w].view(np.int16)).to(dev).view(qt).contiguous() for w in range(2))
        pal.paged_attn_append(h, kn, vn, kc, vc, torch.from_numpy(bt).to(dev), torch.from_numpy(seq_lens).to(dev),
                              torch.from_numpy(q_lens).to(dev), torch.from_numpy(scale.reshape(-1)).to(dev))
        torch.cuda.synchronize()
        got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    finally:
        pal.paged_attn_destroy(h)
    ref_k, ref_v = oracle.append_kv(bits[0], bits[1], in_dtype, pools[0], pools[1], "fp8_e4m3", bt, seq_lens,
                                    q_lens, scale, page_size)
    assert np.array_equal(got_k, ref_k), f"K differs at {np.argwhere(got_k != ref_k)[:5].tolist()}"
    assert np.array_equal(got_v, ref_v), f"V differs at {np.argwhere(got_v != ref_v)[:5].tolist()}"


def test_append_skips_rows_outside_the_cache():
    """Rows whose page id is outside the pool, or whose position is past the
    block table, are not written; q_len > seq_len writes nothing."""
    import torch

    dev = torch.device("cuda")
    hkv, D, pages = 2, 128, 6
    cfg = pal.make_config(8, hkv, D, "f16", "f16", 3, 4, 12)
    h = pal.paged_attn_create(cfg)
    try:
        pool = torch.zeros((pages, hkv, P, D), dtype=torch.float16, device=dev)
        vpool = torch.zeros_like(pool)
        bt = torch.tensor([[0, 99], [1, -1], [2, 3]], dtype=torch.int32, device=dev)
        seq_lens = torch.tensor([20, 3, 40], dtype=torch.int32, device=dev)    # seq 2 past the table (2 pages)
        q_lens = torch.tensor([4, 4, 4], dtype=torch.int32, device=dev)        # seq 1: q_len > seq_len
        new = torch.ones((12, hkv, D), dtype=torch.float16, device=dev)
        pal.paged_attn_append(h, new, new, pool, vpool, bt, seq_lens, q_lens)
        torch.cuda.synchronize()
        written = (pool != 0).any(dim=(1, 3)).cpu().numpy()                   # [page][slot]
    finally:
        pal.paged_attn_destroy(h)
    expect = np.zeros((pages, P), dtype=bool)
    # seq 0: positions 16..19 -> block 1 = page 99: outside the pool, skipped
    # seq 1: nothing; seq 2: positions 36..39 -> block 2: past the table width, skipped
    assert np.array_equal(written, expect)


def _host_pool(inp, attr):
    arr = getattr(inp, attr)
    pool = np.full((inp.num_pages,) + arr.shape[1:], inp.fill_bits, dtype=arr.dtype)
    pool[inp.live_pages] = arr
    return pool


@pytest.mark.parametrize("kind", ["f16_verify", "fp8_mixed"])
def test_append_then_forward(kind):
    """The step a decode loop runs: the new rows' slots start out NaN, the
    append writes them, and the forward then reads them.  The pools after
    the append equal the oracle's append bit for bit, and the forward
    equals the oracle's attention over those pools."""
    import dataclasses

    import torch

    from synth import Spec, generate
    from synth.torch_upload import upload_batch, upload_pool
    from tests.gpu_helpers import compare

    if kind == "f16_verify":
        spec = Spec(name=kind, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=(3001, 650), q_lens=(8, 5),
                    q_dtype="f16", kv_dtype="f16", k_outlier_frac=0.01, seed=41)
    else:
        spec = Spec(name=kind, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=(9000, 2001, 300),
                    q_lens=(1, 4, 8), q_dtype="bf16", kv_dtype="fp8_e4m3", seed=42)
    inp = generate(spec)[0]
    T, hkv, D = inp.num_tokens, inp.num_kv_heads, inp.head_dim
    rng = np.random.default_rng(43)
    x = rng.standard_normal((2, T, hkv, D)).astype(np.float32)
    new_bits = _bits16(x, inp.q_dtype)
    # the cache before the step: the new rows' slots hold NaN
    pools_before = []
    for attr in ("k_live", "v_live"):
        pool = _host_pool(inp, attr)
        t = 0
        for b in range(inp.num_seqs):
            sl, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
            for p in range(sl - ql, sl):
                pool[inp.block_table[b, p // P], :, p % P, :] = inp.fill_bits
        pools_before.append(pool)
    ref_k, ref_v = oracle.append_kv(new_bits[0], new_bits[1], inp.q_dtype, pools_before[0], pools_before[1],
                                    inp.kv_dtype, inp.block_table, inp.seq_lens, inp.q_lens, inp.kv_scale, P)
    after = dataclasses.replace(inp, k_live=ref_k[inp.live_pages], v_live=ref_v[inp.live_pages])
    before = dataclasses.replace(inp, k_live=pools_before[0][inp.live_pages], v_live=pools_before[1][inp.live_pages])
    progress(f"append then forward {kind}: seqs={inp.seq_lens.tolist()} q={inp.q_lens.tolist()}")
    pools = upload_pool([before])
    d = upload_batch(before)
    qt = getattr(torch, TORCH_16[inp.q_dtype])
    kn = torch.from_numpy(new_bits[0].view(np.int16)).cuda().view(qt).contiguous()
    vn = torch.from_numpy(new_bits[1].view(np.int16)).cuda().view(qt).contiguous()
    cfg = pal.make_config(inp.num_q_heads, hkv, D, inp.q_dtype, inp.kv_dtype, inp.num_seqs, int(inp.q_lens.max()), T)
    h = pal.paged_attn_create(cfg)
    try:
        out = torch.full((T, inp.num_q_heads, D), float("nan"), device="cuda")
        lse = torch.full((T, inp.num_q_heads), float("nan"), device="cuda")
        pal.paged_attn_append(h, kn, vn, pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                              d["kv_scale"])
        pal.paged_attn_forward(h, d["q"], pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                               inp.window, inp.scale, d["kv_scale"], out, lse)
        torch.cuda.synchronize()
        got = [pools[w].cpu().numpy().view(np.uint8 if inp.kv_dtype == "fp8_e4m3" else np.uint16) for w in "kv"]
        o, l = out.cpu().numpy(), lse.cpu().numpy()
    finally:
        pal.paged_attn_destroy(h)
    assert np.array_equal(got[0], ref_k) and np.array_equal(got[1], ref_v)
    ref_o, ref_l = oracle.attention(after)
    compare(f"append then forward {kind}", inp.kv_dtype, o, l, ref_o, ref_l)


def test_append_host_argument_errors():
    """Host checks of paged_attn_append, through the C ABI directly: missing
    or unexpected kv_scale, misaligned rows, num_tokens outside the handle's
    range, NULL pointers.  Nothing is launched for a rejected call."""
    import ctypes

    import torch

    from paged_attention_long_amd import binding as B

    lib = pal.load_library()
    hkv, D, pages = 2, 128, 4
    dev = torch.device("cuda")
    for kv in ("fp8_e4m3", "bf16"):
        cfg = pal.make_config(8, hkv, D, "bf16", kv, 2, 4, 8)
        h = pal.paged_attn_create(cfg)
        try:
            st = torch.uint8 if kv == "fp8_e4m3" else torch.bfloat16
            kc = torch.zeros((pages, hkv, P, D), dtype=st, device=dev)
            layout = B.cache_layout(kc)
            new = torch.zeros((9, hkv, D), dtype=torch.bfloat16, device=dev)
            bt = torch.zeros((2, 2), dtype=torch.int32, device=dev)
            sl = torch.tensor([5, 3], dtype=torch.int32, device=dev)
            ql = torch.tensor([4, 3], dtype=torch.int32, device=dev)
            sc = torch.ones(2 * hkv, device=dev)
            good_scale = sc.data_ptr() if kv == "fp8_e4m3" else None
            bad_scale = None if kv == "fp8_e4m3" else sc.data_ptr()

            def call(k_new=new.data_ptr(), num_tokens=7, kv_scale=good_scale, k_cache=kc.data_ptr(),
                     block_table=bt.data_ptr()):
                return lib.paged_attn_append(h.ptr, k_new, new.data_ptr(), num_tokens, k_cache, kc.data_ptr(),
                                             ctypes.byref(layout), block_table, 2, 2, sl.data_ptr(), ql.data_ptr(),
                                             kv_scale, None)

            assert call() == B.PA_OK
            torch.cuda.synchronize()
            for kw in (dict(kv_scale=bad_scale), dict(k_new=new.data_ptr() + 2), dict(num_tokens=0),
                       dict(num_tokens=9), dict(k_new=None), dict(k_cache=None), dict(block_table=None)):
                rc = call(**kw)
                assert rc == B.PA_ERR_INVALID_ARGUMENT, (kv, kw, rc)
                assert pal.paged_attn_last_error(h) != ""
        finally:
            pal.paged_attn_destroy(h)
