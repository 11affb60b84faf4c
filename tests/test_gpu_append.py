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


def _case(rng, kv_dtype, in_dtype, hkv, D, seq_lens, q_lens, pages, width):
    T = int(np.sum(q_lens))
    x = rng.standard_normal((2, T, hkv, D)).astype(np.float32)
    scale = None
    if kv_dtype == "fp8_e4m3":
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
    bits, scale, pools, bt = _case(rng, cs["kv"], cs["q"], cs["hkv"], cs["D"], seq_lens, q_lens, pages, width)
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
