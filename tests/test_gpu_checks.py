"""The device-checked mode (PA_DEBUG_CHECKS), through the C ABI.

With the flag, the kernels check lengths and block-table entries before the
accesses they steer, skip what is bad, finish normally and record the kind
of fault in a device error word ("Dual MI50, part 2", section "Bug 2: the
drafter read freed memory": a reader of freed blocks is this class of
error).  Every case here corrupts a device array that the checks guard, then
reads the status, then runs a valid forward on the same handle."""
import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from synth import Spec, generate
from tests.gpu_helpers import GpuCase, compare, progress

pytestmark = pytest.mark.gpu

B = pal.binding


def _spec(**kw):
    base = dict(name="chk", num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=(3000, 700), q_lens=(8, 1),
                q_dtype="bf16", kv_dtype="bf16", seed=81)
    base.update(kw)
    return Spec(**base)


def _checked_case(inp, extra_q: int = 0, **tuning):
    """A PA_DEBUG_CHECKS handle for inp (max_q_len raised by extra_q)."""
    pos = inp.q_lens[inp.q_lens > 0]
    cfg = pal.make_config(inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.q_dtype, inp.kv_dtype, inp.num_seqs,
                          int(inp.q_lens.max()) + extra_q, inp.num_tokens, page_size=inp.page_size,
                          min_q_len=int(pos.min()), flags=B.PA_DEBUG_CHECKS)
    h = pal.paged_attn_create(cfg)
    if tuning:
        pal.paged_attn_set_tuning(h, **tuning)
    return GpuCase([inp], handle=h)


KINDS = {
    # (spec overrides, tuning): every kernel path
    "valu_planned": (dict(seq_lens=(3000, 700, 40), q_lens=(1, 1, 1)), dict(split_mode=2)),
    "valu_static": (dict(seq_lens=(3000,), q_lens=(1,)), dict(split_mode=1, path=pal.PA_PATH_VALU)),
    "tile_verify": (dict(seq_lens=(3000, 700), q_lens=(8, 4)), dict(path=pal.PA_PATH_MFMA)),
    "tile_fp8": (dict(seq_lens=(3000, 700), q_lens=(8, 4), kv_dtype="fp8_e4m3"), {}),
    "tile_int8": (dict(seq_lens=(3000, 700), q_lens=(8, 4), kv_dtype="int8"), {}),
    "tile_prefill": (dict(num_q_heads=24, num_kv_heads=4, seq_lens=(2000,), q_lens=(300,)), {}),
    "tile_pages48": (dict(seq_lens=(3000, 700), q_lens=(8, 4), page_size=48), {}),
    # head_dim 256: the VALU kernel, then the 128-row tile kernel
    "d256_valu": (dict(num_q_heads=16, num_kv_heads=2, head_dim=256, seq_lens=(3000, 700), q_lens=(4, 1)), {}),
    "d256_tile": (dict(num_q_heads=16, num_kv_heads=2, head_dim=256, seq_lens=(2000, 700), q_lens=(100, 20),
                       kv_dtype="fp8_e4m3"), {}),
}

FAULTS = ["page_high", "page_negative", "q_len_over_seq_len", "seq_len_past_table", "tokens_over"]


def _corrupt(c, fault):
    """Plants one fault in the uploaded device arrays; returns the bit the
    checks must report."""
    import torch

    d = c.dev[0]
    npages = c.pools["k"].shape[0]
    if fault == "page_high":
        d["block_table"][0, 1] = npages + 3
        return B.PA_CHECK_PAGE
    if fault == "page_negative":
        d["block_table"][0, 0] = -1
        return B.PA_CHECK_PAGE
    if fault == "q_len_over_seq_len":
        d["seq_lens"][0] = int(c.batches[0].q_lens[0]) - 1
        return B.PA_CHECK_LENGTHS
    if fault == "seq_len_past_table":
        width = d["block_table"].shape[1]
        d["seq_lens"][0] = width * c.batches[0].page_size + 5
        return B.PA_CHECK_TABLE
    if fault == "tokens_over":
        # (the handle's max_q_len allows the larger q_len; the sum passes num_tokens)
        d["q_lens"][-1] += 1
        return B.PA_CHECK_TOKENS
    raise ValueError(fault)


@pytest.mark.parametrize("fault", FAULTS)
@pytest.mark.parametrize("kind", list(KINDS))
def test_checked_mode_reports_and_survives(kind, fault):
    import torch

    over, tuning = KINDS[kind]
    inp = generate(_spec(name=kind, **over))[0]
    c = _checked_case(inp, extra_q=1 if fault == "tokens_over" else 0, **tuning)
    try:
        progress(f"checks {kind} {fault}")
        bits, msg = pal.paged_attn_debug_status(c.h)
        assert bits == 0 and msg == ""
        saved = {k: v.clone() for k, v in c.dev[0].items() if v is not None}
        want = _corrupt(c, fault)
        c.run()                                        # completes: the checks steer every access in bounds
        bits, msg = pal.paged_attn_debug_status(c.h)
        assert bits & want, (bits, msg)
        assert "device checks" in msg
        assert pal.paged_attn_debug_status(c.h)[0] == 0          # cleared
        # the same handle, valid arrays again: oracle parity
        for k, v in saved.items():
            c.dev[0][k].copy_(v)
        out, lse = c.run()
        assert pal.paged_attn_debug_status(c.h)[0] == 0
    finally:
        c.close()
    ref_o, ref_l = oracle.attention(inp)
    compare(f"checks {kind} after {fault}", inp.kv_dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("kind", list(KINDS))
def test_checked_mode_is_bit_identical_on_valid_inputs(kind):
    over, tuning = KINDS[kind]
    inp = generate(_spec(name=kind, **over))[0]
    c1 = _checked_case(inp, **tuning)
    c2 = GpuCase([inp], **tuning)
    try:
        o1, l1 = c1.run()
        o2, l2 = c2.run()
        assert pal.paged_attn_debug_status(c1.h)[0] == 0
    finally:
        c1.close()
        c2.close()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


def test_last_error_reports_device_checks():
    inp = generate(_spec())[0]
    c = _checked_case(inp)
    try:
        c.dev[0]["block_table"][1, 0] = 1 << 30
        c.run()
        msg = pal.paged_attn_last_error(c.h)
        assert "page id outside" in msg
    finally:
        c.close()


def test_append_checked_mode():
    import torch

    hkv, D, P = 2, 128, 16
    cfg = pal.make_config(8, hkv, D, "f16", "f16", 3, 4, 12, flags=B.PA_DEBUG_CHECKS)
    h = pal.paged_attn_create(cfg)
    try:
        pool = torch.zeros((6, hkv, P, D), dtype=torch.float16, device="cuda")
        vpool = torch.zeros_like(pool)
        bt = torch.tensor([[0, 99], [1, -1], [2, 3]], dtype=torch.int32, device="cuda")
        seq_lens = torch.tensor([20, 3, 40], dtype=torch.int32, device="cuda")
        q_lens = torch.tensor([4, 4, 4], dtype=torch.int32, device="cuda")
        new = torch.ones((12, hkv, D), dtype=torch.float16, device="cuda")
        pal.paged_attn_append(h, new, new, pool, vpool, bt, seq_lens, q_lens)
        torch.cuda.synchronize()
        bits, msg = pal.paged_attn_debug_status(h)
        assert bits & B.PA_CHECK_PAGE and bits & B.PA_CHECK_LENGTHS and bits & B.PA_CHECK_TABLE, (bits, msg)
        assert not (pool != 0).any().item()
    finally:
        pal.paged_attn_destroy(h)


def test_noalloc_refuses_checked_mode():
    import torch

    cfg = pal.make_config(32, 8, 128, "bf16", "bf16", 1, 1, 1, flags=B.PA_DEBUG_CHECKS)
    q = torch.zeros((1, 32, 128), dtype=torch.int16, device="cuda")
    kc = torch.zeros((4, 8, 16, 128), dtype=torch.int16, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    sl = torch.ones(1, dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(pal.PagedAttnError) as e:
        pal.paged_attn_forward_noalloc(cfg, q, kc, kc, bt, sl, sl, 0, 0.088, None, out)
    assert e.value.code == B.PA_ERR_UNSUPPORTED
