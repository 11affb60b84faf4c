"""The forward that allocates nothing (paged_attn_forward_noalloc) against
the handle forward on the same inputs, through the C ABI: two calls in a
row, the second smaller, each checked against the fp64 oracle within the
tolerances of the handle path and bit for bit against the handle path's
output."""
import numpy as np
import pytest

import oracle
import paged_attention_long_amd as pal
from synth import NAMED_SPECS, generate
from tests.gpu_helpers import TOL, GpuCase, compare, progress

pytestmark = pytest.mark.gpu


def _noalloc_run(case: GpuCase, cfg, i: int = 0):
    import torch

    b, d = case.batches[i], case.dev[i]
    out = torch.full_like(case.out[i], float("nan"))
    lse = torch.full_like(case.lse[i], float("nan"))
    pal.paged_attn_forward_noalloc(cfg, d["q"], case.pools["k"], case.pools["v"], d["block_table"], d["seq_lens"],
                                   d["q_lens"], b.window, b.scale, case.kv_scale(i), out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check_pair(name: str, spec):
    inp = generate(spec)[0]
    case = GpuCase([inp])
    try:
        progress(f"no-alloc {name}: handle forward")
        ref_h = case.run(0)
        progress(f"no-alloc {name}: no-alloc forward")
        got = _noalloc_run(case, case.h.cfg)
    finally:
        case.close()
    ref_o, ref_l = oracle.attention(inp)
    compare(f"no-alloc {name} vs oracle", inp.kv_dtype, got[0], got[1], ref_o, ref_l)
    tol_o, tol_l = TOL[inp.kv_dtype]
    eo = float(np.max(np.abs(got[0] - ref_h[0])))
    el = float(np.max(np.abs(got[1] - ref_h[1])))
    progress(f"no-alloc {name} vs handle: max|dout|={eo:.3e} max|dlse|={el:.3e} "
             f"(bit-identical: {np.array_equal(got[0], ref_h[0]) and np.array_equal(got[1], ref_h[1])})")
    assert eo <= tol_o and el <= tol_l
    # same kernels, split sizes and merge order as the handle path: the bits agree
    assert np.array_equal(got[0].view(np.uint32), ref_h[0].view(np.uint32))
    assert np.array_equal(got[1].view(np.uint32), ref_h[1].view(np.uint32))


def test_noalloc_two_calls_second_smaller():
    # a verification batch on the tile kernel, then a smaller decode on the
    # VALU kernel: the second call lays the array out differently and must
    # not see the first call's counters or partials
    verify = NAMED_SPECS["verify"].replace(seq_lens=(20000,), q_lens=(8,), pool_pages=4096, seed=71)
    decode = NAMED_SPECS["decode"].replace(seq_lens=(3000,), q_lens=(1,), pool_pages=1024, seed=72)
    _check_pair("verify 20000x8 f16", verify)
    _check_pair("decode 3000x1 bf16", decode)


def test_noalloc_mixed_fp8_then_tiny():
    mixed = NAMED_SPECS["mixed_fp8"].replace(seq_lens=(40001, 9004, 3000, 257), pool_pages=4096, seed=73)
    tiny = NAMED_SPECS["tiny_decode"].replace(seed=74)
    _check_pair("mixed fp8 4 seqs", mixed)
    _check_pair("tiny decode", tiny)


def test_noalloc_head_dim_256_then_smaller():
    # head_dim 256 on the VALU kernel (two new tokens, 16 rows per KV head,
    # static splits), then a smaller decode of the same width
    verify = NAMED_SPECS["decode"].replace(num_q_heads=16, num_kv_heads=2, head_dim=256, seq_lens=(9000,),
                                           q_lens=(2,), pool_pages=1024, seed=75)
    decode = NAMED_SPECS["decode"].replace(num_q_heads=16, num_kv_heads=2, head_dim=256, seq_lens=(2000, 31),
                                           q_lens=(1, 1), pool_pages=512, kv_dtype="int8", seed=76)
    _check_pair("d256 verify 9000x2 bf16", verify)
    _check_pair("d256 decode int8", decode)


def test_noalloc_rejects_oversized_config():
    cfg = pal.make_config(24, 4, 128, "bf16", "bf16", 1, 2048, 2048)
    import torch

    q = torch.zeros((2048, 24, 128), dtype=torch.int16, device="cuda")
    kc = torch.zeros((64, 4, 16, 128), dtype=torch.int16, device="cuda")
    bt = torch.zeros((1, 64), dtype=torch.int32, device="cuda")
    sl = torch.full((1,), 1024, dtype=torch.int32, device="cuda")
    ql = torch.full((1,), 1024, dtype=torch.int32, device="cuda")
    out = torch.zeros((2048, 24, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(pal.PagedAttnError) as e:
        pal.paged_attn_forward_noalloc(cfg, q, kc, kc, bt, sl, ql, 0, 0.088, None, out)
    assert e.value.code == pal.binding.PA_ERR_UNSUPPORTED
    assert "no-allocation" in pal.paged_attn_last_error(None)
