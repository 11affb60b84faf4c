"""GPU-side helpers for the parity tests: build a handle for generated
inputs, upload them, run the library through its C ABI, compare with the
oracle."""
from __future__ import annotations

import os
import sys
import time
from typing import List, Optional

import numpy as np

import paged_attention_long_amd as pal
from synth.torch_upload import upload_batch, upload_pool

# Tolerances (max abs error against the fp64 oracle): fp16/bf16 caches with
# fp32 accumulation 2e-3 on out and 1e-3 on lse; fp8 caches 2e-2 on out and
# 1e-3 on lse (the oracle reads the same stored codes and scales, which
# enter the scores exactly in fp32, so the lse carries no format error);
# int8 caches (per-row scales) the same as fp8.
TOL = {"f16": (2e-3, 1e-3), "bf16": (2e-3, 1e-3), "fp8_e4m3": (2e-2, 1e-3), "int8": (2e-2, 1e-3)}


def progress(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so it survives a crash)."""
    line = f"[{time.strftime('%H:%M:%S')}] {msg}"
    print(line, file=sys.stderr, flush=True)
    path = os.environ.get("PA_PROGRESS_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
            f.flush()
            os.fsync(f.fileno())


def make_handle(inp, max_q_len: Optional[int] = None, max_num_tokens: Optional[int] = None,
                max_num_seqs: Optional[int] = None, min_q_len: Optional[int] = None, **tuning):
    qmax = max_q_len or int(max(inp.q_lens.max(), 1))
    pos = inp.q_lens[inp.q_lens > 0]
    qmin = min_q_len or int(pos.min() if pos.size else 1)
    cfg = pal.make_config(inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.q_dtype, inp.kv_dtype,
                          max_num_seqs or inp.num_seqs, qmax, max_num_tokens or inp.num_tokens,
                          page_size=inp.page_size, min_q_len=min(qmin, qmax))
    h = pal.paged_attn_create(cfg)
    if tuning:
        pal.paged_attn_set_tuning(h, **tuning)
    return h


class GpuCase:
    """Uploaded batches sharing one pool, plus a handle."""

    def __init__(self, batches: List, layout: str = "hnd", handle=None, **tuning):
        import torch

        self.batches = batches
        self.pools = upload_pool(batches, layout=layout)
        self.dev = [upload_batch(b) for b in batches]
        first = batches[0]
        pos = [int(b.q_lens[b.q_lens > 0].min()) for b in batches if (b.q_lens > 0).any()]
        self.h = handle or make_handle(
            first, max_q_len=max(int(b.q_lens.max()) for b in batches),
            max_num_tokens=max(b.num_tokens for b in batches),
            max_num_seqs=max(b.num_seqs for b in batches), min_q_len=min(pos) if pos else 1, **tuning)
        self.own = handle is None
        self.out = [torch.empty((b.num_tokens, b.num_q_heads, b.head_dim), dtype=torch.float32, device="cuda")
                    for b in batches]
        self.lse = [torch.empty((b.num_tokens, b.num_q_heads), dtype=torch.float32, device="cuda") for b in batches]

    def kv_scale(self, i: int = 0):
        """The kv_scale argument: per-head scales (fp8) or the pool's row
        scales (int8)."""
        return self.pools["row_scale"] if "row_scale" in self.pools else self.dev[i]["kv_scale"]

    def forward(self, i: int = 0, stream=None):
        b, d = self.batches[i], self.dev[i]
        pal.paged_attn_forward(self.h, d["q"], self.pools["k"], self.pools["v"], d["block_table"], d["seq_lens"],
                               d["q_lens"], b.window, b.scale, self.kv_scale(i), self.out[i], self.lse[i],
                               stream=stream)

    def run(self, i: int = 0):
        import torch

        self.out[i].fill_(float("nan"))
        self.lse[i].fill_(float("nan"))
        self.forward(i)
        torch.cuda.synchronize()
        return self.out[i].cpu().numpy().copy(), self.lse[i].cpu().numpy().copy()

    def close(self):
        if self.own:
            pal.paged_attn_destroy(self.h)


def compare(name: str, kv_dtype: str, out, lse, ref_out, ref_lse, rows=None):
    """Max abs errors; asserts the tolerances and finiteness."""
    tol_o, tol_l = TOL[kv_dtype]
    if rows is None:
        assert np.all(np.isfinite(out)), f"{name}: non-finite output"
        assert np.all(np.isfinite(lse)), f"{name}: non-finite lse"
        eo = float(np.max(np.abs(out.astype(np.float64) - ref_out))) if out.size else 0.0
        el = float(np.max(np.abs(lse.astype(np.float64) - ref_lse))) if lse.size else 0.0
    else:
        eo = el = 0.0
        for (t, h), (ro, rl) in rows.items():
            assert np.all(np.isfinite(out[t, h])) and np.isfinite(lse[t, h]), f"{name}: non-finite row {(t, h)}"
            eo = max(eo, float(np.max(np.abs(out[t, h].astype(np.float64) - ro))))
            el = max(el, abs(float(lse[t, h]) - rl))
    progress(f"{name}: max|dout|={eo:.3e} (tol {tol_o}) max|dlse|={el:.3e} (tol {tol_l})")
    assert eo <= tol_o, f"{name}: out error {eo} > {tol_o}"
    assert el <= tol_l, f"{name}: lse error {el} > {tol_l}"
    return eo, el
