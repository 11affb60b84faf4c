"""Seeded generator of paged-KV attention inputs (storage bits only).

The workloads follow the shapes the source pages keep returning to:
decode at a 4k context ("tps-maxxing on amd gpu", section "Baseline"),
speculative verification of k+1 <= 8 rows and the drafter's 2048-token
sliding window ("Dual MI50, part 2", sections "Kernels: why the generic code
is slow here" and "Bug 2: the drafter read freed memory"), a 2048-token
prefill chunk against a 65k cache ("Strix Halo dense cliff patch
attribution", section "The measurement that changed the series"), and a
long-context mixed batch with a quantised cache ("Dual MI50, part 2",
sections "200k context for coding agents" and "Prefill: teach the fork's fast
kernel to read the int8 cache").

Recipe (the same for every workload):
  * one numpy ``SeedSequence(seed)``; child 0 draws a permutation of the
    physical page pool, child 1+k draws batch k's values;
  * every value is float32 N(0,1) from PCG64, rounded to the storage dtype
    by round-to-nearest-even (numpy for fp16, torch for bf16 / fp8);
  * the new query tokens' own keys are already in the cache: a sequence's
    ``seq_len`` counts its ``q_len`` new tokens, which are its last ones;
  * sequence b's logical pages take the next ``ceil(seq_len/P)`` entries of
    the permutation, in order; the block table's padding entries point at a
    dedicated page that holds only NaN;
  * slots of the last page past ``seq_len`` hold NaN, and with
    ``poison_out_of_window`` every page whose tokens all fall before the
    first query row's window holds NaN in K and V (freed-and-reused pages);
  * fp8 (OCP E4M3FN) caches are quantised per (K or V, KV head) with scale
    ``amax/448`` over that head's live tokens, codes saturated to +-448;
  * int8 caches carry one fp32 scale per cached row (one token of one KV
    head, K and V separately), the pages' own cache format ("Dual MI50,
    part 2", section "Prefill: teach the fork's fast kernel to read the int8
    cache"): scale ``amax/127`` over the row's D values, code the nearest
    integer to ``x/scale`` (ties to even, both steps in fp32) within
    [-127, 127]; a dead slot (tail, unused page, poisoned page) holds code
    -128 and a NaN scale.

Nothing here computes attention.  The returned arrays are raw storage bits;
consumers decode them with their own code.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# Canonical quiet-NaN storage patterns.
# (int8 has no NaN code: a dead int8 slot holds -128, never produced by the
# quantiser, and its row scale is NaN.)
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F, "int8": 0x80}
STORAGE_NP = {"f16": np.uint16, "bf16": np.uint16, "fp8_e4m3": np.uint8, "int8": np.uint8}
ELEM_BYTES = {"f16": 2, "bf16": 2, "fp8_e4m3": 1, "int8": 1}
ROW_SCALE_BYTES = {"int8": 4}   # per cached row (token, KV head) of K or of V
FP8_E4M3_MAX = 448.0


@dataclass(frozen=True)
class Spec:
    """Shape and value recipe of one workload."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_lens: tuple
    q_lens: tuple
    q_dtype: str = "f16"
    kv_dtype: str = "f16"
    page_size: int = 16
    pool_pages: int = 0            # 0: smallest pool that fits (plus the NaN page)
    window: int = 0                # <= 0: none; W >= 1: keys p-W+1 .. p
    scale: Optional[float] = None  # None: fp32(1/sqrt(head_dim))
    k_outlier_frac: float = 0.0    # fraction of token positions whose K is multiplied
    k_outlier_mult: float = 4.0
    poison_out_of_window: bool = False
    block_table_width: int = 0     # 0: the longest sequence's page count
    seed: int = 0
    keep_float: bool = False       # also return the float32 values before rounding (small inputs)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


@dataclass
class PagedInputs:
    """One batch of inputs, as raw storage bits plus integer metadata."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    q_dtype: str
    kv_dtype: str
    window: int
    scale: float
    seq_lens: np.ndarray        # int32 [B]
    q_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray     # int32 [B, width]
    num_pages: int              # physical pool size
    live_pages: np.ndarray      # int64 [n_live]: physical id of each live page, (seq, logical page) order
    page_offsets: np.ndarray    # int64 [B+1]: seq b owns live_pages[page_offsets[b]:page_offsets[b+1]]
    k_live: np.ndarray          # uint16/uint8 [n_live, Hkv, P, D]
    v_live: np.ndarray          # same
    q: np.ndarray               # uint16 [T, Hq, D]
    kv_scale: Optional[np.ndarray]  # float32 [2, Hkv] (K row, then V row) for fp8, else None
    fill_bits: int              # storage bits of every pool page that is not live
    nan_page: int               # physical id of the padding page (never live)
    seed: int = 0
    batch: int = 0
    extra: dict = field(default_factory=dict)
    row_scale: Optional[np.ndarray] = None   # float32 [2, n_live, Hkv, P] (K, then V) for int8, else None

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def visible_range(self, b: int):
        """[lo, seq_len) of tokens any query row of sequence b may see."""
        s = int(self.seq_lens[b])
        ql = int(self.q_lens[b])
        if self.window > 0:
            return max(0, s - ql - self.window + 1), s
        return 0, s

    def kv_bytes(self) -> int:
        """K+V bytes of the visible token ranges, once per KV head (with each
        row's scale for int8 caches)."""
        tot = 0
        for b in range(self.num_seqs):
            lo, hi = self.visible_range(b)
            if int(self.q_lens[b]) > 0:
                tot += (hi - lo)
        row = self.head_dim * ELEM_BYTES[self.kv_dtype] + ROW_SCALE_BYTES.get(self.kv_dtype, 0)
        return 2 * tot * self.num_kv_heads * row

    def pair_count(self) -> int:
        """Visible (query row, key) pairs per query head."""
        tot = 0
        for b in range(self.num_seqs):
            s = int(self.seq_lens[b])
            ql = int(self.q_lens[b])
            for i in range(ql):
                p = s - ql + i
                lo = max(0, p - self.window + 1) if self.window > 0 else 0
                tot += p - lo + 1
        return tot

    def flops(self) -> int:
        """4*D per visible (row, key) pair per query head (Q.K^T and P.V)."""
        return 4 * self.head_dim * self.pair_count() * self.num_q_heads


def _int8_rows(x: np.ndarray):
    """Codes (uint8 bits of int8) and fp32 scales of rows x[..., D]: scale =
    amax/127, code = nearest integer to x/scale, ties to even, in [-127, 127];
    a zero row (scale 0) gets zero codes."""
    amax = np.abs(x).max(axis=-1)
    sc = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qv = x / sc[..., None]
    qv = np.where(np.isnan(qv), np.float32(0.0), np.clip(np.rint(qv), -127.0, 127.0))
    return qv.astype(np.int8).view(np.uint8), sc


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (RNE) and return the bits."""
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8_e4m3":
        t = t.clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX)
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def _pages_needed(seq_len: int, page: int) -> int:
    return (seq_len + page - 1) // page


def generate(spec: Spec, seed: Optional[int] = None, batches: int = 1) -> List[PagedInputs]:
    """Draw ``batches`` independent batches of ``spec`` sharing one page pool.

    Batches use disjoint physical pages, so a caller can place all of them in
    one pool and rotate between them.
    """
    seed = spec.seed if seed is None else seed
    H, Hk, D, P = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    if H % Hk:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    seq_lens = np.asarray(spec.seq_lens, dtype=np.int64)
    q_lens = np.asarray(spec.q_lens, dtype=np.int64)
    if seq_lens.shape != q_lens.shape:
        raise ValueError("seq_lens and q_lens differ in length")
    if np.any(q_lens > seq_lens) or np.any(q_lens < 0):
        raise ValueError("need 0 <= q_len <= seq_len")
    B = seq_lens.shape[0]
    npg = np.array([_pages_needed(int(s), P) for s in seq_lens], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(npg)]).astype(np.int64)
    n_live = int(offs[-1])
    width = spec.block_table_width or int(max(npg.max(initial=0), 1))
    if width < npg.max(initial=0):
        raise ValueError("block_table_width too small")
    pool = spec.pool_pages or (batches * n_live + 1)
    if pool < batches * n_live + 1:
        raise ValueError(f"pool of {pool} pages cannot hold {batches} x {n_live} live pages + 1")
    scale = spec.scale if spec.scale is not None else float(np.float32(1.0 / math.sqrt(D)))
    scale = float(np.float32(scale))

    root = np.random.SeedSequence(seed)
    kids = root.spawn(1 + batches)
    perm = np.random.default_rng(kids[0]).permutation(pool).astype(np.int64)
    nan_page = int(perm[batches * n_live])

    out = []
    for bi in range(batches):
        q_ss, k_ss, v_ss, o_ss, _spare = kids[1 + bi].spawn(5)
        live = perm[bi * n_live:(bi + 1) * n_live].copy()
        bt = np.full((B, width), nan_page, dtype=np.int32)
        for b in range(B):
            bt[b, :npg[b]] = live[offs[b]:offs[b + 1]]

        T = int(q_lens.sum())
        qf = np.random.default_rng(q_ss).standard_normal((T, H, D), dtype=np.float32)
        kf = np.random.default_rng(k_ss).standard_normal((n_live, Hk, P, D), dtype=np.float32)
        vf = np.random.default_rng(v_ss).standard_normal((n_live, Hk, P, D), dtype=np.float32)

        if spec.k_outlier_frac > 0:
            orng = np.random.default_rng(o_ss)
            outl = {}
            for b in range(B):
                s = int(seq_lens[b])
                n = int(round(spec.k_outlier_frac * s))
                pos = np.sort(orng.choice(s, size=n, replace=False))
                outl[b] = pos
                pg = offs[b] + pos // P
                kf[pg, :, pos % P, :] *= np.float32(spec.k_outlier_mult)
        else:
            outl = {}

        # Live-token mask (for fp8 amax and for NaN placement).
        live_mask = np.zeros((n_live, P), dtype=bool)
        for b in range(B):
            s = int(seq_lens[b])
            full = s // P
            live_mask[offs[b]:offs[b] + full, :] = True
            if s % P:
                live_mask[offs[b] + full, :s % P] = True

        if spec.keep_float:
            extra_float = {"k_float": kf.copy(), "v_float": vf.copy(), "q_float": qf.copy()}
        else:
            extra_float = {}
        kv_scale = None
        if spec.kv_dtype == "fp8_e4m3":
            kv_scale = np.zeros((2, Hk), dtype=np.float32)
            for which, arr in enumerate((kf, vf)):
                for h in range(Hk):
                    a = np.abs(arr[:, h, :, :][live_mask]).max(initial=0.0)
                    s_h = np.float32(a) / np.float32(FP8_E4M3_MAX) if a > 0 else np.float32(1.0)
                    kv_scale[which, h] = s_h
                    arr[:, h, :, :] /= s_h
        row_scale = None
        if spec.kv_dtype == "int8":
            row_scale = np.empty((2, n_live, Hk, P), dtype=np.float32)
            kb, row_scale[0] = _int8_rows(kf)
            del kf
            vb, row_scale[1] = _int8_rows(vf)
            del vf
        else:
            kb = _to_bits(kf, spec.kv_dtype)
            del kf
            vb = _to_bits(vf, spec.kv_dtype)
            del vf
        qb = _to_bits(qf, spec.q_dtype)
        del qf

        nanb = NAN_BITS[spec.kv_dtype]
        # Tail slots past seq_len: never live.
        dead = ~live_mask
        kb[np.nonzero(dead)[0], :, np.nonzero(dead)[1], :] = nanb
        vb[np.nonzero(dead)[0], :, np.nonzero(dead)[1], :] = nanb
        if row_scale is not None:
            row_scale[:, np.nonzero(dead)[0], :, np.nonzero(dead)[1]] = np.nan
        poisoned = []
        if spec.poison_out_of_window and spec.window > 0:
            for b in range(B):
                s, ql = int(seq_lens[b]), int(q_lens[b])
                lo = max(0, s - ql - spec.window + 1)
                n_dead = lo // P        # pages whose every token precedes lo
                if n_dead:
                    kb[offs[b]:offs[b] + n_dead] = nanb
                    vb[offs[b]:offs[b] + n_dead] = nanb
                    if row_scale is not None:
                        row_scale[:, offs[b]:offs[b] + n_dead] = np.nan
                    poisoned.append((b, n_dead))

        out.append(PagedInputs(
            name=spec.name, num_q_heads=H, num_kv_heads=Hk, head_dim=D, page_size=P,
            q_dtype=spec.q_dtype, kv_dtype=spec.kv_dtype, window=int(spec.window), scale=scale,
            seq_lens=seq_lens.astype(np.int32), q_lens=q_lens.astype(np.int32), block_table=bt,
            num_pages=int(pool), live_pages=live, page_offsets=offs, k_live=kb, v_live=vb, q=qb,
            kv_scale=kv_scale, fill_bits=nanb, nan_page=nan_page, seed=seed, batch=bi, row_scale=row_scale,
            extra={"outliers": outl, "poisoned_pages": poisoned, **extra_float},
        ))
    return out


def permute_pool(inp: PagedInputs, seed: int) -> PagedInputs:
    """Move every live page to another physical page and remap the table.

    The logical cache is unchanged, so attention over it must be unchanged.
    """
    rng = np.random.default_rng(seed)
    perm = rng.permutation(inp.num_pages).astype(np.int64)   # old id -> new id
    new = dataclasses.replace(inp)
    new.live_pages = perm[inp.live_pages]
    new.nan_page = int(perm[inp.nan_page])
    new.block_table = perm[inp.block_table.astype(np.int64)].astype(np.int32)
    return new


# The named workloads (seed 1000 + k for the k-th).
NAMED_SPECS = {
    "tiny_decode": Spec(
        name="tiny_decode", num_q_heads=4, num_kv_heads=1, head_dim=64,
        seq_lens=(257,), q_lens=(1,), q_dtype="f16", kv_dtype="f16", pool_pages=32, seed=1001),
    "decode": Spec(
        name="decode", num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_lens=(4097,), q_lens=(1,), q_dtype="bf16", kv_dtype="bf16", pool_pages=65536, seed=1002),
    "verify": Spec(
        name="verify", num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_lens=(61448,), q_lens=(8,), q_dtype="f16", kv_dtype="f16", pool_pages=8192,
        k_outlier_frac=0.01, k_outlier_mult=4.0, seed=1003),
    "verify_window": Spec(
        name="verify_window", num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_lens=(61448,), q_lens=(8,), q_dtype="f16", kv_dtype="f16", pool_pages=8192,
        k_outlier_frac=0.01, k_outlier_mult=4.0, window=2048, poison_out_of_window=True, seed=1003),
    "prefill": Spec(
        name="prefill", num_q_heads=24, num_kv_heads=4, head_dim=128,
        seq_lens=(67584,), q_lens=(2048,), q_dtype="bf16", kv_dtype="bf16", pool_pages=8192, seed=1004),
    "mixed_fp8": Spec(
        name="mixed_fp8", num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_lens=(200001, 131076, 32776, 4097), q_lens=(1, 4, 8, 1),
        q_dtype="bf16", kv_dtype="fp8_e4m3", pool_pages=32768, seed=1005),
    # chunked prefill at head_dim 256 (the width of the dense models in the
    # pages' long-context prefill measurements); head counts are a reading
    "prefill_d256": Spec(
        name="prefill_d256", num_q_heads=16, num_kv_heads=2, head_dim=256,
        seq_lens=(67584,), q_lens=(2048,), q_dtype="bf16", kv_dtype="bf16", pool_pages=8192, seed=1007),
    # the same long mixed batch on the pages' own cache format: int8 codes
    # with a fp32 scale per cached row
    "mixed_int8": Spec(
        name="mixed_int8", num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_lens=(200001, 131076, 32776, 4097), q_lens=(1, 4, 8, 1),
        q_dtype="bf16", kv_dtype="int8", pool_pages=32768, seed=1006),
    # the chunked prefill on the pages' int8 cache (codes and per-row scales
    # read in place)
    "prefill_int8": Spec(
        name="prefill_int8", num_q_heads=24, num_kv_heads=4, head_dim=128,
        seq_lens=(67584,), q_lens=(2048,), q_dtype="bf16", kv_dtype="int8", pool_pages=8192, seed=1008),
}


def named(name: str, batches: int = 1, **overrides) -> List[PagedInputs]:
    spec = NAMED_SPECS[name]
    if overrides:
        spec = spec.replace(**overrides)
    return generate(spec, batches=batches)


def replicate(inp: PagedInputs, copies: int, seed: int = 0, pool_pages: int = 0) -> List[PagedInputs]:
    """``copies`` batches with inp's logical content at disjoint physical pages.

    Used to rotate a benchmark over more memory than the GPU caches hold,
    without drawing new values.  Copy 0 is inp itself.
    """
    n_live = len(inp.live_pages)
    pool = max(pool_pages, inp.num_pages, copies * n_live + 1)
    rng = np.random.default_rng(seed)
    used = set(inp.live_pages.tolist()) | {inp.nan_page}
    free = np.array([p for p in rng.permutation(pool) if p not in used], dtype=np.int64)
    out = [dataclasses.replace(inp, num_pages=int(pool))]
    for c in range(1, copies):
        new_live = free[(c - 1) * n_live:c * n_live]
        remap = dict(zip(inp.live_pages.tolist(), new_live.tolist()))
        bt = np.vectorize(lambda x: remap.get(int(x), inp.nan_page), otypes=[np.int64])(inp.block_table)
        out.append(dataclasses.replace(inp, num_pages=int(pool), live_pages=new_live,
                                       block_table=bt.astype(np.int32), batch=c))
    return out
