"""fp64 paged attention from its definition (oracle, test only).

Every function takes an input object with the attributes the seeded
generator fills in (storage bits, block table, lengths, window, scale); it
does not import the generator.

Readings of the source pages used here (each is listed with its reason in
the design notes):
  * a sequence's ``seq_len`` already counts its ``q_len`` new tokens, whose
    keys are the last ``q_len`` entries of the cache, and query row i sits at
    position p_i = seq_len - q_len + i ("Dual MI50, part 2", section
    "Kernels: why the generic code is slow here": verification scores k+1
    new tokens; "tps-maxxing on amd gpu", section "Speculative decoding:
    native MTP vs. DFlash": the candidates follow the cached prefix);
  * row i sees key j iff j <= p_i (causal inside the new rows) and, with a
    window W >= 1, j >= p_i - W + 1: the W most recent keys including itself
    ("Dual MI50, part 2", section "Bug 2: the drafter read freed memory");
  * query head h reads KV head h // (Hq / Hkv) ("Dual MI50, part 2",
    section "Decode: a new kernel for the shape MTP actually runs": several
    query heads share each KV head);
  * the fp8 cache value is code * scale[K or V, kv head]; the int8 cache
    value is code * (the fp32 scale of its own row: one token of one KV
    head, K and V separately), the pages' own cache format ("Dual MI50,
    part 2", section "Prefill: teach the fork's fast kernel to read the int8
    cache": the cache is read in place with its per-row scales); the softmax
    scale multiplies q.k after that dequantisation;
  * lse is the natural log of the sum of exp over the visible scaled scores.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .codec import decode_bits

NEG_INF = float("-inf")


# ---------------------------------------------------------------- positions

def query_positions(seq_len: int, q_len: int) -> np.ndarray:
    """Cache positions of the q_len new query rows: the last q_len tokens."""
    return np.arange(seq_len - q_len, seq_len, dtype=np.int64)


def visible_bounds(p: int, window: int) -> Tuple[int, int]:
    """Inclusive key range [lo, p] that a row at position p may see."""
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, p


# ---------------------------------------------------------------- de-paging

def _live_index(inp) -> np.ndarray:
    """Physical page id -> index into the live page arrays, -1 if not live."""
    idx = np.full(int(inp.num_pages), -1, dtype=np.int64)
    idx[np.asarray(inp.live_pages, dtype=np.int64)] = np.arange(len(inp.live_pages))
    return idx


def _page_bits(inp, which: str, phys: int, live_index: np.ndarray) -> np.ndarray:
    """Storage bits [Hkv, P, D] of physical page ``phys`` of the K or V pool."""
    arr = inp.k_live if which == "k" else inp.v_live
    li = live_index[phys]
    if li < 0:
        return np.full(arr.shape[1:], inp.fill_bits, dtype=arr.dtype)
    return arr[li]


def _page_row_scales(inp, which: str, phys: int, live_index: np.ndarray) -> np.ndarray:
    """fp32 row scales [Hkv, P] of physical page ``phys`` (int8 caches); a page
    that holds no live data has NaN scales."""
    li = live_index[phys]
    shape = inp.row_scale.shape[2:]
    if li < 0:
        return np.full(shape, np.nan, dtype=np.float32)
    return inp.row_scale[0 if which == "k" else 1, li]


def depage(inp, which: str, b: int, g: int, lo: int, hi: int,
           live_index: Optional[np.ndarray] = None) -> np.ndarray:
    """Explicit copy of logical tokens [lo, hi) of sequence b, KV head g.

    Token j lives in physical page block_table[b][j // P], slot j % P.
    Returns float64 [hi - lo, D] holding the dequantised values (an int8
    row times its own scale from the same page and slot).  Only the
    requested tokens' pages are touched.
    """
    P = int(inp.page_size)
    D = int(inp.head_dim)
    if live_index is None:
        live_index = _live_index(inp)
    outv = np.empty((max(hi - lo, 0), D), dtype=np.float64)
    j = lo
    while j < hi:
        logical_page = j // P
        phys = int(inp.block_table[b][logical_page])
        page = _page_bits(inp, which, phys, live_index)          # [Hkv, P, D]
        s0 = j % P
        s1 = min(P, s0 + (hi - j))
        outv[j - lo:j - lo + (s1 - s0)] = decode_bits(page[g, s0:s1, :], inp.kv_dtype)
        if inp.kv_dtype == "int8":
            rs = _page_row_scales(inp, which, phys, live_index)[g, s0:s1].astype(np.float64)
            outv[j - lo:j - lo + (s1 - s0)] *= rs[:, None]
        j += s1 - s0
    if inp.kv_dtype == "fp8_e4m3":
        s = float(inp.kv_scale[0 if which == "k" else 1][g])
        outv *= s
    return outv


def _q_row(inp, t: int, h: int) -> np.ndarray:
    return decode_bits(inp.q[t, h, :], inp.q_dtype)


def _cu_q(inp) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(inp.q_lens, dtype=np.int64))])


# ---------------------------------------------------------------- core

def _rows_attention(qrows: np.ndarray, pos: np.ndarray, K: np.ndarray, V: np.ndarray,
                    base: int, window: int, scale64: float):
    """Attention of rows (query vectors ``qrows`` at positions ``pos``) over
    keys K/V holding logical tokens [base, base + len(K)).

    Sums run only over each row's visible keys.  The score block is formed
    with one matrix product over the rows' common key range and masked
    entries are excluded by -inf (their exp is exactly 0).  The P.V product
    is taken over the common range only if V is finite there (then the
    excluded zeros add exact zeros); otherwise each row is summed over its
    own slice.
    """
    n_rows = qrows.shape[0]
    D = qrows.shape[1]
    out = np.empty((n_rows, D), dtype=np.float64)
    lse = np.empty(n_rows, dtype=np.float64)
    bounds = [visible_bounds(int(p), window) for p in pos]
    u0 = min(lo for lo, _ in bounds)
    u1 = max(hi for _, hi in bounds) + 1
    Ku = K[u0 - base:u1 - base]
    Vu = V[u0 - base:u1 - base]
    S = scale64 * (qrows @ Ku.T)                                  # [rows, u1-u0]
    cols = np.arange(u0, u1)
    vis = np.zeros(S.shape, dtype=bool)
    for r, (lo, hi) in enumerate(bounds):
        vis[r] = (cols >= lo) & (cols <= hi)
    S = np.where(vis, S, NEG_INF)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])                                    # exp(-inf) == 0 exactly
    E = np.where(vis, E, 0.0)
    l = E.sum(axis=1)
    if np.all(np.isfinite(Vu)):
        out[:] = (E @ Vu) / l[:, None]
    else:
        for r, (lo, hi) in enumerate(bounds):
            out[r] = (E[r, lo - u0:hi - u0 + 1] @ Vu[lo - u0:hi - u0 + 1]) / l[r]
    lse[:] = m + np.log(l)
    return out, lse, E / l[:, None], bounds, u0


def _rows_per_block(n_keys: int, budget: int = 8_000_000) -> int:
    return max(1, budget // max(n_keys, 1))


def attention(inp, return_probs: bool = False):
    """Full attention of every query row.

    Returns (out float64 [T, Hq, D], lse float64 [T, Hq]) and, if asked, a
    dict (t, h) -> (lo, probabilities over keys lo..p_t).
    """
    T = int(inp.q.shape[0])
    Hq, Hk, D = int(inp.num_q_heads), int(inp.num_kv_heads), int(inp.head_dim)
    G = Hq // Hk
    scale64 = float(np.float32(inp.scale))
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    probs = {} if return_probs else None
    cu = _cu_q(inp)
    live_index = _live_index(inp)
    for b in range(len(inp.seq_lens)):
        s, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
        if ql == 0:
            continue
        pos = query_positions(s, ql)
        lo_all = visible_bounds(int(pos[0]), inp.window)[0]
        for g in range(Hk):
            K = depage(inp, "k", b, g, lo_all, s, live_index)
            V = depage(inp, "v", b, g, lo_all, s, live_index)
            # rows in (token, head-in-group) order
            rows = [(i, g * G + hh) for i in range(ql) for hh in range(G)]
            step = _rows_per_block(s - lo_all)
            for r0 in range(0, len(rows), step):
                blk = rows[r0:r0 + step]
                qrows = np.stack([_q_row(inp, int(cu[b]) + i, h) for i, h in blk])
                ppos = np.array([pos[i] for i, _ in blk])
                o, l, Pm, bounds, u0 = _rows_attention(qrows, ppos, K, V, lo_all, inp.window, scale64)
                for k, (i, h) in enumerate(blk):
                    t = int(cu[b]) + i
                    out[t, h] = o[k]
                    lse[t, h] = l[k]
                    if probs is not None:
                        lo, hi = bounds[k]
                        probs[(t, h)] = (lo, Pm[k, lo - u0:hi - u0 + 1].copy())
    if return_probs:
        return out, lse, probs
    return out, lse


def attention_rows(inp, rows: Iterable[Tuple[int, int]]) -> Dict[Tuple[int, int], Tuple[np.ndarray, float]]:
    """Attention of selected (token t, query head h) rows only.

    Used at full workload sizes, where computing every row would be slow.
    """
    Hq, Hk = int(inp.num_q_heads), int(inp.num_kv_heads)
    G = Hq // Hk
    scale64 = float(np.float32(inp.scale))
    cu = _cu_q(inp)
    live_index = _live_index(inp)
    by_group: Dict[Tuple[int, int], List[Tuple[int, int, int]]] = {}
    for t, h in rows:
        b = int(np.searchsorted(cu, t, side="right") - 1)
        by_group.setdefault((b, h // G), []).append((t, h, t - int(cu[b])))
    res = {}
    for (b, g), lst in by_group.items():
        s, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
        pos = query_positions(s, ql)
        lo_all = min(visible_bounds(int(pos[i]), inp.window)[0] for _, _, i in lst)
        hi_all = max(int(pos[i]) for _, _, i in lst) + 1
        K = depage(inp, "k", b, g, lo_all, hi_all, live_index)
        V = depage(inp, "v", b, g, lo_all, hi_all, live_index)
        qrows = np.stack([_q_row(inp, t, h) for t, h, _ in lst])
        ppos = np.array([pos[i] for _, _, i in lst])
        o, l, _, _, _ = _rows_attention(qrows, ppos, K, V, lo_all, inp.window, scale64)
        for k, (t, h, _) in enumerate(lst):
            res[(t, h)] = (o[k], float(l[k]))
    return res


# ---------------------------------------------------------------- split + merge

def row_partial(inp, t: int, h: int, key_lo: int, key_hi: int):
    """Attention of one row over its visible keys that fall in [key_lo, key_hi).

    Returns (out [D], lse); an empty key set gives (zeros, -inf).  Splitting
    the context into pieces and merging the pieces' partial results is how
    the pages' decode kernel keeps every compute unit busy ("Dual MI50,
    part 2", section "Decode: a new kernel for the shape MTP actually runs").
    """
    Hq, Hk, D = int(inp.num_q_heads), int(inp.num_kv_heads), int(inp.head_dim)
    G = Hq // Hk
    cu = _cu_q(inp)
    b = int(np.searchsorted(cu, t, side="right") - 1)
    i = t - int(cu[b])
    s, ql = int(inp.seq_lens[b]), int(inp.q_lens[b])
    p = int(query_positions(s, ql)[i])
    lo, hi = visible_bounds(p, inp.window)
    lo, hi = max(lo, key_lo), min(hi, key_hi - 1)
    if hi < lo:
        return np.zeros(D), NEG_INF
    K = depage(inp, "k", b, h // G, lo, hi + 1)
    V = depage(inp, "v", b, h // G, lo, hi + 1)
    q = _q_row(inp, t, h)
    sc = float(np.float32(inp.scale)) * (K @ q)
    m = sc.max()
    e = np.exp(sc - m)
    l = e.sum()
    return (e @ V) / l, m + np.log(l)


def merge_partials(parts: Sequence[Tuple[np.ndarray, float]]):
    """Combine (out_s, lse_s) over disjoint key sets into (out, lse).

    lse = M + ln sum_s exp(lse_s - M) with M = max_s lse_s, and
    out = sum_s exp(lse_s - lse) out_s.  Exact in real arithmetic.
    """
    lses = np.array([l for _, l in parts], dtype=np.float64)
    M = lses.max()
    if M == NEG_INF:
        return np.zeros_like(parts[0][0]), NEG_INF
    w = np.exp(lses - M)
    L = w.sum()
    lse = M + np.log(L)
    out = sum(np.exp(l - lse) * o for o, l in parts)
    return out, lse
