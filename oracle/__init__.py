"""fp64 CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import or run anything in this package.  The library and its Python
binding never call it: there is no CPU fallback for the GPU path.

What it computes is the plain definition of attention of a few new query
rows against a paged KV cache:

    out = softmax(scale * Q K^T + mask) V,   lse = log sum exp(scale * Q K^T + mask)

with grouped-query heads (query head h reads KV head h // (Hq/Hkv)), a causal
mask inside the new rows, an optional sliding window, and a dequantised fp8
(per-head scales) or int8 (per-row scales) cache.  The cache is first copied out of its pages into a dense, logical
token order (an explicit de-paging step), then every sum runs only over the
keys a row may see, in float64.  Sources: "Dual MI50, part 2" (blog.sbm-labs
.com), sections "Bug 2: the drafter read freed memory", "Kernels: why the
generic code is slow here", "Prefill: teach the fork's fast kernel to read
the int8 cache", "Decode: a new kernel for the shape MTP actually runs" and
"Did quality change?".

It shares no code with the HIP path; its only inputs are the storage bits and
integer metadata that the seeded generator produces.
"""
from .codec import decode_bits, fp8_e4m3_table  # noqa: F401
from .append import append_kv, e4m3_encode, int8_encode_row, new_row_positions  # noqa: F401
from .attention import (  # noqa: F401
    attention,
    attention_rows,
    depage,
    row_partial,
    merge_partials,
    query_positions,
    visible_bounds,
)
from .bruteforce import dense_attention_bruteforce  # noqa: F401
