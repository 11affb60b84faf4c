/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged-attention library.
 *
 * The library computes attention of a few new query rows against a long,
 * growing KV cache that is stored in fixed-size pages and addressed through
 * a block table:
 *
 *     out[t, h, :] = sum_j softmax_j(scale * q[t, h, :] . k~[g, j, :]) v~[g, j, :]
 *     lse[t, h]    = ln sum_j exp(scale * q[t, h, :] . k~[g, j, :])
 *
 * over the keys j that row t may see, with query head h reading KV head
 * g = h / (Hq / Hkv) (grouped-query attention: several query heads share each
 * KV head, "Dual MI50, part 2", section "Decode: a new kernel for the shape
 * MTP actually runs").  k~, v~ are the cached values after dequantisation.
 *
 * Positions.  A sequence's seq_len counts every cached token including its
 * q_len new ones; the new tokens' keys and values are already in the cache
 * as its last q_len entries, and new row i sits at position
 * p_i = seq_len - q_len + i.  Row i sees key j iff j <= p_i (causal inside
 * the new rows: speculative verification scores k+1 tokens in one pass,
 * "Dual MI50, part 2", section "Kernels: why the generic code is slow here")
 * and, when window W >= 1, j >= p_i - W + 1 (the W most recent keys, the
 * drafter's sliding window of "Dual MI50, part 2", section "Bug 2: the
 * drafter read freed memory").  Pages whose tokens all lie before the first
 * row's window, slots past seq_len and unused block-table entries are never
 * read, so their contents (freed and reused pages, NaN) cannot reach the
 * output.
 *
 * The cache is read in place, with no copies ("Dual MI50, part 2", section
 * "Prefill: teach the fork's fast kernel to read the int8 cache"), and
 * forward allocates nothing and never waits on the host, so it can be
 * captured in a HIP graph ("Dual MI50, part 2", section "Decode: a new
 * kernel for the shape MTP actually runs").
 *
 * Conventions shared by every entry point:
 *   - return value: PA_OK (0) or a PA_ERR_* code; paged_attn_last_error()
 *     gives a message.  Nothing is launched when an argument is rejected.
 *   - pointers named "device" must be device memory of the handle's GPU;
 *     "host" pointers are read before the call returns.
 *   - the caller owns every tensor and the stream; the handle owns only its
 *     device workspace.
 *   - all work is enqueued on `stream` (a hipStream_t, NULL = default
 *     stream); results are visible once the stream reaches that point.
 *   - a handle may be used by one stream at a time (its workspace is shared
 *     between calls); use one handle per concurrent stream.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PA_OK                    0
#define PA_ERR_INVALID_ARGUMENT  1
#define PA_ERR_UNSUPPORTED       2
#define PA_ERR_OUT_OF_MEMORY     3
#define PA_ERR_HIP               4

/* element types */
#define PA_DTYPE_F16       1   /* IEEE binary16 */
#define PA_DTYPE_BF16      2   /* bfloat16 */
#define PA_DTYPE_FP8_E4M3  3   /* OCP E4M3FN: bias 7, max 448, no inf, S.1111.111 = NaN */
#define PA_DTYPE_INT8      4   /* two's-complement int8 codes, one fp32 scale per cached row */

/* pa_config_t.flags */
#define PA_DEBUG_CHECKS    1   /* device-checked mode, see paged_attn_debug_status */

/* bits of the device error word of the checked mode */
#define PA_CHECK_LENGTHS   1   /* q_len < 0, q_len > seq_len, q_len > max_q_len or seq_len < 0 */
#define PA_CHECK_TABLE     2   /* a sequence needs more pages than its block-table row holds */
#define PA_CHECK_PAGE      4   /* a block-table entry that is read lies outside [0, num_pages) */
#define PA_CHECK_TOKENS    8   /* the q_lens add up to more than num_tokens */

/* execution paths (pa_tuning_t.path) */
#define PA_PATH_AUTO   0   /* head_dim 128: VALU split-KV kernel for <= 8 rows per KV head over a short
                              block table (batches: <= 16,384 tokens; a single sequence: <= 1,536),
                              MFMA tile kernel otherwise; head_dim 64: VALU; head_dim 256: VALU up
                              to 64 rows per KV head, then the tile kernel past 8 */
#define PA_PATH_VALU   1   /* every sequence through the VALU split-KV kernel (handles whose
                              max_q_len * Hq / Hkv is at most 64; else PA_ERR_UNSUPPORTED) */
#define PA_PATH_MFMA   2   /* every sequence through the MFMA tile kernel (head_dim 128 or 256) */

typedef struct pa_config {
    int32_t num_q_heads;     /* Hq >= 1 */
    int32_t num_kv_heads;    /* Hkv >= 1, Hq % Hkv == 0, Hq / Hkv <= 16 */
    int32_t head_dim;        /* D: 64, 128 or 256.  64 runs on the VALU kernel only and needs
                                max_q_len * Hq / Hkv <= 64 (else PA_ERR_UNSUPPORTED at create).
                                256: the VALU kernel takes every sequence while no row count
                                passes 64 per KV head; past that (chunked prefill) a tile kernel
                                with 128-row items takes the sequences of more than 8 rows. */
    int32_t page_size;       /* P: tokens per page, a multiple of 16 in 16..65536 (the cache is read in
                                place at any such block size: "Dual MI50, part 2", section "Prefill:
                                teach the fork's fast kernel to read the int8 cache"; the pages use
                                1,056- and 1,584-token pages).  With P > 16 the layout's page stride
                                must be a multiple of 16 token rows (true of HND and NHD), num_pages
                                x page_stride / (16 x token_stride) below 2^31, and
                                block_table_stride x P below 2^28 (else PA_ERR_UNSUPPORTED). */
    int32_t q_dtype;         /* PA_DTYPE_F16 or PA_DTYPE_BF16 */
    int32_t kv_dtype;        /* PA_DTYPE_F16, PA_DTYPE_BF16 (== q_dtype), PA_DTYPE_FP8_E4M3 or
                                PA_DTYPE_INT8 (the pages' own cache: int8 codes with a fp32 scale per
                                row, "Dual MI50, part 2", section "Prefill: teach the fork's fast kernel
                                to read the int8 cache") */
    int32_t max_num_seqs;    /* largest num_seqs passed to forward, 1..1024 */
    int32_t max_q_len;       /* largest q_len of any sequence, >= 1 */
    int32_t min_q_len;       /* smallest q_len of any sequence with q_len > 0 (1..max_q_len); a
                                hint: kernels for narrower rows are not launched */
    int64_t max_num_tokens;  /* largest T = sum of q_lens, >= 1 */
    int32_t device;          /* HIP device ordinal the handle runs on */
    int32_t flags;           /* 0 or PA_DEBUG_CHECKS; other bits must be 0 */
} pa_config_t;

/* Physical layout of the K and V page pools (identical for both).  Strides
 * are in elements.  Within a token the D elements are contiguous; a token
 * row must start on a 16-byte boundary.  The default (HND) layout
 * [num_pages][Hkv][P][D] has page_stride = Hkv*P*D, head_stride = P*D,
 * token_stride = D, so each (page, head) block is one contiguous run. */
typedef struct pa_cache_layout {
    int64_t num_pages;
    int64_t page_stride;
    int64_t head_stride;
    int64_t token_stride;
} pa_cache_layout_t;

/* Optional knobs, mainly for tests and measurement.  Zero means automatic. */
typedef struct pa_tuning {
    int32_t path;             /* PA_PATH_* */
    int32_t pages_per_split;  /* VALU kernel: KV pages per split (0: sized from the live context) */
    int32_t kv_tiles_per_split; /* MFMA kernel: key tiles per split (32-key tiles; 64-key for
                                   fp8 caches at prefill widths; 0: automatic) */
    int32_t grid;             /* workgroups per launch (0: from the CU count) */
    int32_t split_mode;       /* VALU kernel: 0 automatic, 1 static splits from the block-table
                                 width (one round trip to start), 2 splits planned on the device
                                 from the live lengths (balances mixed lengths) */
} pa_tuning_t;

typedef struct pa_handle pa_handle_t;

/*
 * paged_attn_create: validate `cfg`, allocate the device workspace on
 * cfg->device (split partials and merge counters, sized from the maxima in
 * cfg) and return a handle in *out.  Returns PA_ERR_INVALID_ARGUMENT or
 * PA_ERR_UNSUPPORTED (with *out left NULL) for a bad or unsupported config,
 * PA_ERR_OUT_OF_MEMORY if the workspace cannot be allocated, PA_ERR_HIP for
 * other runtime failures.  May synchronise the device once (workspace
 * clearing); forward never does.
 */
int paged_attn_create(const pa_config_t* cfg, pa_handle_t** out);

/*
 * paged_attn_forward: enqueue attention of every sequence's new rows.
 *
 *  q            device, [T][Hq][D] of cfg.q_dtype, rows packed by sequence
 *               (sequence b's q_len rows follow sequence b-1's); 16-B aligned.
 *  num_tokens   host int: T = sum of q_lens (1..cfg.max_num_tokens).
 *  k_cache,     device page pools of cfg.kv_dtype laid out per `layout`;
 *  v_cache      16-B aligned.
 *  layout       host, see pa_cache_layout_t.
 *  block_table  device int32 [num_seqs][block_table_stride]: entry
 *               [b][i] is the physical page holding tokens i*P .. i*P+P-1
 *               of sequence b (P = cfg.page_size); entries past the
 *               sequence's last page are never read.
 *  num_seqs     host int, 1..cfg.max_num_seqs.
 *  seq_lens     device int32 [num_seqs]: cached tokens incl. the new ones.
 *  q_lens       device int32 [num_seqs]: new rows, 0 <= q_len <= min(seq_len,
 *               cfg.max_q_len); sum must equal num_tokens.
 *  window       host int: <= 0 no window; W >= 1 the W most recent keys.
 *  scale        host float > 0: multiplies q.k (after dequantisation).
 *  kv_scale     fp8 cache: device float [2][Hkv] (K scales, then V scales):
 *               k~ = code * kv_scale[0][g], v~ = code * kv_scale[1][g];
 *               every scale > 0.
 *               int8 cache: device float [2][R] with R = num_pages *
 *               page_stride / head_dim, one scale per cached row (one token
 *               of one KV head), K rows then V rows: the row of page p, KV
 *               head g, slot s has its scale at index (p * page_stride +
 *               g * head_stride + s * token_stride) / head_dim, i.e. the
 *               scales are laid out like the cache with rows of one element
 *               ([2][pages][Hkv][P] for HND, [2][pages][P][Hkv] for NHD);
 *               k~ = code * scale of its row.  Every stride must be a
 *               multiple of head_dim.  Scales of slots no row reaches are
 *               never read; dead rows' scales may hold anything (NaN).
 *               Must be NULL for fp16/bf16 caches.
 *  out          device float [T][Hq][D].
 *  lse          device float [T][Hq] (natural log), or NULL.
 *  stream       hipStream_t or NULL.
 *
 * Device-array contents (block table, lengths) are trusted: they are not
 * read on the host.  Violating the documented ranges is undefined, unless
 * the handle was created with PA_DEBUG_CHECKS: then the kernels check every
 * sequence's lengths against the block-table width, max_q_len and
 * num_tokens, and every block-table entry they use against num_pages,
 * before the accesses these values steer.  A bad sequence is skipped, a bad
 * page id replaced by page 0, every kernel completes normally, and the kind
 * of fault is recorded for paged_attn_debug_status (the freed-block reads
 * of "Dual MI50, part 2", section "Bug 2: the drafter read freed memory",
 * are this class of error).  The outputs of an affected forward are
 * unspecified.
 * Returns PA_ERR_INVALID_ARGUMENT for a rejected host argument (null or
 * misaligned pointer, size out of range, scale not finite and positive, kv_scale given
 * or missing), PA_ERR_HIP if the launch fails.
 */
int paged_attn_forward(pa_handle_t* h,
                       const void* q, int64_t num_tokens,
                       const void* k_cache, const void* v_cache,
                       const pa_cache_layout_t* layout,
                       const int32_t* block_table, int32_t num_seqs, int32_t block_table_stride,
                       const int32_t* seq_lens, const int32_t* q_lens,
                       int32_t window, float scale, const float* kv_scale,
                       float* out, float* lse, void* stream);

/* paged_attn_destroy: free the workspace and the handle (NULL is a no-op).
 * Does not synchronise: the caller must make sure no enqueued forward on the
 * handle is still running. */
void paged_attn_destroy(pa_handle_t* h);

/* paged_attn_last_error: message of the last failed call on `h` (or of the
 * last failed create / handle-less call on this thread when h is NULL);
 * "" if none.  Valid until the next call on the same handle / thread.  On a
 * handle created with PA_DEBUG_CHECKS it first collects the device error
 * word as paged_attn_debug_status does (a synchronous device read: call it
 * once the stream work has finished), so a fault the kernels recorded is
 * the message. */
const char* paged_attn_last_error(const pa_handle_t* h);

/*
 * paged_attn_debug_status: on a handle created with PA_DEBUG_CHECKS, reads
 * the device error word that forward and append set (a synchronous device
 * read: the caller synchronises its stream first), stores its PA_CHECK_*
 * bits in *bits_out (may be NULL), clears it, and returns PA_OK if it was 0
 * or PA_ERR_INVALID_ARGUMENT with a message naming the faults.  Returns
 * PA_ERR_UNSUPPORTED on a handle without the flag, PA_ERR_HIP if the read
 * fails.
 */
int paged_attn_debug_status(pa_handle_t* h, int32_t* bits_out);

/* paged_attn_set_tuning: replace the handle's knobs (NULL restores the
 * defaults).  Results stay within the stated tolerances for every setting;
 * only speed and the summation order change. */
int paged_attn_set_tuning(pa_handle_t* h, const pa_tuning_t* t);

/*
 * paged_attn_debug_gather: de-page K through the same address computation
 * the attention kernels use.  For every sequence b and every token j of its
 * visible range [lo_b, seq_len_b) (lo_b = max(0, seq_len_b - q_len_b - W + 1)
 * when window W >= 1, else 0), in order of b then j, it writes the token's
 * physical slot index (page * P + slot) to slots_out and the raw bytes of
 * its Hkv x D elements (KV head major) to rows_out.  Sequences with
 * q_len == 0 contribute nothing.
 *
 *  slots_out   device int64 [n_visible]
 *  rows_out    device bytes [n_visible][Hkv][D * element size]
 *  capacity    host int: entries slots_out / rows_out can hold; tokens past
 *              it are not written.
 *  Other arguments as in paged_attn_forward.
 */
int paged_attn_debug_gather(pa_handle_t* h,
                            const void* k_cache, const pa_cache_layout_t* layout,
                            const int32_t* block_table, int32_t num_seqs, int32_t block_table_stride,
                            const int32_t* seq_lens, const int32_t* q_lens, int32_t window,
                            int64_t* slots_out, void* rows_out, int64_t capacity, void* stream);

/*
 * paged_attn_append: write a step's new K and V rows into their pages, the
 * step just before attention reads them ("Dual MI50, part 2", sections
 * "Bug 2: the drafter read freed memory" and "Prefill: teach the fork's
 * fast kernel to read the int8 cache").  Sequence b's rows are its last
 * q_len_b positions (seq_len_b counts them): its row i is logical position
 * p = seq_len_b - q_len_b + i, stored in page block_table[b][p / P], slot
 * p % P, for every KV head.  A 16-bit cache receives the input bits
 * unchanged; an fp8 E4M3FN cache receives, per element, the code nearest to
 * x / s (s = kv_scale[0][g] for K, kv_scale[1][g] for V; the quotient
 * rounded once in fp32), ties to the even code, magnitudes of 448 and more
 * (and infinities) stored as 448, NaN as NaN, the sign kept.  An int8 cache
 * receives, per row (one token of one KV head), the scale s = amax / 127
 * (amax the largest |x| of the row's D values, NaN if one is NaN; fp32
 * division), written to the row's place in the row-scale pool kv_scale
 * (laid out as in paged_attn_forward), and per element the integer nearest
 * to x / s (one fp32 division, ties to even) limited to [-127, 127], a NaN
 * quotient (a zero or non-finite row) stored as 0.
 *
 *  k_new, v_new  device, q_dtype, contiguous [num_tokens][Hkv][D], rows of
 *                sequence 0 first; 16-byte aligned.  Read only.
 *  k_cache, v_cache, layout, block_table, num_seqs, block_table_stride,
 *  seq_lens, q_lens, kv_scale, stream: as in paged_attn_forward (the caches
 *                are written; kv_scale is required for an fp8 cache, which
 *                only reads it, and for an int8 cache, whose row scales of
 *                the written rows it receives; NULL otherwise).
 *
 * Only the addressed slots are written.  A sequence with q_len <= 0,
 * q_len > seq_len, or rows past num_tokens writes nothing; a row whose
 * position lies past the block table's width, or whose page id is outside
 * [0, num_pages), is skipped.  Asynchronous on `stream`; allocates nothing.
 * Returns PA_OK or PA_ERR_INVALID_ARGUMENT / PA_ERR_UNSUPPORTED (host
 * checks, nothing enqueued) or PA_ERR_HIP.
 */
int paged_attn_append(pa_handle_t* h, const void* k_new, const void* v_new, int64_t num_tokens,
                      void* k_cache, void* v_cache, const pa_cache_layout_t* layout,
                      const int32_t* block_table, int32_t num_seqs, int32_t block_table_stride,
                      const int32_t* seq_lens, const int32_t* q_lens, float* kv_scale, void* stream);

/*
 * paged_attn_forward_noalloc: paged_attn_forward for callers that cannot
 * allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes the configuration
 * instead of a handle and allocates nothing: its split partials, merge
 * descriptors and counters live in one fixed device array of
 * PA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends (set up on the first call on a device).
 *
 *  cfg          host, validated as in paged_attn_create (default tuning).
 *  other arguments as in paged_attn_forward; the result is the same as a
 *               handle created from cfg would give.
 *
 * Each call first zeroes, with a small kernel on `stream`, the counters the
 * kernels expect at zero.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams, threads) race and give
 * wrong results; serialise them.  A configuration whose workspace exceeds
 * the array -- prefill-sized row counts, large batches -- is rejected with
 * PA_ERR_UNSUPPORTED and a message naming the size it needs, as is
 * cfg->flags = PA_DEBUG_CHECKS (its error word belongs to a handle); decode and
 * verification widths of the usual head counts fit.  Errors are reported by
 * paged_attn_last_error(NULL) on the calling thread.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_attn_forward_noalloc(const pa_config_t* cfg,
                               const void* q, int64_t num_tokens,
                               const void* k_cache, const void* v_cache,
                               const pa_cache_layout_t* layout,
                               const int32_t* block_table, int32_t num_seqs, int32_t block_table_stride,
                               const int32_t* seq_lens, const int32_t* q_lens,
                               int32_t window, float scale, const float* kv_scale,
                               float* out, float* lse, void* stream);

/* paged_attn_version: library version, e.g. "0.2.0". */
const char* paged_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
