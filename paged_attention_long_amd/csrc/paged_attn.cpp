// Host side of the paged-attention C ABI: argument validation, workspace
// ownership and kernel dispatch.  Every entry point validates its host
// arguments before touching the GPU, so rejected calls launch nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "paged_attn.h"
#include "pa_kernels.h"

struct pa_handle {
    pa_config_t cfg;
    pa_tuning_t tune;
    int cu_count = 0;
    int grid_default = 0;
    int max_items_valu = 0;  // split-partial slots of the VALU kernel
    int r_max_valu = 0;      // rows per VALU slot (largest rows-per-KV-head it may handle)
    bool valu_all_ok = false;  // the VALU kernel's slots hold every sequence's rows
    int mfma_wr = 1;         // MFMA kernel: waves along rows (rows per item = 32 * mfma_wr)
    int max_items_mfma = 0;
    int mfma_grid = 0;       // tile-kernel workgroups: one per resident slot
    int merge_rows = 0;      // largest row count of one merge group
    int mfma_item_off = 0;   // first partial item of the tile kernel
    int desc_cap = 0;        // merge descriptors the workspace holds
    float* ws_o = nullptr;
    float* ws_lse = nullptr;
    pa::MergeDesc* mdesc = nullptr;   // merge groups published by the attention kernels
    pa::MergeDesc* sdesc = nullptr;   // fixed merge slots for static splits (zeroed; each merge clears what it used)
    int* arrive = nullptr;            // per-group arrival counters for static splits merged in-kernel (zeroed; the last arrival clears its own)
    int sdesc_upg = 1;                // merge units per (sequence, KV head) group in sdesc
    int64_t sdesc_groups = 0;         // groups sdesc holds
    int* mcount = nullptr;            // [0] groups published, [1] merge workgroups done
    void* ws = nullptr;
    size_t ws_bytes = 0;
    std::string err;
};

namespace {

thread_local std::string g_err;

int fail(pa_handle* h, int code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
int fail(pa_handle* h, int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (h) h->err = buf; else g_err = buf;
    return code;
}

int elem_bytes(int dt) { return dt == PA_DTYPE_FP8_E4M3 ? 1 : 2; }

int pow2ceil(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMinPagesPerSplit = 4;
constexpr int kValuRowsMax = 8;   // rows per KV head handled by the VALU kernel under PA_PATH_AUTO
constexpr int kValuMaxKeys = 16384;   // and visible keys (longer contexts go to the tile kernel)

int validate_config(const pa_config_t* c, std::string* why) {
    char buf[256];
    auto bad = [&](int code, const char* msg) { *why = msg; return code; };
    if (!c) return bad(PA_ERR_INVALID_ARGUMENT, "config is NULL");
    if (c->num_q_heads < 1 || c->num_kv_heads < 1) return bad(PA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
    if (c->num_q_heads % c->num_kv_heads) return bad(PA_ERR_INVALID_ARGUMENT, "num_q_heads % num_kv_heads != 0");
    if (c->num_q_heads / c->num_kv_heads > 16) return bad(PA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
    if (c->head_dim != 64 && c->head_dim != 128) return bad(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (c->page_size != 16) return bad(PA_ERR_UNSUPPORTED, "page_size must be 16");
    if (c->q_dtype != PA_DTYPE_F16 && c->q_dtype != PA_DTYPE_BF16)
        return bad(PA_ERR_UNSUPPORTED, "q_dtype must be F16 or BF16");
    if (c->kv_dtype != PA_DTYPE_F16 && c->kv_dtype != PA_DTYPE_BF16 && c->kv_dtype != PA_DTYPE_FP8_E4M3)
        return bad(PA_ERR_UNSUPPORTED, "kv_dtype must be F16, BF16 or FP8_E4M3");
    if (c->kv_dtype != PA_DTYPE_FP8_E4M3 && c->kv_dtype != c->q_dtype)
        return bad(PA_ERR_UNSUPPORTED, "a 16-bit cache must have the query's dtype");
    if (c->max_num_seqs < 1 || c->max_num_seqs > 1024) return bad(PA_ERR_INVALID_ARGUMENT, "max_num_seqs must be 1..1024");
    if (c->max_q_len < 1) return bad(PA_ERR_INVALID_ARGUMENT, "max_q_len must be >= 1");
    if (c->min_q_len < 1 || c->min_q_len > c->max_q_len)
        return bad(PA_ERR_INVALID_ARGUMENT, "min_q_len must be 1..max_q_len");
    if (c->head_dim == 64 && (int64_t)c->max_q_len * (c->num_q_heads / c->num_kv_heads) > 64)
        return bad(PA_ERR_UNSUPPORTED, "head_dim 64 supports at most 64 rows per KV head");
    if (c->max_num_tokens < 1 || c->max_num_tokens > (int64_t)1 << 24)
        return bad(PA_ERR_INVALID_ARGUMENT, "max_num_tokens must be 1..2^24");
    if ((int64_t)c->max_q_len * (c->num_q_heads / c->num_kv_heads) > (1 << 20))
        return bad(PA_ERR_UNSUPPORTED, "max_q_len * group too large");
    if (c->flags != 0) return bad(PA_ERR_INVALID_ARGUMENT, "flags must be 0");
    if (c->device < 0) return bad(PA_ERR_INVALID_ARGUMENT, "device must be >= 0");
    (void)buf;
    return PA_OK;
}

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) return;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

}  // namespace

extern "C" {

const char* paged_attn_version(void) { return "0.1.0"; }

const char* paged_attn_last_error(const pa_handle_t* h) { return h ? h->err.c_str() : g_err.c_str(); }

int paged_attn_create(const pa_config_t* cfg, pa_handle_t** out) {
    if (!out) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    std::string why;
    int rc = validate_config(cfg, &why);
    if (rc != PA_OK) return fail(nullptr, rc, "%s", why.c_str());

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= cfg->device)
        return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "device %d not present (%d devices)", cfg->device, ndev);
    DeviceGuard guard(cfg->device);
    if (!guard.ok) return fail(nullptr, PA_ERR_HIP, "hipSetDevice(%d) failed", cfg->device);

    pa_handle* h = new (std::nothrow) pa_handle();
    if (!h) return fail(nullptr, PA_ERR_OUT_OF_MEMORY, "host allocation failed");
    h->cfg = *cfg;
    std::memset(&h->tune, 0, sizeof h->tune);
    if (hipDeviceGetAttribute(&h->cu_count, hipDeviceAttributeMultiprocessorCount, cfg->device) != hipSuccess ||
        h->cu_count <= 0)
        h->cu_count = 256;
    h->grid_default = 2 * h->cu_count;

    const int G = cfg->num_q_heads / cfg->num_kv_heads;
    const int D = cfg->head_dim;
    const int64_t rows_max = (int64_t)cfg->max_q_len * G;
    // Split-partial slots.  Each kernel raises its split size until its items
    // fit: the VALU kernel has at most grid + one item per (sequence, KV head),
    // the MFMA kernel grid + one per (sequence, KV head, row block).
    const int grid_cap = 8 * h->cu_count;
    h->valu_all_ok = rows_max <= 64;
    h->r_max_valu = (int)(h->valu_all_ok ? rows_max : kValuRowsMax);
    h->max_items_valu = grid_cap + cfg->max_num_seqs * cfg->num_kv_heads;
    // rows per tile-kernel item: 32 (verification widths), else 256 rows over
    // eight waves for 16-bit caches and 128 over four for fp8
    h->mfma_wr = rows_max > 64 ? (cfg->kv_dtype == PA_DTYPE_FP8_E4M3 ? 4 : 8) : 1;
    // The tile kernel launches exactly one round of resident workgroups; its
    // in-kernel plan sizes the splits for that many items.
    h->mfma_grid = D == 128 ? h->cu_count * pa::mfma_blocks_per_cu(cfg->kv_dtype, cfg->q_dtype, h->mfma_wr,
                                                                    cfg->max_num_seqs)
                            : h->cu_count;
    const int bm = 32 * h->mfma_wr;
    const int64_t qblocks = ((int64_t)cfg->max_num_tokens * G + bm - 1) / bm + cfg->max_num_seqs;
    h->max_items_mfma = (int)std::min<int64_t>((int64_t)1 << 30, grid_cap + qblocks * cfg->num_kv_heads);
    h->merge_rows = (int)std::max<int64_t>(h->r_max_valu, D == 128 ? bm : 0);
    // The two kernels' partials live side by side until the merge launch: VALU
    // slots first, then the tile kernel's, starting at a whole tile item.
    const size_t valu_slots = ((size_t)h->max_items_valu * h->r_max_valu + bm - 1) / bm * bm;
    h->mfma_item_off = (int)(valu_slots / bm);
    const size_t slots = valu_slots + (D == 128 ? (size_t)h->max_items_mfma * bm : (size_t)0);
    const size_t o_bytes = slots * D * sizeof(float);
    const size_t l_bytes = slots * sizeof(float);
    // a merge group has at least two items
    h->desc_cap = (int)std::max<size_t>(1, ((size_t)h->max_items_valu + (D == 128 ? (size_t)h->max_items_mfma : 0)) / 2);
    const size_t d_bytes = (size_t)h->desc_cap * sizeof(pa::MergeDesc);
    const size_t c_bytes = 2 * sizeof(int);
    // Fixed slots for the VALU kernel's static splits (at most 8 workgroups
    // per CU, so at most that many (sequence, KV head) groups).
    h->sdesc_upg = (h->r_max_valu + pa::merge_rows_per_unit(D) - 1) / pa::merge_rows_per_unit(D);
    h->sdesc_groups = std::min<int64_t>((int64_t)cfg->max_num_seqs * cfg->num_kv_heads, (int64_t)8 * h->cu_count);
    const size_t s_bytes = (size_t)h->sdesc_groups * h->sdesc_upg * sizeof(pa::MergeDesc);
    const size_t a_bytes = (size_t)h->sdesc_groups * sizeof(int);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    h->ws_bytes = up(o_bytes) + up(l_bytes) + up(d_bytes) + up(c_bytes) + up(s_bytes) + up(a_bytes);
    if (hipMalloc(&h->ws, h->ws_bytes) != hipSuccess) {
        const size_t want = h->ws_bytes;
        delete h;
        (void)hipGetLastError();
        return fail(nullptr, PA_ERR_OUT_OF_MEMORY, "workspace of %zu bytes could not be allocated", want);
    }
    char* p = static_cast<char*>(h->ws);
    h->ws_o = reinterpret_cast<float*>(p);
    h->ws_lse = reinterpret_cast<float*>(p + up(o_bytes));
    h->mdesc = reinterpret_cast<pa::MergeDesc*>(p + up(o_bytes) + up(l_bytes));
    h->mcount = reinterpret_cast<int*>(p + up(o_bytes) + up(l_bytes) + up(d_bytes));
    h->sdesc = reinterpret_cast<pa::MergeDesc*>(p + up(o_bytes) + up(l_bytes) + up(d_bytes) + up(c_bytes));
    h->arrive = reinterpret_cast<int*>(p + up(o_bytes) + up(l_bytes) + up(d_bytes) + up(c_bytes) + up(s_bytes));
    if (hipMemset(h->mcount, 0, up(c_bytes) + up(s_bytes) + up(a_bytes)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(h->ws);
        delete h;
        return fail(nullptr, PA_ERR_HIP, "workspace clear failed");
    }
    *out = h;
    return PA_OK;
}

void paged_attn_destroy(pa_handle_t* h) {
    if (!h) return;
    if (h->ws) {
        DeviceGuard guard(h->cfg.device);
        (void)hipFree(h->ws);
    }
    delete h;
}

int paged_attn_set_tuning(pa_handle_t* h, const pa_tuning_t* t) {
    if (!h) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (!t) {
        std::memset(&h->tune, 0, sizeof h->tune);
        return PA_OK;
    }
    if (t->path < PA_PATH_AUTO || t->path > PA_PATH_MFMA) return fail(h, PA_ERR_INVALID_ARGUMENT, "bad path %d", t->path);
    if (t->path == PA_PATH_MFMA && h->cfg.head_dim != 128)
        return fail(h, PA_ERR_UNSUPPORTED, "the MFMA path needs head_dim 128");
    if (t->path == PA_PATH_VALU && !h->valu_all_ok)
        return fail(h, PA_ERR_UNSUPPORTED, "the VALU path holds at most 64 rows per KV head");
    if (t->pages_per_split < 0 || t->kv_tiles_per_split < 0 || t->grid < 0 || t->grid > 8 * h->cu_count ||
        t->split_mode < 0 || t->split_mode > 2)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "tuning values out of range (grid <= %d)", 8 * h->cu_count);
    h->tune = *t;
    return PA_OK;
}

static int validate_cache(pa_handle* h, const pa_cache_layout_t* L, const void* k, const void* v) {
    const pa_config_t& c = h->cfg;
    const int eb = elem_bytes(c.kv_dtype);
    if (!L) return fail(h, PA_ERR_INVALID_ARGUMENT, "layout is NULL");
    if (!k || !v) return fail(h, PA_ERR_INVALID_ARGUMENT, "k_cache / v_cache is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(h, PA_ERR_INVALID_ARGUMENT, "caches must be 16-byte aligned");
    if (L->num_pages < 1) return fail(h, PA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
    if (L->page_stride < 1 || L->head_stride < 1 || L->token_stride < c.head_dim)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "strides must be positive and token_stride >= head_dim");
    if ((L->page_stride * eb) % 16 || (L->head_stride * eb) % 16 || (L->token_stride * eb) % 16)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "every stride must be a multiple of 16 bytes");
    if (L->num_pages > ((int64_t)1 << 31)) return fail(h, PA_ERR_INVALID_ARGUMENT, "num_pages must fit in int32");
    return PA_OK;
}

int paged_attn_forward(pa_handle_t* h, const void* q, int64_t num_tokens, const void* k_cache, const void* v_cache,
                       const pa_cache_layout_t* layout, const int32_t* block_table, int32_t num_seqs,
                       int32_t block_table_stride, const int32_t* seq_lens, const int32_t* q_lens, int32_t window,
                       float scale, const float* kv_scale, float* out, float* lse, void* stream) {
    if (!h) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "handle is NULL");
    const pa_config_t& c = h->cfg;
    if (!q || !out || !block_table || !seq_lens || !q_lens)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "q, out, block_table, seq_lens and q_lens must be non-NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(h, PA_ERR_INVALID_ARGUMENT, "q and out must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(h, PA_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    if (num_tokens < 1 || num_tokens > c.max_num_tokens)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "num_tokens %lld outside 1..%lld", (long long)num_tokens,
                    (long long)c.max_num_tokens);
    if (num_seqs < 1 || num_seqs > c.max_num_seqs)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "num_seqs %d outside 1..%d", num_seqs, c.max_num_seqs);
    if (block_table_stride < 1) return fail(h, PA_ERR_INVALID_ARGUMENT, "block_table_stride must be >= 1");
    if (!std::isfinite(scale) || !(scale > 0.f)) return fail(h, PA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if ((c.kv_dtype == PA_DTYPE_FP8_E4M3) != (kv_scale != nullptr))
        return fail(h, PA_ERR_INVALID_ARGUMENT, "kv_scale is required for an fp8 cache and must be NULL otherwise");
    int rc = validate_cache(h, layout, k_cache, v_cache);
    if (rc != PA_OK) return rc;

    DeviceGuard guard(c.device);
    if (!guard.ok) return fail(h, PA_ERR_HIP, "hipSetDevice(%d) failed", c.device);

    const int G = c.num_q_heads / c.num_kv_heads;
    pa::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.q_lens = q_lens;
    a.kv_scale = kv_scale;
    a.out = out;
    a.lse = lse;
    a.ws_o = h->ws_o;
    a.ws_lse = h->ws_lse;
    a.mdesc = h->mdesc;
    a.mcount = h->mcount;
    a.sdesc = nullptr;
    a.sdesc_upg = h->sdesc_upg;
    a.arrive = nullptr;
    a.page_stride = layout->page_stride;
    a.head_stride = layout->head_stride;
    a.token_stride = layout->token_stride;
    a.num_seqs = num_seqs;
    a.bt_stride = block_table_stride;
    a.num_q_heads = c.num_q_heads;
    a.num_kv_heads = c.num_kv_heads;
    a.group = G;
    a.window = window;
    a.scale = scale;
    const int grid = h->tune.grid > 0 ? h->tune.grid : h->grid_default;
    a.target_items = grid;
    hipStream_t st = static_cast<hipStream_t>(stream);

    // Each sequence goes to one kernel, decided on the device from its
    // lengths: a few rows per KV head over a short context stream K/V through
    // the vector ALUs (lowest latency); verification widths, prefill chunks
    // and long contexts go to the MFMA tile kernel, whose per-key VALU work is
    // several times smaller.  The host launches a kernel only if some
    // sequence can belong to it.
    const int rows_min = c.min_q_len * G, rows_max = c.max_q_len * G;
    const int64_t cap_tokens = (int64_t)block_table_stride * c.page_size;
    bool run_valu, run_mfma;
    if (c.head_dim != 128 || h->tune.path == PA_PATH_VALU) {
        run_valu = true; run_mfma = false;
        a.cls_rows = 1 << 30; a.cls_len = 1 << 30;
    } else if (h->tune.path == PA_PATH_MFMA) {
        run_valu = false; run_mfma = true;
        a.cls_rows = 0; a.cls_len = 0;
    } else {
        a.cls_rows = kValuRowsMax; a.cls_len = kValuMaxKeys;
        run_valu = rows_min <= kValuRowsMax;
        run_mfma = rows_max > kValuRowsMax || cap_tokens > kValuMaxKeys;
        // A tile launch with 32-row items takes the few-row sequences as well:
        // a VALU launch before it on the same stream would add its whole
        // latency, and per key the tile kernel costs less.  (With prefill-sized
        // items a few-row sequence would fill a small part of each tile.)
        if (run_mfma && h->mfma_wr == 1) {
            run_valu = false;
            a.cls_rows = 0; a.cls_len = 0;
        }
    }
    bool need_merge_valu = run_valu;
    if (run_valu) {
        a.cls_side = 0;
        a.min_pps = kMinPagesPerSplit;
        a.forced_pps = h->tune.pages_per_split;
        a.max_items = h->max_items_valu;
        a.r_max = h->r_max_valu;
        const int rw = std::min(kValuRowsMax, pow2ceil(G));
        // Static splits: a workgroup's (sequence, KV head, split) follows from
        // its index, so its first loads need no plan.  Used for one sequence
        // or a batch whose whole block-table capacity is small; the device
        // plan balances mixed lengths otherwise.
        int vgrid = grid;
        a.static_pps = 0;
        a.static_splits = 0;
        {
            // Pages a VALU-class sequence can reach (static splits count from
            // page 0): without a window its visible keys start at 0.
            const int64_t cap_pages =
                window > 0 ? (int64_t)block_table_stride
                           : std::min<int64_t>(block_table_stride, (int64_t)a.cls_len / c.page_size + 1);
            const int64_t units = (int64_t)num_seqs * c.num_kv_heads * cap_pages;
            // one workgroup per CU: a second resident workgroup on some CUs
            // would double their share of the bytes
            const int sgrid = h->tune.grid > 0 ? h->tune.grid : h->cu_count;
            int64_t pps = h->tune.pages_per_split > 0
                              ? h->tune.pages_per_split
                              : std::max<int64_t>(kMinPagesPerSplit, (units + sgrid - 1) / sgrid);
            pps = std::max<int64_t>(pps, (cap_pages + pa::kMaxSplits - 1) / pa::kMaxSplits);
            if (h->tune.pages_per_split <= 0) pps = (pps + kMinPagesPerSplit - 1) / kMinPagesPerSplit * kMinPagesPerSplit;
            const int64_t S = (cap_pages + pps - 1) / pps;
            const int64_t items = (int64_t)num_seqs * c.num_kv_heads * S;
            const bool small = num_seqs == 1 || units <= (int64_t)4 * kMinPagesPerSplit * grid;
            const bool want = h->tune.split_mode == 1 || (h->tune.split_mode == 0 && small);
            if (want && pps <= pa::kPidChunkPages && items <= h->max_items_valu && items <= 8 * h->cu_count) {
                a.static_pps = (int)pps;
                a.static_splits = (int)S;
                vgrid = (int)items;
                // Alone on the stream, the groups are merged without a merge
                // launch by the last workgroup of each to arrive (small grids:
                // measured faster up to about half the CUs), or else through
                // fixed merge slots.
                if (!run_mfma && S > 1 && (int64_t)num_seqs * c.num_kv_heads <= h->sdesc_groups) {
                    if (vgrid <= h->cu_count / 2) a.arrive = h->arrive;
                    else a.sdesc = h->sdesc;
                }
            }
        }
        hipError_t e = pa::launch_decode_valu(a, c.head_dim, c.kv_dtype, c.q_dtype, rw, vgrid, st);
        if (e != hipSuccess) return fail(h, PA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
        if (a.static_pps > 0 && (a.static_splits == 1 || a.arrive != nullptr)) need_merge_valu = false;
    }
    const bool static_merge = a.sdesc != nullptr;
    const int static_splits = a.static_splits;
    if (run_mfma) {
        a.static_pps = 0;
        a.static_splits = 0;
        a.sdesc = nullptr;
        a.arrive = nullptr;
        a.cls_side = 1;
        a.min_pps = 1;
        a.forced_pps = h->tune.kv_tiles_per_split;
        a.max_items = h->max_items_mfma;
        a.r_max = pa::mfma_rows_per_item(h->mfma_wr);
        a.item_off = h->mfma_item_off;
        const int tgrid = h->tune.grid > 0 ? h->tune.grid : h->mfma_grid;
        a.target_items = tgrid;
        hipError_t e = pa::launch_mfma_attn(a, c.head_dim, c.kv_dtype, c.q_dtype, h->mfma_wr, tgrid, st);
        if (e != hipSuccess) return fail(h, PA_ERR_HIP, "tile launch failed: %s", hipGetErrorString(e));
    }
    if (static_merge && need_merge_valu) {
        // one workgroup per fixed slot; empty slots leave at once
        const int64_t su = (int64_t)num_seqs * c.num_kv_heads * h->sdesc_upg;
        pa::MergeArgs m{h->ws_o,   h->ws_lse,   h->mdesc,     h->mcount,    out,         lse,
                        c.num_q_heads, G,       h->merge_rows, h->desc_cap, h->sdesc, (int)su,
                        h->sdesc_upg,  static_splits, h->r_max_valu};
        hipError_t e = pa::launch_merge(m, c.head_dim, (int)su, 32, st);
        if (e != hipSuccess) return fail(h, PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
    } else if (need_merge_valu || run_mfma) {
        // Merges whatever split groups the launches above published.  Grid:
        // enough workgroups for the most units those launches can publish
        // (each group is merged in units of a few rows).
        const int64_t upg = (h->merge_rows + pa::merge_rows_per_unit(c.head_dim) - 1) / pa::merge_rows_per_unit(c.head_dim);
        int64_t groups = 0;
        if (need_merge_valu) groups += (int64_t)num_seqs * c.num_kv_heads;
        if (run_mfma) {
            const int bm = pa::mfma_rows_per_item(h->mfma_wr);
            groups += (int64_t)c.num_kv_heads * ((num_tokens * G + bm - 1) / bm + num_seqs);
        }
        // Many units (prefill): the low-register variant, four workgroups per
        // CU (every workgroup also takes one turn on the shared arrival
        // counter, so a wider grid costs more than it gains); otherwise at
        // most two per CU, with fewer rows in flight per thread once the grid
        // is wider than the CUs.
        const int64_t units = groups * upg;
        const bool many = units > 4 * (int64_t)h->cu_count;
        const int mgrid = (int)std::max<int64_t>(1, std::min<int64_t>((many ? 4 : 2) * (int64_t)h->cu_count, units));
        const int batch = many ? 8 : (mgrid > h->cu_count ? 16 : 32);
        pa::MergeArgs m{h->ws_o, h->ws_lse, h->mdesc, h->mcount, out, lse, c.num_q_heads, G, h->merge_rows,
                        h->desc_cap, nullptr, 0, 1, 0, 0};
        hipError_t e = pa::launch_merge(m, c.head_dim, mgrid, batch, st);
        if (e != hipSuccess) return fail(h, PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
    }
    return PA_OK;
}

int paged_attn_debug_gather(pa_handle_t* h, const void* k_cache, const pa_cache_layout_t* layout,
                            const int32_t* block_table, int32_t num_seqs, int32_t block_table_stride,
                            const int32_t* seq_lens, const int32_t* q_lens, int32_t window, int64_t* slots_out,
                            void* rows_out, int64_t capacity, void* stream) {
    if (!h) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "handle is NULL");
    const pa_config_t& c = h->cfg;
    int rc = validate_cache(h, layout, k_cache, k_cache);
    if (rc != PA_OK) return rc;
    if (!block_table || !seq_lens || !q_lens || !slots_out || !rows_out)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (!aligned16(rows_out)) return fail(h, PA_ERR_INVALID_ARGUMENT, "rows_out must be 16-byte aligned");
    if (num_seqs < 1 || num_seqs > c.max_num_seqs || block_table_stride < 1 || capacity < 0)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "size argument out of range");
    DeviceGuard guard(c.device);
    if (!guard.ok) return fail(h, PA_ERR_HIP, "hipSetDevice(%d) failed", c.device);
    pa::GatherArgs a{};
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.q_lens = q_lens;
    a.slots_out = slots_out;
    a.rows_out = static_cast<uint8_t*>(rows_out);
    a.capacity = capacity;
    a.page_stride = layout->page_stride;
    a.head_stride = layout->head_stride;
    a.token_stride = layout->token_stride;
    a.num_seqs = num_seqs;
    a.bt_stride = block_table_stride;
    a.num_kv_heads = c.num_kv_heads;
    a.head_dim = c.head_dim;
    a.elem_bytes = elem_bytes(c.kv_dtype);
    a.page_size = c.page_size;
    a.window = window;
    hipError_t e = pa::launch_debug_gather(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(h, PA_ERR_HIP, "gather launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

int paged_attn_append(pa_handle_t* h, const void* k_new, const void* v_new, int64_t num_tokens, void* k_cache,
                      void* v_cache, const pa_cache_layout_t* layout, const int32_t* block_table, int32_t num_seqs,
                      int32_t block_table_stride, const int32_t* seq_lens, const int32_t* q_lens,
                      const float* kv_scale, void* stream) {
    if (!h) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "handle is NULL");
    const pa_config_t& c = h->cfg;
    int rc = validate_cache(h, layout, k_cache, v_cache);
    if (rc != PA_OK) return rc;
    if (!k_new || !v_new || !block_table || !seq_lens || !q_lens)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "k_new, v_new, block_table, seq_lens and q_lens must be non-NULL");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(h, PA_ERR_INVALID_ARGUMENT, "k_new and v_new must be 16-byte aligned");
    if (num_tokens < 1 || num_tokens > c.max_num_tokens)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "num_tokens %lld outside 1..%lld", (long long)num_tokens,
                    (long long)c.max_num_tokens);
    if (num_seqs < 1 || num_seqs > c.max_num_seqs)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "num_seqs %d outside 1..%d", num_seqs, c.max_num_seqs);
    if (block_table_stride < 1) return fail(h, PA_ERR_INVALID_ARGUMENT, "block_table_stride must be >= 1");
    if ((c.kv_dtype == PA_DTYPE_FP8_E4M3) != (kv_scale != nullptr))
        return fail(h, PA_ERR_INVALID_ARGUMENT, "kv_scale is required for an fp8 cache and must be NULL otherwise");
    if (c.page_size != pa::kAppendPage) return fail(h, PA_ERR_UNSUPPORTED, "page_size must be 16");
    DeviceGuard guard(c.device);
    if (!guard.ok) return fail(h, PA_ERR_HIP, "hipSetDevice(%d) failed", c.device);
    pa::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.q_lens = q_lens;
    a.kv_scale = kv_scale;
    a.num_pages = layout->num_pages;
    a.page_stride = layout->page_stride;
    a.head_stride = layout->head_stride;
    a.token_stride = layout->token_stride;
    a.num_tokens = num_tokens;
    a.num_seqs = num_seqs;
    a.bt_stride = block_table_stride;
    a.num_kv_heads = c.num_kv_heads;
    a.head_dim = c.head_dim;
    hipError_t e = pa::launch_append(a, c.kv_dtype, c.q_dtype, c.max_q_len, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(h, PA_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

}  // extern "C"
