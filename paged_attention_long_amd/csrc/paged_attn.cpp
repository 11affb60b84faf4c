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

#include "paged_attn.h"
#include "pa_host.h"
#include "pa_kernels.h"

namespace pa {

namespace {

thread_local char g_err[512];

int elem_bytes(int dt) { return (dt == PA_DTYPE_FP8_E4M3 || dt == PA_DTYPE_INT8) ? 1 : 2; }
bool scaled_cache(int dt) { return dt == PA_DTYPE_FP8_E4M3 || dt == PA_DTYPE_INT8; }

int pow2ceil(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMinPagesPerSplit = 4;
constexpr int kValuRowsMax = 8;   // rows per KV head handled by the VALU kernel under PA_PATH_AUTO
constexpr int kValuMaxKeys = 16384;   // and visible keys (longer contexts go to the tile kernel)
// A single sequence past this many tokens of block table goes to the tile
// kernel even at a few rows per KV head: its one-sequence plan is a few
// scalar instructions, and from about 1.5k keys on its forward is the shorter
// one (4,097-token decode at 32/8 heads: 15.3 against 16.8 us; 1,025 tokens:
// 14.0 against 13.7).  Batches keep kValuMaxKeys: their device plan costs the
// tile kernel more (two 2,049-token sequences: 18.0 against 16.8 us).
constexpr int kValuMaxKeysOne = 1536;

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// c / d == umulhi(c, magic) >> shift for every c < 2^24 and 2 <= d <= 4096:
// with 2^shift < d <= 2^(shift+1) and magic = ceil(2^(32+shift) / d) < 2^32,
// c * magic / 2^(32+shift) exceeds c / d by less than 2^24 / 2^(32+shift),
// which is below 1/d, so the floor is unchanged.
void chunk_magic(int d, uint32_t* magic, int* shift) {
    if (d <= 1) {
        *magic = 0;
        *shift = 0;
        return;
    }
    int s = 0;
    while ((1 << (s + 1)) < d) ++s;
    *shift = s;
    *magic = (uint32_t)((((uint64_t)1 << (32 + s)) + (uint64_t)d - 1) / (uint64_t)d);
}

}  // namespace

int fail(pa_handle* h, int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(h ? h->err : g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

const char* thread_error() { return g_err; }

int validate_config(const pa_config_t* c, char* why, size_t why_len) {
    auto bad = [&](int code, const char* msg) {
        snprintf(why, why_len, "%s", msg);
        return code;
    };
    if (!c) return bad(PA_ERR_INVALID_ARGUMENT, "config is NULL");
    if (c->num_q_heads < 1 || c->num_kv_heads < 1) return bad(PA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
    if (c->num_q_heads % c->num_kv_heads) return bad(PA_ERR_INVALID_ARGUMENT, "num_q_heads % num_kv_heads != 0");
    if (c->num_q_heads / c->num_kv_heads > 16) return bad(PA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
        return bad(PA_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
    if (c->page_size < 16 || c->page_size > 65536 || c->page_size % 16)
        return bad(PA_ERR_UNSUPPORTED, "page_size must be a multiple of 16 in 16..65536");
    if (c->q_dtype != PA_DTYPE_F16 && c->q_dtype != PA_DTYPE_BF16)
        return bad(PA_ERR_UNSUPPORTED, "q_dtype must be F16 or BF16");
    if (c->kv_dtype != PA_DTYPE_F16 && c->kv_dtype != PA_DTYPE_BF16 && c->kv_dtype != PA_DTYPE_FP8_E4M3 &&
        c->kv_dtype != PA_DTYPE_INT8)
        return bad(PA_ERR_UNSUPPORTED, "kv_dtype must be F16, BF16, FP8_E4M3 or INT8");
    if (!scaled_cache(c->kv_dtype) && c->kv_dtype != c->q_dtype)
        return bad(PA_ERR_UNSUPPORTED, "a 16-bit cache must have the query's dtype");
    if (c->max_num_seqs < 1 || c->max_num_seqs > 1024) return bad(PA_ERR_INVALID_ARGUMENT, "max_num_seqs must be 1..1024");
    if (c->max_q_len < 1) return bad(PA_ERR_INVALID_ARGUMENT, "max_q_len must be >= 1");
    if (c->min_q_len < 1 || c->min_q_len > c->max_q_len)
        return bad(PA_ERR_INVALID_ARGUMENT, "min_q_len must be 1..max_q_len");
    if (c->head_dim == 64 && (int64_t)c->max_q_len * (c->num_q_heads / c->num_kv_heads) > 64)
        return bad(PA_ERR_UNSUPPORTED, "head_dim 64 supports at most 64 rows per KV head (max_q_len * group)");
    if (c->max_num_tokens < 1 || c->max_num_tokens > (int64_t)1 << 24)
        return bad(PA_ERR_INVALID_ARGUMENT, "max_num_tokens must be 1..2^24");
    if ((int64_t)c->max_q_len * (c->num_q_heads / c->num_kv_heads) > (1 << 20))
        return bad(PA_ERR_UNSUPPORTED, "max_q_len * group too large");
    if (c->flags & ~PA_DEBUG_CHECKS) return bad(PA_ERR_INVALID_ARGUMENT, "flags must be 0 or PA_DEBUG_CHECKS");
    if (c->device < 0) return bad(PA_ERR_INVALID_ARGUMENT, "device must be >= 0");
    return PA_OK;
}

void size_handle(pa_handle* h, const pa_config_t* cfg, int cu_count) {
    h->cfg = *cfg;
    std::memset(&h->tune, 0, sizeof h->tune);
    h->cu_count = cu_count > 0 ? cu_count : 256;
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
    // eight waves
    h->mfma_wr = rows_max > 64 ? 8 : 1;
    if (D == 256) h->mfma_wr = 4;   // the head_dim 256 tile kernel: 128-row items
    // The tile kernel launches exactly one round of resident workgroups; its
    // in-kernel plan sizes the splits for that many items.
    h->mfma_grid = D == 128   ? h->cu_count * mfma_blocks_per_cu(cfg->kv_dtype, cfg->q_dtype, h->mfma_wr,
                                                                  cfg->max_num_seqs)
                   : D == 256 ? h->cu_count * tile256_blocks_per_cu(cfg->kv_dtype, cfg->q_dtype, cfg->max_num_seqs)
                              : h->cu_count;
    const int bm = 32 * h->mfma_wr;
    const int64_t qblocks = ((int64_t)cfg->max_num_tokens * G + bm - 1) / bm + cfg->max_num_seqs;
    h->max_items_mfma = (int)std::min<int64_t>((int64_t)1 << 30, grid_cap + qblocks * cfg->num_kv_heads);
    h->merge_rows = (int)std::max<int64_t>(h->r_max_valu, D != 64 ? bm : 0);
    // Fixed slots for the VALU kernel's static splits (at most 8 workgroups
    // per CU, so at most that many (sequence, KV head) groups).
    h->sdesc_upg = (h->r_max_valu + merge_rows_per_unit(D) - 1) / merge_rows_per_unit(D);
    h->sdesc_groups = std::min<int64_t>((int64_t)cfg->max_num_seqs * cfg->num_kv_heads, (int64_t)8 * h->cu_count);
}

WsLayout layout_workspace(const pa_handle* h, bool valu, bool mfma) {
    const int D = h->cfg.head_dim;
    mfma = mfma && D != 64;
    const int bm = 32 * h->mfma_wr;
    WsLayout L{};
    // The two kernels' partials live side by side until the merge launch: VALU
    // slots first, then the tile kernel's, starting at a whole tile item.
    const size_t valu_slots = valu ? ((size_t)h->max_items_valu * h->r_max_valu + bm - 1) / bm * bm : 0;
    L.mfma_item_off = (int)(valu_slots / bm);
    const size_t slots = valu_slots + (mfma ? (size_t)h->max_items_mfma * bm : (size_t)0);
    const size_t o_bytes = slots * D * sizeof(float);
    const size_t l_bytes = slots * sizeof(float);
    // a merge group has at least two items
    L.desc_cap = (int)std::max<size_t>(
        1, ((valu ? (size_t)h->max_items_valu : 0) + (mfma ? (size_t)h->max_items_mfma : 0)) / 2);
    const size_t d_bytes = (size_t)L.desc_cap * sizeof(MergeDesc);
    const size_t c_bytes = kMergeCounterInts * sizeof(int);
    const size_t s_bytes = valu ? (size_t)h->sdesc_groups * h->sdesc_upg * sizeof(MergeDesc) : 0;
    const size_t a_bytes = valu ? (size_t)h->sdesc_groups * sizeof(int) : 0;
    const size_t e_bytes = sizeof(int);
    L.o_off = 0;
    L.l_off = L.o_off + up256(o_bytes);
    L.d_off = L.l_off + up256(l_bytes);
    L.c_off = L.d_off + up256(d_bytes);
    L.s_off = L.c_off + up256(c_bytes);
    L.a_off = L.s_off + up256(s_bytes);
    L.e_off = L.a_off + up256(a_bytes);
    L.total = L.e_off + up256(e_bytes);
    L.zero_begin = L.c_off;
    L.zero_end = L.total;
    return L;
}

void bind_workspace(pa_handle* h, void* base, const WsLayout& L) {
    char* p = static_cast<char*>(base);
    h->ws_o = reinterpret_cast<float*>(p + L.o_off);
    h->ws_lse = reinterpret_cast<float*>(p + L.l_off);
    h->mdesc = reinterpret_cast<MergeDesc*>(p + L.d_off);
    h->mcount = reinterpret_cast<int*>(p + L.c_off);
    h->sdesc = reinterpret_cast<MergeDesc*>(p + L.s_off);
    h->arrive = reinterpret_cast<int*>(p + L.a_off);
    h->err_word = reinterpret_cast<int*>(p + L.e_off);
    h->mfma_item_off = L.mfma_item_off;
    h->desc_cap = L.desc_cap;
}

}  // namespace pa

using namespace pa;

namespace pa {

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
    if (c.kv_dtype == PA_DTYPE_INT8 &&
        (L->page_stride % c.head_dim || L->head_stride % c.head_dim || L->token_stride % c.head_dim))
        return fail(h, PA_ERR_INVALID_ARGUMENT, "an int8 cache needs every stride to be a multiple of head_dim");
    const int cpp = c.page_size / 16;
    if (cpp > 1) {
        // pages of more than 16 tokens are addressed as 16-token virtual pages
        if (L->page_stride % (16 * L->token_stride))
            return fail(h, PA_ERR_UNSUPPORTED,
                        "with pages of %d tokens the page stride must be a multiple of 16 token rows", c.page_size);
        if (L->num_pages * (L->page_stride / (16 * L->token_stride)) >= ((int64_t)1 << 31))
            return fail(h, PA_ERR_UNSUPPORTED, "num_pages x %d-token pages exceeds 2^31 virtual pages", c.page_size);
    }
    return PA_OK;
}

int check_forward(pa_handle* h, const ForwardCall& f) {
    const pa_config_t& c = h->cfg;
    if (!f.q || !f.out || !f.block_table || !f.seq_lens || !f.q_lens)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "q, out, block_table, seq_lens and q_lens must be non-NULL");
    if (!aligned16(f.q) || !aligned16(f.out)) return fail(h, PA_ERR_INVALID_ARGUMENT, "q and out must be 16-byte aligned");
    if (f.lse && (reinterpret_cast<uintptr_t>(f.lse) & 3u)) return fail(h, PA_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    if (f.num_tokens < 1 || f.num_tokens > c.max_num_tokens)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "num_tokens %lld outside 1..%lld", (long long)f.num_tokens,
                    (long long)c.max_num_tokens);
    if (f.num_seqs < 1 || f.num_seqs > c.max_num_seqs)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "num_seqs %d outside 1..%d", f.num_seqs, c.max_num_seqs);
    if (f.bt_stride < 1) return fail(h, PA_ERR_INVALID_ARGUMENT, "block_table_stride must be >= 1");
    if ((int64_t)f.bt_stride * (c.page_size / 16) >= ((int64_t)1 << 24))
        return fail(h, PA_ERR_UNSUPPORTED, "block_table_stride x page_size must be below 2^28 tokens");
    if (!std::isfinite(f.scale) || !(f.scale > 0.f)) return fail(h, PA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (scaled_cache(c.kv_dtype) != (f.kv_scale != nullptr))
        return fail(h, PA_ERR_INVALID_ARGUMENT,
                    "kv_scale is required for an fp8 or int8 cache and must be NULL otherwise");
    if (f.kv_scale && (reinterpret_cast<uintptr_t>(f.kv_scale) & 3u))
        return fail(h, PA_ERR_INVALID_ARGUMENT, "kv_scale must be 4-byte aligned");
    return validate_cache(h, f.layout, f.k_cache, f.v_cache);
}

// Each sequence goes to one kernel, decided on the device from its lengths:
// a few rows per KV head over a short context stream K/V through the vector
// ALUs (lowest latency); verification widths, prefill chunks and long
// contexts go to the MFMA tile kernel, whose per-key VALU work is several
// times smaller.  The host launches a kernel only if some sequence can
// belong to it.
LaunchPlan plan_launches(const pa_handle* h, const ForwardCall& f) {
    const pa_config_t& c = h->cfg;
    const int G = c.num_q_heads / c.num_kv_heads;
    const int rows_min = c.min_q_len * G, rows_max = c.max_q_len * G;
    const int64_t cap_tokens = (int64_t)f.bt_stride * c.page_size;
    LaunchPlan lp{};
    if (c.head_dim == 64 || h->tune.path == PA_PATH_VALU) {
        lp.run_valu = true;
        lp.run_mfma = false;
    } else if (h->tune.path == PA_PATH_MFMA) {
        lp.run_valu = false;
        lp.run_mfma = true;
    } else if (c.head_dim == 256) {
        // The VALU kernel takes every sequence when no row count passes 64;
        // otherwise the sequences of up to 8 rows per KV head (any length),
        // and the tile kernel the rest.
        lp.run_mfma = rows_max > 64;
        lp.run_valu = !lp.run_mfma || rows_min <= kValuRowsMax;
    } else {
        lp.run_valu = rows_min <= kValuRowsMax;
        lp.run_mfma = rows_max > kValuRowsMax || cap_tokens > (f.num_seqs == 1 ? kValuMaxKeysOne : kValuMaxKeys);
        // A tile launch with 32-row items takes the few-row sequences as well:
        // a VALU launch before it on the same stream would add its whole
        // latency, and per key the tile kernel costs less.  (With prefill-sized
        // items a few-row sequence would fill a small part of each tile.)
        if (lp.run_mfma && h->mfma_wr == 1) lp.run_valu = false;
    }
    return lp;
}

int enqueue_forward(pa_handle* h, const ForwardCall& f, const LaunchPlan& lp) {
    const pa_config_t& c = h->cfg;
    const int G = c.num_q_heads / c.num_kv_heads;
    DecodeArgs a{};
    a.q = f.q;
    a.k_cache = f.k_cache;
    a.v_cache = f.v_cache;
    a.block_table = f.block_table;
    a.seq_lens = f.seq_lens;
    a.q_lens = f.q_lens;
    a.kv_scale = f.kv_scale;
    a.out = f.out;
    a.lse = f.lse;
    a.ws_o = h->ws_o;
    a.ws_lse = h->ws_lse;
    a.mdesc = h->mdesc;
    a.mcount = h->mcount;
    a.sdesc = nullptr;
    a.sdesc_upg = h->sdesc_upg;
    a.arrive = nullptr;
    a.cpp = c.page_size / 16;
    chunk_magic(a.cpp, &a.cpp_magic, &a.cpp_shift);
    a.page_stride = a.cpp > 1 ? 16 * f.layout->token_stride : f.layout->page_stride;
    a.vr = a.cpp > 1 ? (int)(f.layout->page_stride / (16 * f.layout->token_stride)) : 1;
    a.head_stride = f.layout->head_stride;
    a.token_stride = f.layout->token_stride;
    a.num_seqs = f.num_seqs;
    a.bt_stride = f.bt_stride;
    a.bt_chunks = f.bt_stride * a.cpp;
    if (c.kv_dtype == PA_DTYPE_INT8) {
        // row scales: laid out like the cache with rows of one element
        a.row_scale = f.kv_scale;
        a.rs_v = f.layout->num_pages * f.layout->page_stride / c.head_dim;
        a.rs_page = a.page_stride / c.head_dim;
        a.rs_head = f.layout->head_stride / c.head_dim;
        a.rs_tok = f.layout->token_stride / c.head_dim;
    }
    a.num_q_heads = c.num_q_heads;
    a.num_kv_heads = c.num_kv_heads;
    a.group = G;
    a.window = f.window;
    a.scale = f.scale;
    a.checks = (c.flags & PA_DEBUG_CHECKS) != 0;
    a.err_word = h->err_word;
    a.num_pages = f.layout->num_pages;
    a.max_q_len = c.max_q_len;
    a.num_tokens = f.num_tokens;
    const int grid = h->tune.grid > 0 ? h->tune.grid : h->grid_default;
    a.target_items = grid;
    hipStream_t st = f.stream;
    const int num_seqs = f.num_seqs;
    const int window = f.window;
    const int32_t block_table_stride = f.bt_stride;
    const bool run_valu = lp.run_valu, run_mfma = lp.run_mfma;
    if (c.head_dim == 64 || h->tune.path == PA_PATH_VALU || (c.head_dim == 256 && !run_mfma)) {
        a.cls_rows = 1 << 30; a.cls_len = 1 << 30;
    } else if (h->tune.path == PA_PATH_MFMA || (run_mfma && h->mfma_wr == 1)) {
        a.cls_rows = 0; a.cls_len = 0;
    } else if (c.head_dim == 256) {
        a.cls_rows = kValuRowsMax; a.cls_len = 1 << 30;
    } else {
        a.cls_rows = kValuRowsMax; a.cls_len = kValuMaxKeys;
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
            // 16-token chunks a VALU-class sequence can reach (static splits
            // count from chunk 0): without a window its visible keys start at 0.
            const int64_t cap_pages =
                window > 0 ? (int64_t)a.bt_chunks : std::min<int64_t>(a.bt_chunks, (int64_t)a.cls_len / 16 + 1);
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
        hipError_t e = c.head_dim == 256 ? pa::launch_tile256(a, c.kv_dtype, c.q_dtype, tgrid, st)
                                         : pa::launch_mfma_attn(a, c.head_dim, c.kv_dtype, c.q_dtype, h->mfma_wr, tgrid, st);
        if (e != hipSuccess) return fail(h, PA_ERR_HIP, "tile launch failed: %s", hipGetErrorString(e));
    }
    if (static_merge && need_merge_valu) {
        // one workgroup per fixed slot; empty slots leave at once
        const int64_t su = (int64_t)num_seqs * c.num_kv_heads * h->sdesc_upg;
        pa::MergeArgs m{h->ws_o,   h->ws_lse,   h->mdesc,     h->mcount,    f.out,       f.lse,
                        c.num_q_heads, G,       h->merge_rows, h->desc_cap, h->sdesc, (int)su,
                        h->sdesc_upg,  static_splits, h->r_max_valu};
        hipError_t e = pa::launch_merge(m, c.head_dim, (int)su, st);
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
            groups += (int64_t)c.num_kv_heads * ((f.num_tokens * G + bm - 1) / bm + num_seqs);
        }
        // Many units (prefill): units of a few rows, four workgroups per CU
        // (every workgroup also takes one turn on the shared arrival counter,
        // so a wider grid costs more than it gains).  Few units (decode,
        // verification, mixed batches): one row per unit, each row's splits
        // spread over a workgroup, up to two workgroups per CU.
        const int64_t units = groups * upg;
        const bool many = units > 4 * (int64_t)h->cu_count;
        pa::MergeArgs m{h->ws_o, h->ws_lse, h->mdesc, h->mcount, f.out, f.lse, c.num_q_heads, G, h->merge_rows,
                        h->desc_cap, nullptr, 0, 1, 0, 0};
        const int64_t row_units = groups * h->merge_rows;
        hipError_t e = many ? pa::launch_merge(m, c.head_dim,
                                               (int)std::min<int64_t>(4 * (int64_t)h->cu_count, units), st)
                            : pa::launch_merge_rows(m, c.head_dim,
                                                    (int)std::max<int64_t>(1, std::min<int64_t>(2 * (int64_t)h->cu_count, row_units)), st);
        if (e != hipSuccess) return fail(h, PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
    }
    return PA_OK;
}

}  // namespace pa

extern "C" {

const char* paged_attn_version(void) { return "0.2.0"; }

namespace {

// Reads and clears the checked mode's device error word; a message on h.
int collect_device_checks(pa_handle* h, int32_t* bits_out) {
    int w = 0;
    DeviceGuard guard(h->cfg.device);
    if (!guard.ok || hipMemcpy(&w, h->err_word, sizeof w, hipMemcpyDeviceToHost) != hipSuccess ||
        (w != 0 && hipMemset(h->err_word, 0, sizeof w) != hipSuccess))
        return fail(h, PA_ERR_HIP, "reading the device error word failed");
    if (bits_out) *bits_out = w;
    if (w == 0) return PA_OK;
    return fail(h, PA_ERR_INVALID_ARGUMENT, "device checks (0x%x):%s%s%s%s", w,
                (w & PA_CHECK_LENGTHS) ? " q_len/seq_len outside their ranges;" : "",
                (w & PA_CHECK_TABLE) ? " seq_len past the block-table width;" : "",
                (w & PA_CHECK_PAGE) ? " block-table page id outside [0, num_pages);" : "",
                (w & PA_CHECK_TOKENS) ? " q_lens add up past num_tokens;" : "");
}

}  // namespace

const char* paged_attn_last_error(const pa_handle_t* h) {
    if (!h) return pa::thread_error();
    pa_handle* hm = const_cast<pa_handle*>(h);
    if (hm->cfg.flags & PA_DEBUG_CHECKS) (void)collect_device_checks(hm, nullptr);
    return h->err;
}

int paged_attn_debug_status(pa_handle_t* h, int32_t* bits_out) {
    if (!h) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (bits_out) *bits_out = 0;
    if (!(h->cfg.flags & PA_DEBUG_CHECKS)) return fail(h, PA_ERR_UNSUPPORTED, "the handle has no PA_DEBUG_CHECKS");
    return collect_device_checks(h, bits_out);
}

int paged_attn_create(const pa_config_t* cfg, pa_handle_t** out) {
    if (!out) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    char why[256];
    int rc = validate_config(cfg, why, sizeof why);
    if (rc != PA_OK) return fail(nullptr, rc, "%s", why);

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= cfg->device)
        return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "device %d not present (%d devices)", cfg->device, ndev);
    DeviceGuard guard(cfg->device);
    if (!guard.ok) return fail(nullptr, PA_ERR_HIP, "hipSetDevice(%d) failed", cfg->device);

    pa_handle* h = new (std::nothrow) pa_handle();
    if (!h) return fail(nullptr, PA_ERR_OUT_OF_MEMORY, "host allocation failed");
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, cfg->device) != hipSuccess) cu = 0;
    size_handle(h, cfg, cu);
    // The handle's workspace holds the partials of both kernels.
    const WsLayout L = layout_workspace(h, true, true);
    h->ws_bytes = L.total;
    if (hipMalloc(&h->ws, h->ws_bytes) != hipSuccess) {
        const size_t want = h->ws_bytes;
        delete h;
        (void)hipGetLastError();
        return fail(nullptr, PA_ERR_OUT_OF_MEMORY, "workspace of %zu bytes could not be allocated", want);
    }
    bind_workspace(h, h->ws, L);
    if (hipMemset(static_cast<char*>(h->ws) + L.zero_begin, 0, L.zero_end - L.zero_begin) != hipSuccess ||
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
    if (t->path == PA_PATH_MFMA && h->cfg.head_dim == 64)
        return fail(h, PA_ERR_UNSUPPORTED, "the MFMA path needs head_dim 128 or 256");
    if (t->path == PA_PATH_VALU && !h->valu_all_ok)
        return fail(h, PA_ERR_UNSUPPORTED, "the VALU path holds at most 64 rows per KV head");
    if (t->pages_per_split < 0 || t->kv_tiles_per_split < 0 || t->grid < 0 || t->grid > 8 * h->cu_count ||
        t->split_mode < 0 || t->split_mode > 2)
        return fail(h, PA_ERR_INVALID_ARGUMENT, "tuning values out of range (grid <= %d)", 8 * h->cu_count);
    h->tune = *t;
    return PA_OK;
}

int paged_attn_forward(pa_handle_t* h, const void* q, int64_t num_tokens, const void* k_cache, const void* v_cache,
                       const pa_cache_layout_t* layout, const int32_t* block_table, int32_t num_seqs,
                       int32_t block_table_stride, const int32_t* seq_lens, const int32_t* q_lens, int32_t window,
                       float scale, const float* kv_scale, float* out, float* lse, void* stream) {
    if (!h) return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "handle is NULL");
    const ForwardCall f{q,        num_tokens, k_cache,  v_cache, layout, block_table, num_seqs, block_table_stride,
                        seq_lens, q_lens,     window,   scale,   kv_scale, out,       lse,      static_cast<hipStream_t>(stream)};
    int rc = check_forward(h, f);
    if (rc != PA_OK) return rc;
    DeviceGuard guard(h->cfg.device);
    if (!guard.ok) return fail(h, PA_ERR_HIP, "hipSetDevice(%d) failed", h->cfg.device);
    return enqueue_forward(h, f, plan_launches(h, f));
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
                      float* kv_scale, void* stream) {
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
    if (scaled_cache(c.kv_dtype) != (kv_scale != nullptr))
        return fail(h, PA_ERR_INVALID_ARGUMENT,
                    "kv_scale is required for an fp8 or int8 cache and must be NULL otherwise");
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
    a.page_size = c.page_size;
    a.cpp = c.page_size / 16;
    chunk_magic(a.cpp, &a.cpp_magic, &a.cpp_shift);
    a.checks = (c.flags & PA_DEBUG_CHECKS) != 0;
    a.err_word = h->err_word;
    if (c.kv_dtype == PA_DTYPE_INT8) {
        a.kv_scale = nullptr;
        a.row_scale = kv_scale;
        a.rs_v = layout->num_pages * layout->page_stride / c.head_dim;
        a.rs_page = layout->page_stride / c.head_dim;
        a.rs_head = layout->head_stride / c.head_dim;
        a.rs_tok = layout->token_stride / c.head_dim;
    }
    hipError_t e = pa::launch_append(a, c.kv_dtype, c.q_dtype, c.max_q_len, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(h, PA_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

}  // extern "C"
