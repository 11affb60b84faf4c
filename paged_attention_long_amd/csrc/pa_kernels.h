// Kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kMaxSplits = 64;        // splits per (sequence, KV head) the merge reads in one pass
constexpr int kPidChunkPages = 1024;  // page ids a workgroup stages in LDS at a time
constexpr int kMergeThreads = 256;    // threads of a merge workgroup
constexpr int kMergeArrive = 32;      // first-level arrival counters of a merge launch
constexpr int kMergeArriveStride = 32;   // ints between counters (one 128-byte cache line each)
// The merge counters: [0] groups published, [1] second-level arrivals, then
// kMergeArrive first-level arrival counters kMergeArriveStride ints apart.
constexpr int kMergeCounterInts = kMergeArriveStride * (1 + kMergeArrive);
// Rows of one merge unit: a merge thread owns a float4 column of one row.
constexpr int merge_rpu(int head_dim) { return kMergeThreads / (head_dim / 4); }

// One group of split partials to merge: rows [0, rows) of items
// first_item .. first_item + n_splits - 1 (row stride rstride in the partial
// arrays) become output rows row0 .. row0 + rows - 1 of KV head g.
struct MergeDesc {
    int first_item;
    int n_splits;
    int rows;
    int rstride;
    int q_off;
    int g;
    int row0;
    float out_scale;   // fp8 V scale, else 1
};

// Arguments of the split-KV kernels (VALU decode/verify and MFMA tile).
struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* q_lens;
    const float* kv_scale;     // fp8: [2][Hkv]; int8: the row scales (see row_scale); else null
    // int8 caches: one fp32 scale per cached row, laid out like the cache
    // with rows of one element.  The scale of (virtual page p, KV head g,
    // slot s) is row_scale[p * rs_page + g * rs_head + s * rs_tok], plus
    // rs_v for V.
    const float* row_scale;
    int64_t rs_v, rs_page, rs_head, rs_tok;
    float* out;
    float* lse;                // may be null
    float* ws_o;               // split partials [max_items][r_max][D]
    float* ws_lse;             // [max_items][r_max] (log2 domain)
    MergeDesc* mdesc;          // merge groups published by this forward
    int* mcount;               // merge counters: [0] groups published, then the merge's arrival counters
    // Fixed merge slots (static splits, VALU kernel only): when set, the group
    // of (sequence b, KV head g) writes its descriptor to slots
    // (b * Hkv + g) * sdesc_upg + u for each merge unit u its rows cover,
    // instead of appending to mdesc.
    MergeDesc* sdesc;
    int sdesc_upg;
    // Arrival counters (static splits, VALU kernel only): when set, the
    // workgroups of group (b, g) count their arrivals in arrive[b * Hkv + g]
    // and the last one merges the group's partials itself (no merge launch).
    int* arrive;
    // Pages of P = 16 * cpp tokens are addressed as cpp virtual pages of 16
    // tokens: 16-token chunk c of a sequence lives in virtual page
    // block_table[c / cpp] * vr + c % cpp, whose rows start page_stride
    // elements apart (16 * token_stride when cpp > 1; see chunk_page()).
    int64_t page_stride, head_stride, token_stride;   // elements
    int num_seqs, bt_stride;
    int cpp;                   // 16-token chunks per page (1: 16-token pages)
    uint32_t cpp_magic;        // c / cpp == umulhi(c, cpp_magic) >> cpp_shift for c < 2^24 (cpp > 1)
    int cpp_shift;
    int vr;                    // virtual pages per physical page (cpp > 1)
    int bt_chunks;             // 16-token chunks the block-table row covers (bt_stride * cpp)
    int num_q_heads, num_kv_heads, group;
    int window;
    float scale;
    // Checked mode (PA_DEBUG_CHECKS): lengths and page ids are validated
    // before the accesses they steer; a bad value is replaced by a safe one
    // (the sequence skipped, page 0 read) and its kind or-ed into *err_word.
    int checks;
    int* err_word;
    int64_t num_pages;         // physical pages of the pool
    int max_q_len;
    int64_t num_tokens;
    int cls_side;              // 0: VALU launch (short, few-row sequences), 1: tile launch (the rest)
    int cls_rows, cls_len;     // VALU class: rows per KV head <= cls_rows and visible keys <= cls_len
    int target_items, min_pps, forced_pps, max_items, r_max;   // forced_pps: pages (VALU) or tiles (MFMA) per split
    int static_pps;            // VALU kernel: > 0 selects static splits of this many pages
    int static_splits;         // splits per (sequence, KV head) in static mode
    int item_off;              // tile kernel: its partial items start at this item
};

// Merge every group the attention kernels of this forward published, then
// reset the group count for the next forward.
struct MergeArgs {
    const float* ws_o;
    const float* ws_lse;
    const MergeDesc* mdesc;
    int* mcount;
    float* out;
    float* lse;
    int num_q_heads, group, max_rows;
    int desc_cap;              // descriptors the workspace holds
    // Fixed slots: > 0 selects them; workgroup u merges the unit whose
    // descriptor is in sdesc[u] (units per group: sdesc_upg), if one was
    // written this forward, and clears it.  mdesc and mcount are then unused.
    // The groups' items are numbered as in the static split mode (group
    // q = b * Hkv + g owns items q * static_splits ..., static_rstride rows
    // each), so the partials are requested together with the descriptor.
    MergeDesc* sdesc;
    int static_units, sdesc_upg, static_splits, static_rstride;
};
// Fixed slots (m.static_units > 0): one workgroup per slot.  Otherwise the
// published groups in units of merge_rows_per_unit rows, eight partial rows in
// flight per thread (registers low enough for several resident workgroups:
// launches with many groups, i.e. prefill).
hipError_t launch_merge(const MergeArgs& m, int head_dim, int grid, hipStream_t stream);
int merge_rows_per_unit(int head_dim);
// The published groups merged one row per unit (m.max_rows units per group),
// each row's splits spread over the workgroup's threads.
hipError_t launch_merge_rows(const MergeArgs& m, int head_dim, int grid, hipStream_t stream);

hipError_t launch_decode_valu(const DecodeArgs& a, int head_dim, int kv_dtype, int q_dtype, int rw, int grid,
                              hipStream_t stream);

// wr: waves along query rows (8: 256-row blocks for prefill, every cache
// type; 1: 32-row blocks, four waves splitting the keys, for verification
// widths and few-row sequences).
hipError_t launch_mfma_attn(const DecodeArgs& a, int head_dim, int kv_dtype, int q_dtype, int wr, int grid,
                            hipStream_t stream);
int mfma_rows_per_item(int wr);
// Workgroups of the tile kernel resident per CU (registers and LDS bound it).
int mfma_blocks_per_cu(int kv_dtype, int q_dtype, int wr, int max_num_seqs);
// head_dim 256 tile kernel (rows per item, resident workgroups per CU, launch)
int tile256_rows_per_item();
int tile256_blocks_per_cu(int kv_dtype, int q_dtype, int max_num_seqs);
hipError_t launch_tile256(const DecodeArgs& a, int kv_dtype, int q_dtype, int grid, hipStream_t stream);

struct GatherArgs {
    const uint8_t* k_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* q_lens;
    int64_t* slots_out;
    uint8_t* rows_out;
    int64_t capacity;
    int64_t page_stride, head_stride, token_stride;   // elements
    int num_seqs, bt_stride, num_kv_heads, head_dim, elem_bytes, page_size, window;
};

hipError_t launch_debug_gather(const GatherArgs& a, hipStream_t stream);

// Arguments of the cache append (new K/V rows written into their pages).
struct AppendArgs {
    const void* k_new;         // [num_tokens][Hkv][D], 16-bit
    const void* v_new;
    void* k_cache;
    void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* q_lens;
    const float* kv_scale;     // [2][Hkv] (fp8 caches)
    float* row_scale;          // int8 caches: the row-scale pool (written), laid out like the cache with
    int64_t rs_v, rs_page, rs_head, rs_tok;   // rows of one element; rs_v: offset of the V scales
    int64_t num_pages, page_stride, head_stride, token_stride;   // elements
    int64_t num_tokens;
    int num_seqs, bt_stride, num_kv_heads, head_dim, page_size;
    int cpp;                   // page_size / 16
    uint32_t cpp_magic;        // c / cpp == umulhi(c, cpp_magic) >> cpp_shift for c < 2^24 (cpp > 1)
    int cpp_shift;
    int checks;                // PA_DEBUG_CHECKS: skipped rows are reported in *err_word
    int* err_word;
};

// max_rows: the largest q_len of the call (sizes the grid along the rows).
hipError_t launch_append(const AppendArgs& a, int kv_dtype, int in_dtype, int max_rows, hipStream_t stream);

}  // namespace pa
