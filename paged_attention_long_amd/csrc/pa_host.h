// Host-side internals of the C ABI shared by the handle entry points
// (paged_attn.cpp) and the entry point that runs on a fixed device array
// (pa_static.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

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
    int* mcount = nullptr;            // merge counters ([0] groups published; kMergeCounterInts ints)
    int* err_word = nullptr;          // device error word of the checked mode (PA_DEBUG_CHECKS)
    void* ws = nullptr;
    size_t ws_bytes = 0;
    char err[512] = {0};
};

namespace pa {

// Byte layout of one workspace: split partials, their LSEs, merge
// descriptors, then the words that must be zero when a forward starts
// (merge counters, fixed merge slots, arrival counters, the error word).
struct WsLayout {
    size_t o_off, l_off, d_off, c_off, s_off, a_off, e_off;
    size_t zero_begin, zero_end;   // the must-be-zero range
    size_t total;
    int mfma_item_off;
    int desc_cap;
};

// Validates cfg (no GPU calls); PA_OK or an error code with the reason in why.
int validate_config(const pa_config_t* c, char* why, size_t why_len);

// Fills the handle's sizing fields from cfg and the device (CU count, tile
// kernel occupancy).  No allocation.
void size_handle(pa_handle* h, const pa_config_t* cfg, int cu_count);

// Workspace layout for the kernels a forward may launch.
WsLayout layout_workspace(const pa_handle* h, bool valu, bool mfma);

// Points the handle's workspace fields into `base` per `L`.
void bind_workspace(pa_handle* h, void* base, const WsLayout& L);

// Arguments of one forward as the ABI receives them.
struct ForwardCall {
    const void* q;
    int64_t num_tokens;
    const void* k_cache;
    const void* v_cache;
    const pa_cache_layout_t* layout;
    const int32_t* block_table;
    int32_t num_seqs, bt_stride;
    const int32_t* seq_lens;
    const int32_t* q_lens;
    int32_t window;
    float scale;
    const float* kv_scale;
    float* out;
    float* lse;
    hipStream_t stream;
};

// Checks the host arguments of a forward against the handle's configuration.
int check_forward(pa_handle* h, const ForwardCall& f);

// Which kernels a forward launches (decided on the host from the
// configuration and the call's host arguments).
struct LaunchPlan {
    bool run_valu, run_mfma;
};
LaunchPlan plan_launches(const pa_handle* h, const ForwardCall& f);

// Enqueues the forward on the workspace the handle points to.
int enqueue_forward(pa_handle* h, const ForwardCall& f, const LaunchPlan& lp);

// Records an error message (on h, or the thread's handle-less message).
int fail(pa_handle* h, int code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));

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

// Zero-fills n 32-bit words at p on `stream` (a kernel, so that it can be
// captured into a graph).
hipError_t launch_zero_words(int* p, size_t n, hipStream_t stream);

}  // namespace pa
