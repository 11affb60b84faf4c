// Debug de-paging of K through the attention kernels' address computation
// (kv_offset in pa_common.h), for bit-exact checks of the block-table
// gather.  Not on the attention path.
#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {

namespace {

// One workgroup per sequence; its output rows start after every earlier
// sequence's visible tokens.
__global__ __launch_bounds__(256) void debug_gather_kernel(GatherArgs a) {
    const int b = blockIdx.x;
    int64_t base = 0;
    for (int s = 0; s < b; ++s) {
        const int ql = a.q_lens[s];
        if (ql > 0) base += a.seq_lens[s] - seq_visible_lo(a.seq_lens[s], ql, a.window);
    }
    const int sl = a.seq_lens[b];
    const int ql = a.q_lens[b];
    if (ql <= 0) return;
    const int lo = seq_visible_lo(sl, ql, a.window);
    const int row_bytes = a.head_dim * a.elem_bytes;
    const int chunks = row_bytes / 16;                // 16-B pieces per token row
    const int per_tok = a.num_kv_heads * chunks;
    const int64_t n = (int64_t)(sl - lo) * per_tok;
    const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
        const int t = (int)(e / per_tok);
        const int rem = (int)(e - (int64_t)t * per_tok);
        const int g = rem / chunks;
        const int c = rem - g * chunks;
        const int j = lo + t;
        const int64_t idx = base + t;
        if (idx >= a.capacity) continue;
        const int64_t page = bt[j / a.page_size];
        const int slot = j % a.page_size;
        const int64_t off = kv_offset(page, g, slot, a.page_stride, a.head_stride, a.token_stride) * a.elem_bytes;
        const u32x4_t v = load_b128_cached(a.k_cache + off + c * 16);
        *reinterpret_cast<u32x4_t*>(a.rows_out + (idx * a.num_kv_heads + g) * row_bytes + c * 16) = v;
        if (g == 0 && c == 0) a.slots_out[idx] = page * a.page_size + slot;
    }
}

}  // namespace

hipError_t launch_debug_gather(const GatherArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(debug_gather_kernel, dim3(a.num_seqs), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
