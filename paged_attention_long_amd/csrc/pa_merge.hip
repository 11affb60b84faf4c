// Merge of split-KV partial results: one launch per forward, ordered after
// the attention kernels on the caller's stream (see pa_merge.h).
//
// A unit is RPU consecutive rows of one published group; a thread owns one
// float4 column of one row and requests that column of every split's partial
// before the weights are known, so the partial reads overlap the LSE reads.
#include "pa_common.h"
#include "pa_merge.h"
#include "pa_kernels.h"

namespace pa {

namespace {

// BATCH: partial rows in flight per thread (see launch_merge).
template <int D, int BATCH>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs m) {
    constexpr int kMergeBatch = BATCH;
    constexpr int EPR = D / 4;                    // float4 columns per row
    constexpr int RPU = kMergeThreads / EPR;      // rows per unit
    constexpr int NW = kMergeThreads / kWave;
    __shared__ float w_sh[RPU][kMaxSplits];
    __shared__ float lse_sh[RPU];
    __shared__ int n_sh;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;

    static_assert(RPU == merge_rpu(D), "unit size shared with the publishers");
    const int upg = (m.max_rows + RPU - 1) / RPU;   // units per group
    // The attention kernels' writes are visible across the kernel boundary.
    // This workgroup's first group descriptor is read together with the count
    // (one round trip for both); it is only used if the group exists.
    const MergeDesc d_first = m.mdesc[min((int)(blockIdx.x / upg), m.desc_cap - 1)];
    if (tid == 0) n_sh = __hip_atomic_load(m.mcount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid == 0) {
        // Every workgroup has read the count (it is in LDS) before it arrives
        // here; the last to arrive clears the count for the next forward.
        // Past 64 workgroups, arrivals go through kMergeArrive first-level
        // counters on separate cache lines (workgroup w on counter
        // w % kMergeArrive), whose last arrivals count themselves in on the
        // second-level counter: atomics on one address are serialised, so a
        // thousand workgroups on a single counter would queue for
        // microseconds (prefill's merge: 15 us less).  Smaller grids count
        // on the second-level counter directly (one hop less).  Every counter
        // is cleared by the last arrival on it.
        const int nc = gridDim.x > 64 ? kMergeArrive : 1;
        const int j = (int)(blockIdx.x % nc);
        const int expect = (int)gridDim.x / nc + (j < (int)gridDim.x % nc ? 1 : 0);
        int* c1 = m.mcount + kMergeArriveStride * (1 + j);
        const int done = nc == 1 ? expect - 1 : __hip_atomic_fetch_add(c1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == expect - 1) {
            if (nc > 1) __hip_atomic_store(c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int top = nc == 1 ? (int)gridDim.x : nc;
            const int done2 = __hip_atomic_fetch_add(m.mcount + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (done2 == top - 1) {
                __hip_atomic_store(m.mcount + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(m.mcount, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    const int n_groups = n_sh;
    const int64_t n_units = (int64_t)n_groups * upg;
    const int rl = tid / EPR;                       // row of this thread within the unit
    const int col = (tid - rl * EPR) * 4;           // first of its four columns
    MergeTarget tgt{m.out, m.lse, m.num_q_heads, m.group, 1.0f};

    for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
        const int gidx = (int)(u / upg);
        const int r0 = (int)(u - (int64_t)gidx * upg) * RPU;
        const MergeDesc d = (u == blockIdx.x) ? d_first : m.mdesc[gidx];
        if (r0 >= d.rows) continue;                  // uniform
        const int nr = min(RPU, d.rows - r0);
        const int S = d.n_splits;
        const bool act = rl < nr;
        const int64_t sstride = (int64_t)d.rstride * D;
        // Branch-free requests: a thread past the unit's rows reads row r0 and
        // a split past the group's last reads the last one (both written by
        // this group in this forward, so finite); their weights are 0.
        const float* src = m.ws_o + ((int64_t)d.first_item * d.rstride + r0 + (act ? rl : 0)) * D + col;
        float4 o[kMergeBatch];
        auto issue = [&](int s0) {
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k)
                o[k] = *reinterpret_cast<const float4*>(src + (int64_t)min(s0 + k, S - 1) * sstride);
        };
        issue(0);
        // each wave weighs rows wid, wid + NW, ...: their LSE loads first, together
        constexpr int RPW = (RPU + NW - 1) / NW;
        float ls[RPW];
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int r = wid + k * NW;
            ls[k] = (r < nr && lane < S) ? m.ws_lse[((int64_t)d.first_item + lane) * d.rstride + r0 + r] : kNegInf;
        }
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int r = wid + k * NW;
            if (r < nr) {
                const float M = wave_max(ls[k]);
                const float w = (ls[k] == kNegInf) ? 0.f : fast_exp2(ls[k] - M);
                const float L = wave_sum(w);
                w_sh[r][lane] = (L > 0.f) ? w / L : 0.f;
                if (lane == 0) lse_sh[r] = (L > 0.f) ? M + fast_log2(L) : kNegInf;
            }
        }
        __syncthreads();
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        static_assert(kMaxSplits % kMergeBatch == 0, "weights of a whole batch are in w_sh");
        for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
            if (s0 > 0) issue(s0);
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const float w = w_sh[rl][s0 + k];   // 0 past the group's splits
                acc.x = fmaf(w, o[k].x, acc.x);
                acc.y = fmaf(w, o[k].y, acc.y);
                acc.z = fmaf(w, o[k].z, acc.z);
                acc.w = fmaf(w, o[k].w, acc.w);
            }
        }
        if (act) {
            const int64_t orow = out_row(tgt, d.q_off, d.g, d.row0 + r0 + rl);
            const float sc = d.out_scale;
            *reinterpret_cast<float4*>(m.out + orow * D + col) =
                make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
            if (m.lse != nullptr && col == 0) {
                const float l2 = lse_sh[rl];
                m.lse[orow] = (l2 == kNegInf) ? kNegInf : l2 * kLn2;
            }
        }
        __syncthreads();   // w_sh is rewritten by the next unit
    }
}

// Fixed slots (static splits): workgroup u merges the unit whose descriptor is
// in m.sdesc[u], if one was written this forward, and clears the slot once
// every thread has its copy, so a group merged directly in a later forward
// finds it empty.  No count and no arrival counter.  The partials and LSEs of
// every split the group can own are requested together with the descriptor
// (one round trip); splits outside the descriptor's range are skipped.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_slots_kernel(MergeArgs m) {
    constexpr int EPR = D / 4;                    // float4 columns per row
    constexpr int RPU = kMergeThreads / EPR;      // rows per unit
    constexpr int NW = kMergeThreads / kWave;
    constexpr int RPW = (RPU + NW - 1) / NW;
    constexpr int B = 32;                         // partial rows in flight per thread
    static_assert(RPU == merge_rpu(D), "unit size shared with the publishers");
    __shared__ float w_sh[RPU][kMaxSplits];
    __shared__ float lse_sh[RPU];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int q = (int)(blockIdx.x / m.sdesc_upg);            // group b * Hkv + g
    const int r0 = (int)(blockIdx.x % m.sdesc_upg) * RPU;
    const int rl = tid / EPR;
    const int col = (tid - rl * EPR) * 4;
    const int S_all = m.static_splits;
    const int rs = m.static_rstride;
    const int64_t item0 = (int64_t)q * S_all;
    const int64_t sstride = (int64_t)rs * D;
    // requests that do not wait for the descriptor (rows past the item's row
    // stride are not requested: they belong to the next item)
    const bool in_rows = r0 + rl < rs;
    const float* src = m.ws_o + (item0 * rs + r0 + rl) * D + col;
    float4 o[B];
#pragma unroll
    for (int k = 0; k < B; ++k)
        o[k] = (in_rows && k < S_all) ? *reinterpret_cast<const float4*>(src + (int64_t)k * sstride)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    float ls[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int r = wid + k * NW;
        ls[k] = (r0 + r < rs && lane < S_all) ? m.ws_lse[(item0 + lane) * rs + r0 + r] : kNegInf;
    }
    const MergeDesc d = m.sdesc[blockIdx.x];
    __syncthreads();
    if (d.n_splits == 0) return;
    if (tid == 0) m.sdesc[blockIdx.x].n_splits = 0;
    // the group's splits are items d.first_item .. d.first_item + n_splits - 1
    const int s0 = (int)(d.first_item - item0), S = d.n_splits;
    const int nr = min(RPU, d.rows - r0);
    const bool act = rl < nr;
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int r = wid + k * NW;
        if (r < nr) {
            const float l = (lane >= s0 && lane < s0 + S) ? ls[k] : kNegInf;
            const float M = wave_max(l);
            const float w = (l == kNegInf) ? 0.f : fast_exp2(l - M);
            const float L = wave_sum(w);
            w_sh[r][lane] = (L > 0.f) ? w / L : 0.f;
            if (lane == 0) lse_sh[r] = (L > 0.f) ? M + fast_log2(L) : kNegInf;
        }
    }
    __syncthreads();
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int b0 = 0; b0 < s0 + S; b0 += B) {
        if (b0 > 0) {
#pragma unroll
            for (int k = 0; k < B; ++k)
                o[k] = (in_rows && b0 + k < S_all) ? *reinterpret_cast<const float4*>(src + (int64_t)(b0 + k) * sstride)
                                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < B; ++k) {
            const int s = b0 + k;
            // outside the group's range the partial may be stale: skipped, not weighted by 0
            if (s >= s0 && s < s0 + S) {
                const float w = w_sh[rl][s];
                acc.x = fmaf(w, o[k].x, acc.x);
                acc.y = fmaf(w, o[k].y, acc.y);
                acc.z = fmaf(w, o[k].z, acc.z);
                acc.w = fmaf(w, o[k].w, acc.w);
            }
        }
    }
    if (act) {
        MergeTarget tgt{m.out, m.lse, m.num_q_heads, m.group, 1.0f};
        const int64_t orow = out_row(tgt, d.q_off, d.g, d.row0 + r0 + rl);
        const float sc = d.out_scale;
        *reinterpret_cast<float4*>(m.out + orow * D + col) = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
        if (m.lse != nullptr && col == 0) {
            const float l2 = lse_sh[rl];
            m.lse[orow] = (l2 == kNegInf) ? kNegInf : l2 * kLn2;
        }
    }
}


// One row per unit, its splits spread over the workgroup: SG groups of D/4
// threads each take every SG-th split of the row (kMaxSplits / SG partial
// rows in flight per thread), and the groups' sums are added in LDS in group
// order.  For launches with few rows and many splits (decode, verification,
// mixed batches) this spreads the partial reads over many more workgroups
// than units of several rows would.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_row_kernel(MergeArgs m) {
    constexpr int EPR = D / 4;                    // float4 columns per row
    constexpr int SG = kMergeThreads / EPR;       // split groups
    constexpr int B = kMaxSplits / SG;            // partial rows in flight per thread
    static_assert(SG * EPR == kMergeThreads && B * SG == kMaxSplits, "threads cover the row and the splits");
    __shared__ float w_sh[kMaxSplits];
    __shared__ float lse_sh;
    __shared__ float4 red[SG][EPR];
    __shared__ int n_sh;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int col = (tid % EPR) * 4;
    const int sg = tid / EPR;

    const int upg = m.max_rows;                   // units (rows) per group
    const MergeDesc d_first = m.mdesc[min((int)(blockIdx.x / upg), m.desc_cap - 1)];
    if (tid == 0) n_sh = __hip_atomic_load(m.mcount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid == 0) {
        // the arrival turn and the clearing of the count, as in merge_kernel
        const int nc = gridDim.x > 64 ? kMergeArrive : 1;
        const int j = (int)(blockIdx.x % nc);
        const int expect = (int)gridDim.x / nc + (j < (int)gridDim.x % nc ? 1 : 0);
        int* c1 = m.mcount + kMergeArriveStride * (1 + j);
        const int done = nc == 1 ? expect - 1 : __hip_atomic_fetch_add(c1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == expect - 1) {
            if (nc > 1) __hip_atomic_store(c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int top = nc == 1 ? (int)gridDim.x : nc;
            const int done2 = __hip_atomic_fetch_add(m.mcount + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (done2 == top - 1) {
                __hip_atomic_store(m.mcount + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(m.mcount, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    const int64_t n_units = (int64_t)n_sh * upg;
    MergeTarget tgt{m.out, m.lse, m.num_q_heads, m.group, 1.0f};
    for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
        const int gidx = (int)(u / upg);
        const int r = (int)(u - (int64_t)gidx * upg);
        const MergeDesc d = (u == blockIdx.x) ? d_first : m.mdesc[gidx];
        if (r >= d.rows) continue;                    // uniform
        const int S = d.n_splits;
        const int64_t sstride = (int64_t)d.rstride * D;
        // Branch-free requests: a split past the group's last re-reads the
        // last one (finite, written this forward) with weight 0.
        const float* src = m.ws_o + ((int64_t)d.first_item * d.rstride + r) * D + col;
        float4 o[B];
#pragma unroll
        for (int k = 0; k < B; ++k) o[k] = *reinterpret_cast<const float4*>(src + (int64_t)min(sg + k * SG, S - 1) * sstride);
        if (tid < kWave) {
            const float ls = lane < S ? m.ws_lse[((int64_t)d.first_item + lane) * d.rstride + r] : kNegInf;
            const float M = wave_max(ls);
            const float w = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
            const float L = wave_sum(w);
            w_sh[lane] = (L > 0.f) ? w / L : 0.f;
            if (lane == 0) lse_sh = (L > 0.f) ? M + fast_log2(L) : kNegInf;
        }
        __syncthreads();
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < B; ++k) {
            const float w = w_sh[sg + k * SG];   // 0 past the group's splits
            acc.x = fmaf(w, o[k].x, acc.x);
            acc.y = fmaf(w, o[k].y, acc.y);
            acc.z = fmaf(w, o[k].z, acc.z);
            acc.w = fmaf(w, o[k].w, acc.w);
        }
        red[sg][tid % EPR] = acc;
        __syncthreads();
        if (sg == 0) {
            float4 t = red[0][tid];
#pragma unroll
            for (int q = 1; q < SG; ++q) {
                const float4 v = red[q][tid];
                t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
            }
            const int64_t orow = out_row(tgt, d.q_off, d.g, d.row0 + r);
            const float sc = d.out_scale;
            *reinterpret_cast<float4*>(m.out + orow * D + col) = make_float4(t.x * sc, t.y * sc, t.z * sc, t.w * sc);
            if (m.lse != nullptr && tid == 0) {
                const float l2 = lse_sh;
                m.lse[orow] = (l2 == kNegInf) ? kNegInf : l2 * kLn2;
            }
        }
        __syncthreads();   // w_sh and red are rewritten by the next unit
    }
}

}  // namespace

int merge_rows_per_unit(int head_dim) { return merge_rpu(head_dim); }

hipError_t launch_merge_rows(const MergeArgs& m, int head_dim, int grid, hipStream_t stream) {
    if (head_dim == 64) hipLaunchKernelGGL((merge_row_kernel<64>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
    else if (head_dim == 256) hipLaunchKernelGGL((merge_row_kernel<256>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
    else hipLaunchKernelGGL((merge_row_kernel<128>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& m, int head_dim, int grid, hipStream_t stream) {
    if (m.static_units > 0) {
        if (head_dim == 64) hipLaunchKernelGGL((merge_slots_kernel<64>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
        else if (head_dim == 256) hipLaunchKernelGGL((merge_slots_kernel<256>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
        else hipLaunchKernelGGL((merge_slots_kernel<128>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
        return hipGetLastError();
    }
    if (head_dim == 64) hipLaunchKernelGGL((merge_kernel<64, 8>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
    else if (head_dim == 256) hipLaunchKernelGGL((merge_kernel<256, 8>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
    else hipLaunchKernelGGL((merge_kernel<128, 8>), dim3(grid), dim3(kMergeThreads), 0, stream, m);
    return hipGetLastError();
}

}  // namespace pa
