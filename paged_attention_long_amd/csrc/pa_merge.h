// Split-KV partial results and their log-sum-exp merge.
//
// The context of a sequence is cut into splits that run on different
// workgroups; each split leaves its normalised partial output o_s and its
// log2-sum-exp lse_s, and the last workgroup to finish merges them:
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  o = sum_s w_s o_s / sum_s w_s,
//   lse = M + log2(sum_s w_s).
// Splitting along the context and merging the partial results at the end is
// how the pages' decode kernel keeps every compute unit busy ("Dual MI50,
// part 2", section "Decode: a new kernel for the shape MTP actually runs").
// A (sequence, KV head) has at most kMaxSplits splits, so one lane per split
// reads every lse_s in a single round trip; the merge visits splits in index
// order, so results are deterministic.
#pragma once

#include "pa_common.h"

namespace pa {

struct MergeTarget {
    float* out;          // [T][Hq][D]
    float* lse;          // [T][Hq] or null
    int hq;              // query heads
    int group;           // query heads per KV head
    float out_scale;     // multiplies the final output (fp8 V scale, else 1)
};

constexpr int kMergeRows = 64;   // rows merged per pass

// LDS scratch of one merge pass.
struct MergeShared {
    float w[kMergeRows][kMaxSplits];   // normalised split weights
    float lse[kMergeRows];             // final lse (log2 domain)
};

// Row r (token-major: r = i*G + h_in_group) of KV head g -> output row index.
PA_DEVINLINE int64_t out_row(const MergeTarget& t, int q_off, int g, int r) {
    int i = r / t.group;
    int h = g * t.group + (r - i * t.group);
    return (int64_t)(q_off + i) * t.hq + h;
}

// Signal that this workgroup's partial is written; returns true in every
// thread of the workgroup that finished last.  Resets the counter for the
// next call when it is the last one.
PA_DEVINLINE bool arrive_last(int* counter, int n_splits, int* lds_flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        int old = atomicAdd(counter, 1);
        int last = (old == n_splits - 1);
        if (last) {
            atomicExch(counter, 0);
            __threadfence();
        }
        *lds_flag = last;
    }
    __syncthreads();
    bool last = *lds_flag != 0;
    if (last) __threadfence();
    return last;
}

constexpr int kMergeBatch = 16;   // partials in flight per thread

// Merge n_splits (<= kMaxSplits) partials of `rows` rows:
// ws_o[(base + s) * rstride + r][D], ws_lse[(base + s) * rstride + r];
// write them as rows row0 .. row0 + rows - 1 of KV head g.  All threads of
// the block call.  Each thread's first batch of partial rows is requested
// before the weights are known, so the two reads overlap.
template <int D>
PA_DEVINLINE void merge_splits(const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int64_t base,
                               int n_splits, int rows, int rstride, const MergeTarget& t, int q_off, int g,
                               MergeShared& sh, int row0 = 0) {
    const int nthr = blockDim.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int nwaves = nthr / kWave;
    const int64_t sstride = (int64_t)rstride * D;
    for (int r0 = 0; r0 < rows; r0 += kMergeRows) {
        const int nr = min(kMergeRows, rows - r0);
        const int n_el = nr * (D / 4);
        // prefetch the first element's first batch
        const int e0 = threadIdx.x;
        float4 pre[kMergeBatch];
        if (e0 < n_el) {
            const int rl = e0 / (D / 4);
            const float* src = ws_o + ((base * rstride) + r0 + rl) * (int64_t)D + (e0 - rl * (D / 4)) * 4;
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k)
                pre[k] = (k < n_splits) ? *reinterpret_cast<const float4*>(src + k * sstride)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int rl = wid; rl < nr; rl += nwaves) {
            const float ls = (lane < n_splits) ? ws_lse[(base + lane) * rstride + r0 + rl] : kNegInf;
            const float M = wave_max(ls);
            const float w = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
            const float L = wave_sum(w);
            sh.w[rl][lane] = (L > 0.f) ? w / L : 0.f;
            if (lane == 0) sh.lse[rl] = (L > 0.f) ? M + fast_log2(L) : kNegInf;
        }
        __syncthreads();
        for (int e = e0; e < n_el; e += nthr) {
            const int rl = e / (D / 4);
            const int d4 = (e - rl * (D / 4)) * 4;
            const float* src = ws_o + ((base * rstride) + r0 + rl) * (int64_t)D + d4;
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int s0 = 0; s0 < n_splits; s0 += kMergeBatch) {
                float4 o[kMergeBatch];
                if (e == e0 && s0 == 0) {
#pragma unroll
                    for (int k = 0; k < kMergeBatch; ++k) o[k] = pre[k];
                } else {
#pragma unroll
                    for (int k = 0; k < kMergeBatch; ++k)
                        o[k] = (s0 + k < n_splits) ? *reinterpret_cast<const float4*>(src + (s0 + k) * sstride)
                                                   : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int k = 0; k < kMergeBatch; ++k) {
                    const float w = (s0 + k < n_splits) ? sh.w[rl][s0 + k] : 0.f;
                    acc.x = fmaf(w, o[k].x, acc.x);
                    acc.y = fmaf(w, o[k].y, acc.y);
                    acc.z = fmaf(w, o[k].z, acc.z);
                    acc.w = fmaf(w, o[k].w, acc.w);
                }
            }
            const float sc = t.out_scale;
            const int64_t orow = out_row(t, q_off, g, row0 + r0 + rl);
            *reinterpret_cast<float4*>(t.out + orow * D + d4) =
                make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
            if (t.lse != nullptr && d4 == 0) {
                const float l2 = sh.lse[rl];
                t.lse[orow] = (l2 == kNegInf) ? kNegInf : l2 * kLn2;
            }
        }
        __syncthreads();
    }
}

}  // namespace pa
