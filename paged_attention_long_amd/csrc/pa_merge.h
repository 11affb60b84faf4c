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
// The merge visits splits in index order, so results are deterministic.
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

// Merge n_splits partials of `rows` rows: ws_o[(base + s) * rstride + r][D],
// ws_lse[(base + s) * rstride + r]; write final rows.  All threads call.
template <int D>
PA_DEVINLINE void merge_splits(const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int64_t base,
                               int n_splits, int rows, int rstride, const MergeTarget& t, int q_off, int g) {
    const int nthr = blockDim.x;
    const int total = rows * (D / 4);
    for (int e = threadIdx.x; e < total; e += nthr) {
        const int r = e / (D / 4);
        const int d4 = (e - r * (D / 4)) * 4;
        float M = kNegInf;
        for (int s = 0; s < n_splits; ++s) M = fmaxf(M, ws_lse[(base + s) * rstride + r]);
        float L = 0.f;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        if (M != kNegInf) {
            for (int s = 0; s < n_splits; ++s) {
                const int64_t slot = (base + s) * rstride + r;
                const float ls = ws_lse[slot];
                const float w = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
                const float4 o = *reinterpret_cast<const float4*>(ws_o + slot * D + d4);
                L += w;
                a0 = fmaf(w, o.x, a0);
                a1 = fmaf(w, o.y, a1);
                a2 = fmaf(w, o.z, a2);
                a3 = fmaf(w, o.w, a3);
            }
        }
        const float inv = (L > 0.f) ? t.out_scale / L : 0.f;
        const int64_t orow = out_row(t, q_off, g, r);
        *reinterpret_cast<float4*>(t.out + orow * D + d4) = make_float4(a0 * inv, a1 * inv, a2 * inv, a3 * inv);
        if (t.lse != nullptr && d4 == 0) t.lse[orow] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
    }
}

}  // namespace pa
