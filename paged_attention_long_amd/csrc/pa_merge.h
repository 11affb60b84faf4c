// Split-KV partial results and their log-sum-exp merge.
//
// The context of a sequence is cut into splits that run on different
// workgroups; each split leaves its normalised partial output o_s and its
// log2-sum-exp lse_s:
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  o = sum_s w_s o_s / sum_s w_s,
//   lse = M + log2(sum_s w_s).
// Splitting along the context and merging the partial results at the end is
// how the pages' decode kernel keeps every compute unit busy ("Dual MI50,
// part 2", section "Decode: a new kernel for the shape MTP actually runs").
//
// The workgroup that runs a group's first split publishes a descriptor; a
// separate merge launch, ordered after the attention kernels on the stream,
// merges every published group with all of its threads.  The kernel boundary
// makes the partials visible, so those attention kernels need no device-wide
// fences or arrival counters.  The one exception is static-split decode on
// a small grid, where the last workgroup of each group to arrive (a
// device-scope acquire-release count) merges the group inside the decode
// kernel.  Splits are visited in index order, so results are deterministic.
// A group has at most kMaxSplits splits.
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

// Called by one thread: append this group to the forward's merge list.
PA_DEVINLINE void publish_merge(const DecodeArgs& a, const MergeDesc& d) {
    const int idx = __hip_atomic_fetch_add(a.mcount, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.mdesc[idx] = d;
}

}  // namespace pa
