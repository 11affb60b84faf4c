// Split-KV decode / verify kernel on the vector ALUs (gfx950).
//
// Shape: a few query rows per KV head (decode: the G query heads of one
// token; verify: q_len tokens x G heads) against a long paged context.  The
// work is bound by reading K and V once from HBM, so the kernel is built
// around the loads:
//   * one lane owns 8 consecutive head-dim elements of one token (16 B of an
//     fp16/bf16 row, 8 B of fp8), so D/8 lanes cover a token row and a
//     wavefront reads 64/(D/8) whole token rows per round; a 16-token page of
//     one KV head is one contiguous run in the HND layout, read with
//     128-bit loads;
//   * every key is converted once and scored against every row the wave
//     holds (the pages' decode kernel did the same: "Dual MI50, part 2",
//     section "Decode: a new kernel for the shape MTP actually runs");
//     scores use the packed dot instruction (v_dot2_f32_{bf16,f16}) with an
//     fp32 accumulator and a DPP all-reduce over the D/8 lanes of a token;
//   * each lane keeps its own online-softmax state (running max m, sum l,
//     fp32 accumulator) for the tokens it sees, so no cross-lane reduction
//     runs per page; the max is raised lazily, only when a score exceeds it
//     by more than 2^8 (exact in real arithmetic, fp32 has the range);
//   * masked keys are excluded by select, never multiplied by zero, and the
//     V of a token outside [lo, seq_len) is zeroed before use, so NaN in
//     freed pages, tail slots or padding cannot leak ("Dual MI50, part 2",
//     section "Bug 2: the drafter read freed memory");
//   * the context of each (sequence, KV head) is split across workgroups
//     sized from the live lengths; the partials are combined by the merge
//     launch that follows (log-sum-exp merge, pa_merge.h), or, for static
//     splits on a small grid, by the last workgroup of the group to finish.
#include "pa_common.h"
#include "pa_merge.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kPage = 16;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kTau = 8.0f;   // lazy max: rescale only when a score exceeds m by 2^8

template <int KVT>
struct KvChunk;
template <>
struct KvChunk<PA_DTYPE_F16> { using T = u32x4_t; static constexpr int bytes = 2; };
template <>
struct KvChunk<PA_DTYPE_BF16> { using T = u32x4_t; static constexpr int bytes = 2; };
template <>
struct KvChunk<PA_DTYPE_FP8_E4M3> { using T = u32x2_t; static constexpr int bytes = 1; };
template <>
struct KvChunk<PA_DTYPE_INT8> { using T = u32x2_t; static constexpr int bytes = 1; };

template <int KVT>
PA_DEVINLINE typename KvChunk<KVT>::T load_chunk(const uint8_t* p) {
    if constexpr (KvChunk<KVT>::bytes == 1) return load_b64(p);
    else return load_b128(p);
}

// Eight K elements -> four packed pairs in the dot-product type QT.
template <int KVT, int QT>
PA_DEVINLINE void k_pairs(const typename KvChunk<KVT>::T& c, uint32_t kp[4]) {
    if constexpr (KVT == PA_DTYPE_FP8_E4M3) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t w = c[i];
            f32x2_t lo = fp8x2_to_f32(w, false);
            f32x2_t hi = fp8x2_to_f32(w, true);
            if constexpr (QT == PA_DTYPE_BF16) {
                kp[2 * i] = f32x2_to_bf16x2(lo);
                kp[2 * i + 1] = f32x2_to_bf16x2(hi);
            } else {
                kp[2 * i] = f32x2_to_f16x2(lo);
                kp[2 * i + 1] = f32x2_to_f16x2(hi);
            }
        }
    } else if constexpr (KVT == PA_DTYPE_INT8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if constexpr (QT == PA_DTYPE_BF16) i8x4_to_bf16x4(c[i], kp[2 * i], kp[2 * i + 1]);
            else i8x4_to_f16x4(c[i], kp[2 * i], kp[2 * i + 1]);
        }
    } else {
        kp[0] = c[0]; kp[1] = c[1]; kp[2] = c[2]; kp[3] = c[3];
    }
}

// Eight V elements -> fp32.
template <int KVT>
PA_DEVINLINE void v_floats(const typename KvChunk<KVT>::T& c, float v[8]) {
    if constexpr (KVT == PA_DTYPE_FP8_E4M3) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            f32x2_t lo = fp8x2_to_f32(c[i], false);
            f32x2_t hi = fp8x2_to_f32(c[i], true);
            v[4 * i] = lo.x; v[4 * i + 1] = lo.y; v[4 * i + 2] = hi.x; v[4 * i + 3] = hi.y;
        }
    } else if constexpr (KVT == PA_DTYPE_INT8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float f[4];
            i8x4_to_f32x4(c[i], f);
            v[4 * i] = f[0]; v[4 * i + 1] = f[1]; v[4 * i + 2] = f[2]; v[4 * i + 3] = f[3];
        }
    } else if constexpr (KVT == PA_DTYPE_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[2 * i] = bf16lo_to_f32(c[i]); v[2 * i + 1] = bf16hi_to_f32(c[i]); }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f32x2_t f = f16x2_to_f32(c[i]); v[2 * i] = f.x; v[2 * i + 1] = f.y; }
    }
}

template <int D>
struct WaveShared {
    float acc[kWaves][8][D];     // [wave][row][d] (RW <= 8)
    float m[kWaves][8];
    float l[kWaves][8];
};

constexpr int kPidChunk = kPidChunkPages;   // page ids staged in LDS at a time

template <int D>
struct Smem {
    Plan plan;
    int stat[4];
    int pid[kPidChunk];
    union {
        WaveShared<D> ws;
    } u;
};

template <int D, int KVT, int QT, int RW>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
    constexpr int LPT = D / 8;            // lanes per token row
    constexpr int TPR = kWave / LPT;      // tokens per round
    constexpr int RPP = kPage / TPR;      // rounds per page
    constexpr int EB = KvChunk<KVT>::bytes;
    using Chunk = typename KvChunk<KVT>::T;

    __shared__ Smem<D> sm;
    extern __shared__ int dyn_lds[];
    Plan& pl = sm.plan;
    if (a.static_pps <= 0)
        build_plan(pl, dyn_lds, a, a.seq_lens, a.q_lens, a.num_seqs, a.window, kPage, a.group, a.num_kv_heads,
                   a.target_items, a.min_pps, a.forced_pps, a.max_items);
    const int n_items = (a.static_pps <= 0) ? pl.n_items : 0;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int tl = lane / LPT;            // token within a round
    const int ch = lane % LPT;            // 8-element chunk of the row

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
    MergeTarget tgt{a.out, a.lse, a.num_q_heads, a.group, 1.0f};
    const int64_t page_bytes = a.page_stride * EB;

    // One work item: pages [p_begin, p_end) of sequence b, KV head g, whose
    // partial goes to slot `it`; the (b, g) pair has n_splits items starting
    // at first_item.  With pid_ready the page ids of the first chunk are
    // already in sm.pid.
    auto run_item = [&](const SeqInfo& si, int b, int g, int it, int p_begin, int p_end, int64_t first_item,
                        int n_splits, bool pid_ready) {
        const int rows = si.q_len * a.group;
        const int n_rg = (rows + RW - 1) / RW;
        const float kscale = (KVT == PA_DTYPE_FP8_E4M3) ? a.kv_scale[g] : 1.0f;
        const float vscale = (KVT == PA_DTYPE_FP8_E4M3) ? a.kv_scale[a.num_kv_heads + g] : 1.0f;
        const float s2 = a.scale * kLog2e * kscale;
        tgt.out_scale = vscale;
        const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
        const bool direct = (n_splits == 1);
        // byte offset of this lane's chunk inside a page, per round (< 2^31: checked on the host)
        uint32_t lane_off[RPP];
#pragma unroll
        for (int rr = 0; rr < RPP; ++rr)
            lane_off[rr] = (uint32_t)(kv_offset(0, g, rr * TPR + tl, a.page_stride, a.head_stride, a.token_stride) * EB +
                                      ch * 8 * EB);
        // int8: this lane's token row scales, at rs_page * page + lane_soff[rr]
        constexpr bool ROWSC = (KVT == PA_DTYPE_INT8);
        int64_t lane_soff[ROWSC ? RPP : 1];
        if constexpr (ROWSC) {
#pragma unroll
            for (int rr = 0; rr < RPP; ++rr) lane_soff[rr] = (int64_t)g * a.rs_head + (int64_t)(rr * TPR + tl) * a.rs_tok;
        }

        // passes over row groups: up to kWaves row groups at a time
        for (int rg0 = 0; rg0 < n_rg; rg0 += kWaves) {
            const int n_here = min(kWaves, n_rg - rg0);
            const int wprg = kWaves / n_here;           // waves per row group
            const int rg = rg0 + wid / wprg;
            const int sub = wid % wprg;
            const bool active = (wid < n_here * wprg);

            float m[RW], l[RW], acc[RW][8];
            int pos[RW], lo_r[RW];
            uint32_t qv[RW][4];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                m[r] = kNegInf; l[r] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
                const int row = rg * RW + r;
                const bool valid = active && row < rows;
                const int i = valid ? row / a.group : 0;
                const int h = g * a.group + (valid ? row - i * a.group : 0);
                pos[r] = valid ? si.seq_len - si.q_len + i : -1;   // -1: sees nothing
                lo_r[r] = (a.window > 0) ? pos[r] - a.window + 1 : 0;
                if (valid) {
                    const u32x4_t qq = load_b128_cached(qbase + ((int64_t)(si.q_off + i) * a.num_q_heads + h) * D + ch * 8);
                    qv[r][0] = qq[0]; qv[r][1] = qq[1]; qv[r][2] = qq[2]; qv[r][3] = qq[3];
                } else {
                    qv[r][0] = qv[r][1] = qv[r][2] = qv[r][3] = 0u;
                }
            }

            for (int c0 = p_begin; c0 < p_end; c0 += kPidChunk) {
                const int c1 = min(p_end, c0 + kPidChunk);
                if (!(pid_ready && c0 == p_begin && rg0 == 0)) {
                    __syncthreads();
                    for (int k = tid; k < c1 - c0; k += kThreads) sm.pid[k] = chunk_page(bt, c0 + k, a);
                }
                __syncthreads();
                if (active) {
                    // Two page buffers in ping-pong: the next page's loads are in flight
                    // while the current one is scored (no register copies of pending loads).
                    Chunk ka[RPP], va[RPP], kb[RPP], vb[RPP];
                    // int8 row scales of the tokens the chunks hold (K, V)
                    float ska[ROWSC ? RPP : 1], sva[ROWSC ? RPP : 1], skb[ROWSC ? RPP : 1], svb[ROWSC ? RPP : 1];
                    auto issue = [&](Chunk (&kd)[RPP], Chunk (&vd)[RPP], float (&sk)[ROWSC ? RPP : 1],
                                     float (&sv)[ROWSC ? RPP : 1], int pg) {
                        // wave-uniform page base (scalar registers) + per-lane 32-bit offsets
                        const int pid = __builtin_amdgcn_readfirstlane(sm.pid[pg - c0]);
                        const int64_t pbase = (int64_t)pid * page_bytes;
                        const uint8_t* kp = kbase + pbase;
                        const uint8_t* vp = vbase + pbase;
#pragma unroll
                        for (int rr = 0; rr < RPP; ++rr) {
                            kd[rr] = load_chunk<KVT>(kp + lane_off[rr]);
                            vd[rr] = load_chunk<KVT>(vp + lane_off[rr]);
                        }
                        if constexpr (ROWSC) {
                            const float* rk = a.row_scale + (int64_t)pid * a.rs_page;
#pragma unroll
                            for (int rr = 0; rr < RPP; ++rr) {
                                sk[rr] = __builtin_nontemporal_load(rk + lane_soff[rr]);
                                sv[rr] = __builtin_nontemporal_load(rk + a.rs_v + lane_soff[rr]);
                            }
                        }
                    };
                    auto consume = [&](const Chunk (&kd)[RPP], const Chunk (&vd)[RPP], const float (&sk)[ROWSC ? RPP : 1],
                                       const float (&sv)[ROWSC ? RPP : 1], int pg) {
#pragma unroll
                        for (int rr = 0; rr < RPP; ++rr) {
                            const int j = pg * kPage + rr * TPR + tl;
                            const bool live = (j >= si.lo) && (j < si.seq_len);
                            // int8: the key's own scale folds into its score; the value's
                            // multiplies its weight (0 for a dead key, whose scale may be NaN)
                            const float s2j = ROWSC ? s2 * sk[ROWSC ? rr : 0] : s2;
                            const float svj = ROWSC ? (live ? sv[ROWSC ? rr : 0] : 0.f) : 1.f;
                            uint32_t kp[4];
                            k_pairs<KVT, QT>(kd[rr], kp);
                            float s[RW];
#pragma unroll
                            for (int r = 0; r < RW; ++r) {
                                float x = dot2<QT>(qv[r][0], kp[0], 0.f);
                                x = dot2<QT>(qv[r][1], kp[1], x);
                                x = dot2<QT>(qv[r][2], kp[2], x);
                                x = dot2<QT>(qv[r][3], kp[3], x);
                                s[r] = group_sum<LPT>(x);
                            }
                            bool need = false;
#pragma unroll
                            for (int r = 0; r < RW; ++r) {
                                const bool vis = (j <= pos[r]) && (j >= lo_r[r]) && live;
                                s[r] = vis ? s[r] * s2j : kNegInf;
                                need |= s[r] > m[r] + kTau;
                            }
                            if (__builtin_expect(wave_any(need), 0)) {
#pragma unroll
                                for (int r = 0; r < RW; ++r) {
                                    const bool nd = s[r] > m[r] + kTau;
                                    const float al = nd ? fast_exp2(m[r] - s[r]) : 1.0f;
                                    m[r] = nd ? s[r] : m[r];
                                    l[r] *= al;
#pragma unroll
                                    for (int e = 0; e < 8; ++e) acc[r][e] *= al;
                                }
                            }
                            float v[8];
                            v_floats<KVT>(vd[rr], v);
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] = live ? v[e] : 0.f;
#pragma unroll
                            for (int r = 0; r < RW; ++r) {
                                const float p = (s[r] == kNegInf) ? 0.f : fast_exp2(s[r] - m[r]);
                                l[r] += p;
                                const float pv = ROWSC ? p * svj : p;
#pragma unroll
                                for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pv, v[e], acc[r][e]);
                            }
                        }
                    };
                    // The prefetch is unconditional (past the end it re-reads a page this
                    // wave already holds) so the wait counts are the same on every path.
                    int pg = c0 + sub;
                    if (pg < c1) {
                        issue(ka, va, ska, sva, pg);
                        while (true) {
                            const int p1 = pg + wprg;
                            issue(kb, vb, skb, svb, p1 < c1 ? p1 : pg);
                            consume(ka, va, ska, sva, pg);
                            if (p1 >= c1) break;
                            const int p2 = p1 + wprg;
                            issue(ka, va, ska, sva, p2 < c1 ? p2 : p1);
                            consume(kb, vb, skb, svb, p1);
                            if (p2 >= c1) break;
                            pg = p2;
                        }
                    }
                }
                __syncthreads();
            }

            // merge the TPR token lanes of this wave (lanes ch, ch+LPT, ...)
            auto lanes_max = [](float x) {
                if constexpr (LPT <= 8) x = xor_max<8>(x);
                if constexpr (LPT <= 16) x = xor_max<16>(x);
                return xor_max<32>(x);
            };
            auto lanes_sum = [](float x) {
                if constexpr (LPT <= 8) x = xor_sum<8>(x);
                if constexpr (LPT <= 16) x = xor_sum<16>(x);
                return xor_sum<32>(x);
            };
            static_assert(LPT == 8 || LPT == 16 || LPT == 32, "token lanes differ in lane bits 3..5, 4..5 or 5");
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float M = lanes_max(m[r]);
                const float al = (m[r] == kNegInf) ? 0.f : fast_exp2(m[r] - M);
                const float lr = lanes_sum(l[r] * al);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] = lanes_sum(acc[r][e] * al);
                m[r] = M;
                l[r] = lr;
            }
            if (active && tl == 0) {
#pragma unroll
                for (int r = 0; r < RW; ++r) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) sm.u.ws.acc[wid][r][ch * 8 + e] = acc[r][e];
                    if (ch == 0) { sm.u.ws.m[wid][r] = m[r]; sm.u.ws.l[wid][r] = l[r]; }
                }
            }
            __syncthreads();
            // combine the waves of each row group; write final rows or split partials
            const int rows_here = min(rows - rg0 * RW, n_here * RW);
            for (int e = tid; e < rows_here * D; e += kThreads) {
                const int rl = e / D;              // row within this pass
                const int d = e - rl * D;
                const int rgl = rl / RW;           // row group within this pass
                const int r = rl - rgl * RW;
                const int w0 = rgl * wprg;
                float M = kNegInf;
                for (int w = 0; w < wprg; ++w) M = fmaxf(M, sm.u.ws.m[w0 + w][r]);
                float L = 0.f, A = 0.f;
                if (M != kNegInf) {
                    for (int w = 0; w < wprg; ++w) {
                        const float mw = sm.u.ws.m[w0 + w][r];
                        const float al = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
                        L = fmaf(sm.u.ws.l[w0 + w][r], al, L);
                        A = fmaf(sm.u.ws.acc[w0 + w][r][d], al, A);
                    }
                }
                const int row = rg0 * RW + rl;
                if (direct) {
                    const int64_t orow = out_row(tgt, si.q_off, g, row);
                    a.out[orow * D + d] = (L > 0.f) ? A * vscale / L : 0.f;
                    if (a.lse != nullptr && d == 0) a.lse[orow] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
                } else {
                    const int64_t slot = (int64_t)it * a.r_max + row;
                    a.ws_o[slot * D + d] = (L > 0.f) ? A / L : 0.f;
                    if (d == 0) a.ws_lse[slot] = (L > 0.f) ? M + fast_log2(L) : kNegInf;
                }
            }
            __syncthreads();
        }

        if (!direct && a.arrive != nullptr) {
            // In-kernel merge (static splits, small grids).  Every thread
            // releases its partial stores at device scope, the barrier joins
            // them, and one device-scope acquire-release increment counts the
            // workgroup in.  The workgroup that completes the count acquires
            // every other workgroup's partials, merges the group (splits in
            // index order, an online max) and clears the counter.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (tid == 0) {
                int* cnt = a.arrive + b * a.num_kv_heads + g;
                const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                const int last = (old == n_splits - 1);
                if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sm.stat[3] = last;
            }
            __syncthreads();
            if (sm.stat[3]) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                constexpr int EPR = D / 4;                 // float4 columns per row
                constexpr int NB = 16;                     // partials in flight per thread
                for (int r0 = 0; r0 < rows; r0 += kThreads / EPR) {
                    const int rl = r0 + tid / EPR;
                    const int col = (tid % EPR) * 4;
                    if (rl < rows) {
                        float M = kNegInf, L = 0.f;
                        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
                        for (int s0 = 0; s0 < n_splits; s0 += NB) {
                            float ls[NB];
                            float4 o[NB];
#pragma unroll
                            for (int k = 0; k < NB; ++k) {
                                const int64_t slot = (first_item + min(s0 + k, n_splits - 1)) * a.r_max + rl;
                                ls[k] = a.ws_lse[slot];
                                o[k] = *reinterpret_cast<const float4*>(a.ws_o + slot * D + col);
                            }
#pragma unroll
                            for (int k = 0; k < NB; ++k) {
                                if (s0 + k < n_splits && ls[k] != kNegInf) {
                                    if (ls[k] > M) {
                                        const float sc = (M == kNegInf) ? 0.f : fast_exp2(M - ls[k]);
                                        L *= sc;
                                        acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
                                        M = ls[k];
                                    }
                                    const float w = fast_exp2(ls[k] - M);
                                    L += w;
                                    acc.x = fmaf(w, o[k].x, acc.x);
                                    acc.y = fmaf(w, o[k].y, acc.y);
                                    acc.z = fmaf(w, o[k].z, acc.z);
                                    acc.w = fmaf(w, o[k].w, acc.w);
                                }
                            }
                        }
                        const int64_t orow = out_row(tgt, si.q_off, g, rl);
                        const float sc = (L > 0.f) ? vscale / L : 0.f;
                        *reinterpret_cast<float4*>(a.out + orow * D + col) =
                            make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
                        if (a.lse != nullptr && col == 0) a.lse[orow] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
                    }
                }
            }
        } else if (!direct && it == first_item && tid == 0) {
            const MergeDesc d{(int)first_item, n_splits, rows, a.r_max, si.q_off, g, 0, vscale};
            if (a.sdesc != nullptr) {
                // fixed slots, one per merge unit the group's rows cover
                MergeDesc* slot = a.sdesc + (int64_t)(b * a.num_kv_heads + g) * a.sdesc_upg;
                const int units = (rows + merge_rpu(D) - 1) / merge_rpu(D);
                for (int u = 0; u < units; ++u) slot[u] = d;
            } else {
                publish_merge(a, d);
            }
        }
    };

    if (a.static_pps > 0) {
        // Static split mode (small batches): workgroup -> (sequence, KV head,
        // split of static_pps pages counted from page 0).  The sequence's
        // lengths, its query offset and the split's page ids are fetched in
        // one round trip; splits outside the visible pages leave at once.
        const int S = a.static_splits;
        const int it = blockIdx.x;
        const int b = it / (a.num_kv_heads * S);
        const int rem = it - b * a.num_kv_heads * S;
        const int g = rem / S;
        const int split = rem - g * S;
        if (b >= a.num_seqs) return;
        const int pps = a.static_pps;
        const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
        // (checked mode: only the sequence's own pages are staged, below)
        if (!a.checks)
            for (int k = tid; k < pps; k += kThreads)
                sm.pid[k] = (split * pps + k < a.bt_chunks) ? chunk_page(bt, split * pps + k, a) : 0;
        if (wid == 0) {
            int qs = 0;
            for (int b0 = 0; b0 < b; b0 += kWave)
                qs += (b0 + lane < b) ? checked_q_len(a, a.seq_lens[b0 + lane], a.q_lens[b0 + lane]) : 0;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) qs += __shfl_xor(qs, o, kWave);
            if (lane == 0) {
                const int sl = a.seq_lens[b];
                int ql = checked_q_len(a, sl, a.q_lens[b]);
                if (a.checks && ql > 0 && (int64_t)qs + ql > a.num_tokens) {
                    debug_flag(a.err_word, PA_CHECK_TOKENS);
                    ql = 0;
                }
                sm.stat[0] = sl;
                sm.stat[1] = ql;
                sm.stat[2] = qs;
            }
        }
        __syncthreads();
        SeqInfo si;
        si.seq_len = sm.stat[0];
        si.q_len = sm.stat[1];
        si.q_off = sm.stat[2];
        si.lo = seq_visible_lo(si.seq_len, si.q_len, a.window);
        si.first_page = si.lo / kPage;
        const int rows = si.q_len * a.group;
        if (si.q_len <= 0 || !in_launch(a, rows, si.seq_len - si.lo)) return;
        const int last_page = (si.seq_len - 1) / kPage;
        si.n_pages = last_page - si.first_page + 1;
        const int s_first = si.first_page / pps, s_last = last_page / pps;
        if (split < s_first || split > s_last) return;
        si.splits = s_last - s_first + 1;
        const int p_begin = max(split * pps, si.first_page);
        const int p_end = min((split + 1) * pps, last_page + 1);
        if (a.checks || p_begin > split * pps) {   // window start inside this split: realign the staged ids
            __syncthreads();
            for (int k = tid; k < p_end - p_begin; k += kThreads) sm.pid[k] = chunk_page(bt, p_begin + k, a);
            __syncthreads();
        }
        const int64_t first_item = (int64_t)(b * a.num_kv_heads + g) * S + s_first;
        run_item(si, b, g, it, p_begin, p_end, first_item, si.splits, true);
        return;
    }

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int b = item_seq(pl, a.num_seqs, it);
        const SeqInfo si = seq_info(pl, b, a.window, kPage);
        const int local = it - pl.item_base[b];
        const int g = local / si.splits;
        const int split = local - g * si.splits;
        const int p_begin = si.first_page + split * pl.pps;
        const int p_end = min(si.first_page + si.n_pages, p_begin + pl.pps);
        const int64_t first_item = pl.item_base[b] + (int64_t)g * si.splits;
        run_item(si, b, g, it, p_begin, p_end, first_item, si.splits, false);
    }
}

}  // namespace

template <int D, int KVT, int QT, int RW>
static hipError_t launch_t(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((decode_valu_kernel<D, KVT, QT, RW>), dim3(grid), dim3(kThreads), plan_lds_bytes(a.num_seqs), st,
                       a);
    return hipGetLastError();
}

template <int D, int KVT, int QT>
static hipError_t launch_rw(const DecodeArgs& a, int rw, int grid, hipStream_t st) {
    switch (rw) {
        case 1: return launch_t<D, KVT, QT, 1>(a, grid, st);
        case 2: return launch_t<D, KVT, QT, 2>(a, grid, st);
        case 4: return launch_t<D, KVT, QT, 4>(a, grid, st);
        default: return launch_t<D, KVT, QT, 8>(a, grid, st);
    }
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, int kvt, int qt, int rw, int grid, hipStream_t st) {
    if (kvt == PA_DTYPE_F16) return launch_rw<D, PA_DTYPE_F16, PA_DTYPE_F16>(a, rw, grid, st);
    if (kvt == PA_DTYPE_BF16) return launch_rw<D, PA_DTYPE_BF16, PA_DTYPE_BF16>(a, rw, grid, st);
    if (kvt == PA_DTYPE_INT8) {
        if (qt == PA_DTYPE_BF16) return launch_rw<D, PA_DTYPE_INT8, PA_DTYPE_BF16>(a, rw, grid, st);
        return launch_rw<D, PA_DTYPE_INT8, PA_DTYPE_F16>(a, rw, grid, st);
    }
    if (qt == PA_DTYPE_BF16) return launch_rw<D, PA_DTYPE_FP8_E4M3, PA_DTYPE_BF16>(a, rw, grid, st);
    return launch_rw<D, PA_DTYPE_FP8_E4M3, PA_DTYPE_F16>(a, rw, grid, st);
}

hipError_t launch_decode_valu(const DecodeArgs& a, int head_dim, int kv_dtype, int q_dtype, int rw, int grid,
                              hipStream_t stream) {
    if (head_dim == 64) return launch_d<64>(a, kv_dtype, q_dtype, rw, grid, stream);
    if (head_dim == 256) return launch_d<256>(a, kv_dtype, q_dtype, rw, grid, stream);
    return launch_d<128>(a, kv_dtype, q_dtype, rw, grid, stream);
}

}  // namespace pa
