// Device-side building blocks shared by the paged-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paged_attn.h"
#include "pa_kernels.h"

#define PA_DEVINLINE __device__ __forceinline__

namespace pa {

constexpr int kMaxSeqs = 1024;          // largest num_seqs a handle accepts
constexpr int kWave = 64;               // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- loads

// 16-byte global load (global_load_dwordx4); p must be 16-B aligned.
PA_DEVINLINE u32x4_t load_b128(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
PA_DEVINLINE u32x4_t load_b128_cached(const void* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}
PA_DEVINLINE u32x2_t load_b64(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

// ----------------------------------------------------------------- conversions

PA_DEVINLINE float bf16lo_to_f32(uint32_t u) { return __uint_as_float(u << 16); }
PA_DEVINLINE float bf16hi_to_f32(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

PA_DEVINLINE f32x2_t f16x2_to_f32(uint32_t u) {
    f16x2_t h = __builtin_bit_cast(f16x2_t, u);
    return f32x2_t{(float)h.x, (float)h.y};
}

// Two OCP E4M3FN bytes (low or high half of u) -> two floats, exact.
PA_DEVINLINE f32x2_t fp8x2_to_f32(uint32_t u, bool hi) {
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(u, true) : __builtin_amdgcn_cvt_pk_f32_fp8(u, false);
}

// Four int8 codes (one dword) -> four f16 values, exactly, as two packed
// pairs (codes 0, 1 in lo; 2, 3 in hi).  Each byte b (signed v) becomes
// u = v + 128 (flip its top bit); the f16 with bits 0x64uu is 1024 + u
// (the unit in the last place of [1024, 2048) is 1), and subtracting 1152
// in packed f16 leaves v.
PA_DEVINLINE void i8x4_to_f16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const uint32_t u = w ^ 0x80808080u;
    // v_perm_b32: selector byte k picks byte k of {src1 (0..3), src0 (4..7)}
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const f16x2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) - off);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, b) - off);
}

// Four int8 codes -> four floats, exactly: the float with bits 0x4B0000uu is
// 2^23 + u (u = v + 128), and subtracting 2^23 + 128 leaves v.
PA_DEVINLINE void i8x4_to_f32x4(uint32_t w, float (&f)[4]) {
    const uint32_t u = w ^ 0x80808080u;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        f[k] = __uint_as_float(0x4B000000u | ((u >> (8 * k)) & 0xffu)) - 8388736.0f;
}

// Four int8 codes -> four bf16 values, exactly (|v| <= 128 has at most 8
// significant bits, so the upper half of its float is the bf16 value).
PA_DEVINLINE void i8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    float f[4];
    i8x4_to_f32x4(w, f);
    lo = __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
    hi = __builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u);
}

// Exact narrowing of two floats that are representable in bf16 / f16.
PA_DEVINLINE uint32_t f32x2_to_bf16x2(f32x2_t f) {
    bf16x2_t b = {(__bf16)f.x, (__bf16)f.y};
    return __builtin_bit_cast(uint32_t, b);
}
PA_DEVINLINE uint32_t f32x2_to_f16x2(f32x2_t f) {
    f16x2_t h = {(_Float16)f.x, (_Float16)f.y};
    return __builtin_bit_cast(uint32_t, h);
}

// Dot product of two packed pairs, accumulated in fp32 (v_dot2_f32_{bf16,f16}).
template <int QT>
PA_DEVINLINE float dot2(uint32_t a, uint32_t b, float c);
template <>
PA_DEVINLINE float dot2<PA_DTYPE_BF16>(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}
template <>
PA_DEVINLINE float dot2<PA_DTYPE_F16>(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// ----------------------------------------------------------------- cross-lane

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // reverse within each 8-lane half row
constexpr int kDppRowMirror = 0x140;    // reverse within each 16-lane row
constexpr int kDppRowShr = 0x110;       // + n: shift right by n lanes within each row
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 to rows 2 and 3

template <int CTRL>
PA_DEVINLINE float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// All-reduce over aligned groups of N lanes (N = 8 or 16 inside a row, 32: two rows).
template <int N>
PA_DEVINLINE float group_sum(float x) {
    static_assert(N == 8 || N == 16 || N == 32, "group size");
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N == 32) {
        // rows 2k and 2k+1 exchange through the gfx950 row swap (the sum of
        // the pair is the same on both lanes)
        const uint32_t u = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}

PA_DEVINLINE float shfl_xor(float x, int m) { return __shfl_xor(x, m, kWave); }

// Returns {x[l], x[l ^ O]} (in some order) on every lane l.  O = 16 and 32 use
// the gfx950 row and half-wave swaps (VALU, no LDS round trip); smaller O a
// cross-lane permute.
template <int O>
PA_DEVINLINE f32x2_t xor_pair(float x) {
    if constexpr (O == 16 || O == 32) {
        const uint32_t u = __float_as_uint(x);
        const auto r = (O == 16) ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                                 : __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return f32x2_t{__uint_as_float(r[0]), __uint_as_float(r[1])};
    } else {
        return f32x2_t{x, __shfl_xor(x, O, kWave)};
    }
}
template <int O>
PA_DEVINLINE float xor_sum(float x) {
    const f32x2_t p = xor_pair<O>(x);
    return p.x + p.y;
}
template <int O>
PA_DEVINLINE float xor_max(float x) {
    const f32x2_t p = xor_pair<O>(x);
    return fmaxf(p.x, p.y);
}

PA_DEVINLINE float wave_max(float x) {
    x = xor_max<32>(x);
    x = xor_max<16>(x);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
    return x;
}
PA_DEVINLINE float wave_sum(float x) {
    x = xor_sum<32>(x);
    x = xor_sum<16>(x);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}


PA_DEVINLINE bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Inclusive prefix sum over the wave without LDS: shifts by 1, 2, 4, 8 within
// each 16-lane row (zeros shifted in), then the last lane of row 0 is added to
// rows 1 and 3 and the last lane of row 1 (now rows 0-1) to rows 2 and 3.
PA_DEVINLINE int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 1, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 2, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 4, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 8, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xC, 0xF, false);
    return x;
}

// Sum / maximum over the wave without LDS; every lane gets the result.
// Quads, half rows and rows combine through DPP (each step pairs two groups
// that already hold their own totals), then rows and wave halves through the
// lane swaps.
template <int CTRL>
PA_DEVINLINE int dpp_i32(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false); }
template <int O>
PA_DEVINLINE void xor_pair_u32(uint32_t x, uint32_t& a, uint32_t& b) {
    const auto r = (O == 16) ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                             : __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
}
PA_DEVINLINE int wave_max_i32(int x) {
    x = max(x, dpp_i32<kDppQuadXor1>(x));
    x = max(x, dpp_i32<kDppQuadXor2>(x));
    x = max(x, dpp_i32<kDppHalfMirror>(x));
    x = max(x, dpp_i32<kDppRowMirror>(x));
    uint32_t a, b;
    xor_pair_u32<16>((uint32_t)x, a, b);
    x = max((int)a, (int)b);
    xor_pair_u32<32>((uint32_t)x, a, b);
    return max((int)a, (int)b);
}
// 64-bit sum: each lane's value is split into 32-bit halves that travel
// through the same lane moves; the halves are recombined before each add.
PA_DEVINLINE long long wave_sum_i64(long long v) {
    auto join = [](uint32_t lo, uint32_t hi) { return (long long)(((unsigned long long)hi << 32) | lo); };
    auto step_dpp = [&](auto ctrl_c) {
        constexpr int C = decltype(ctrl_c)::value;
        const uint32_t lo = (uint32_t)dpp_i32<C>((int)(uint32_t)v);
        const uint32_t hi = (uint32_t)dpp_i32<C>((int)(uint32_t)((unsigned long long)v >> 32));
        v += join(lo, hi);
    };
    step_dpp(std::integral_constant<int, kDppQuadXor1>{});
    step_dpp(std::integral_constant<int, kDppQuadXor2>{});
    step_dpp(std::integral_constant<int, kDppHalfMirror>{});
    step_dpp(std::integral_constant<int, kDppRowMirror>{});
    auto step_swap = [&](auto o_c) {
        constexpr int O = decltype(o_c)::value;
        uint32_t la, lb, ha, hb;
        xor_pair_u32<O>((uint32_t)v, la, lb);
        xor_pair_u32<O>((uint32_t)((unsigned long long)v >> 32), ha, hb);
        v = join(la, ha) + join(lb, hb);
    };
    step_swap(std::integral_constant<int, 16>{});
    step_swap(std::integral_constant<int, 32>{});
    return v;
}

// ceil(a / b) for 0 <= a, 0 < b; 32-bit division when both fit (uniform branch)
PA_DEVINLINE long long div_ceil_i64(long long a, long long b) {
    if (((unsigned long long)a | (unsigned long long)b) >> 31 == 0) {
        const uint32_t ua = (uint32_t)a, ub = (uint32_t)b;
        return (long long)((ua + ub - 1u) / ub);
    }
    return (a + b - 1) / b;
}

PA_DEVINLINE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
PA_DEVINLINE float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ----------------------------------------------------------------- positions

// Visible key range of the new rows of one sequence: [lo, seq_len).
PA_DEVINLINE int seq_visible_lo(int seq_len, int q_len, int window) {
    return window > 0 ? max(0, seq_len - q_len - window + 1) : 0;
}

// Element offset of token slot `slot` of KV head g in physical page `page`.
PA_DEVINLINE int64_t kv_offset(int64_t page, int g, int slot, int64_t page_stride, int64_t head_stride,
                               int64_t token_stride) {
    return page * page_stride + (int64_t)g * head_stride + (int64_t)slot * token_stride;
}

// Virtual page holding 16-token chunk c of the sequence whose block-table row
// is bt (c < 2^24).  With 16-token pages it is the page id itself.  A page of
// P = 16 * cpp tokens is cut into cpp virtual pages of 16 token rows each:
// chunk c is virtual page bt[c / cpp] * vr + c % cpp, and the kernels address
// virtual pages with a stride of 16 token rows, so every kernel keeps its
// 16-token loops for any page size that is a multiple of 16 ("Dual MI50,
// part 2", section "Prefill: teach the fork's fast kernel to read the int8
// cache": the cache is read in place at any block size).  The quotient is a
// multiply-high and a shift with a magic number from the host.
// In the checked mode a page id outside [0, num_pages) is reported and
// replaced by page 0, so no access leaves the pool.
PA_DEVINLINE void debug_flag(int* err_word, int bit) {
    __hip_atomic_fetch_or(err_word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename BT>
PA_DEVINLINE int chunk_page(BT bt, int c, const DecodeArgs& a) {
    int q = c, sub = 0;
    if (a.cpp != 1) {
        q = (int)(__umulhi((uint32_t)c, a.cpp_magic) >> a.cpp_shift);
        sub = c - q * a.cpp;
    }
    int pid = bt[q];
    if (a.checks && (unsigned)pid >= (unsigned long long)a.num_pages) {
        debug_flag(a.err_word, PA_CHECK_PAGE);
        pid = 0;
    }
    return a.cpp == 1 ? pid : pid * a.vr + sub;
}

// The q_len a kernel uses for a sequence of seq_len sl: in the checked mode
// an invalid pair (q_len < 0 or > seq_len or > max_q_len, seq_len < 0, or
// more pages than the block-table row holds) is reported and the sequence
// skipped (q_len 0).  The result depends on (sl, ql) alone, so every kernel
// and every prefix sum over q_lens sees the same value.
PA_DEVINLINE int checked_q_len(const DecodeArgs& a, int sl, int ql) {
    if (!a.checks) return ql;
    if (ql < 0 || sl < 0 || ql > sl || ql > a.max_q_len) {
        debug_flag(a.err_word, PA_CHECK_LENGTHS);
        return 0;
    }
    if (ql > 0 && (sl - 1) / 16 >= a.bt_chunks) {
        debug_flag(a.err_word, PA_CHECK_TABLE);
        return 0;
    }
    return ql;
}

// ----------------------------------------------------------------- split plan

// Work items of one launch, computed identically by every workgroup from the
// device-resident lengths (no host round trip).  A sequence belongs to the
// launch if in_launch() says so.  Its visible pages are cut into splits of `pps` pages; an item is one
// (sequence, KV head, split).

// Per-sequence plan arrays live in dynamic LDS, sized from num_seqs by the
// host (plan_lds_bytes).
// The per-sequence arrays live in dynamic LDS; typed as LDS pointers so that
// accesses through them are LDS instructions, not generic (flat) ones.
typedef __attribute__((address_space(3))) int lds_int_t;
struct Plan {
    int pps;        // pages (or tiles) per split
    int n_items;
    int red[32];
    lds_int_t* item_base;  // [num_seqs + 1] items before sequence b; [num_seqs] = n_items
    lds_int_t* q_off;      // [num_seqs + 1] first query row of sequence b
    lds_int_t* seq_len;    // [num_seqs]
    lds_int_t* q_len;      // [num_seqs]
    lds_int_t* aux;        // [num_seqs] kernel-specific per-sequence value
};

inline __host__ __device__ size_t plan_lds_bytes(int num_seqs) { return (size_t)(5 * num_seqs + 2) * sizeof(int); }

PA_DEVINLINE void plan_bind(Plan& pl, int* dyn_generic, int num_seqs) {
    lds_int_t* dyn = (lds_int_t*)dyn_generic;   // the caller's extern __shared__ array
    pl.item_base = dyn;
    pl.q_off = dyn + (num_seqs + 1);
    pl.seq_len = dyn + 2 * (num_seqs + 1);
    pl.q_len = pl.seq_len + num_seqs;
    pl.aux = pl.q_len + num_seqs;
}

struct SeqInfo {
    int seq_len, q_len, q_off, lo, first_page, n_pages, splits;
};

PA_DEVINLINE SeqInfo seq_info(const Plan& pl, int b, int window, int page_size) {
    SeqInfo s;
    s.seq_len = pl.seq_len[b];
    s.q_len = pl.q_len[b];
    s.q_off = pl.q_off[b];
    s.lo = seq_visible_lo(s.seq_len, s.q_len, window);
    s.first_page = s.lo / page_size;
    s.n_pages = s.q_len > 0 ? (s.seq_len - 1) / page_size - s.first_page + 1 : 0;
    s.splits = (s.n_pages + pl.pps - 1) / pl.pps;
    return s;
}

// Block-wide exclusive scan of one int per thread, chunked over sequences.
// Returns this thread's exclusive prefix plus `carry`; *total gets the chunk sum.
PA_DEVINLINE int block_exclusive_scan(int v, int* red, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    const int inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) red[wid] = inc;
    __syncthreads();
    int off = 0, tot = 0;
    for (int w = 0; w < nwaves; ++w) {
        const int x = red[w];
        if (w < wid) off += x;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return off + inc - v;
}

// Which launch takes a sequence.  The VALU kernel takes sequences with at
// most cls_rows rows per KV head and at most cls_len visible keys; the tile
// kernel takes every other sequence.  cls_side selects the side (0: VALU).
PA_DEVINLINE bool in_launch(const DecodeArgs& a, int rows, int vis_len) {
    const bool valu = rows <= a.cls_rows && vis_len <= a.cls_len;
    return a.cls_side == 0 ? valu : !valu;
}

// Split plan of the paged split-KV kernel: a sequence belongs to the launch if
// in_launch() says so; its visible
// pages are cut into splits of `pps` pages; an item is one (sequence, KV head,
// split).  Computed identically by every workgroup from the device-resident
// lengths (no host round trip).  All threads of the block call.
PA_DEVINLINE void build_plan(Plan& pl, int* dyn, const DecodeArgs& a, const int32_t* seq_lens, const int32_t* q_lens,
                             int num_seqs, int window, int page_size, int group, int num_kv_heads,
                             int target_items, int min_pps, int forced_pps, int max_items) {
    plan_bind(pl, dyn, num_seqs);
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int nwaves = nthr / kWave;
    long long pages_total = 0;
    int max_np = 0;
    int carry_q = 0;
    for (int b0 = 0; b0 < num_seqs; b0 += nthr) {
        const int b = b0 + tid;
        int ql = 0, np = 0;
        if (b < num_seqs) {
            const int sl = seq_lens[b];
            ql = checked_q_len(a, sl, q_lens[b]);
            pl.seq_len[b] = sl;
            pl.q_len[b] = ql;
            const int rows = ql * group;
            const int lo = seq_visible_lo(sl, ql, window);
            if (ql > 0 && in_launch(a, rows, sl - lo)) np = (sl - 1) / page_size - lo / page_size + 1;
            pl.aux[b] = np;
        }
        int tot;
        const int ex = block_exclusive_scan(ql, pl.red, &tot);
        if (b < num_seqs) pl.q_off[b] = carry_q + ex;
        if (a.checks && b < num_seqs && ql > 0 && (int64_t)carry_q + ex + ql > a.num_tokens) {
            // rows past num_tokens: skipped (and so is every later sequence)
            debug_flag(a.err_word, PA_CHECK_TOKENS);
            pl.q_len[b] = 0;
            pl.aux[b] = 0;
            np = 0;
        }
        carry_q += tot;
        const int npw = (int)wave_sum_i64(np), npm = wave_max_i32(np);
        if (lane == 0) { pl.red[wid] = npw; pl.red[16 + wid] = npm; }
        __syncthreads();
        for (int w = 0; w < nwaves; ++w) { pages_total += pl.red[w]; max_np = max(max_np, pl.red[16 + w]); }
        __syncthreads();
    }
    pages_total *= num_kv_heads;
    int pps;
    if (forced_pps > 0) {
        pps = forced_pps;
    } else {
        const long long t = target_items > 0 ? target_items : 1;
        pps = (int)div_ceil_i64(pages_total, t);
        pps = max(pps, min_pps);
    }
    // at most kMaxSplits splits per (sequence, KV head)
    pps = max(pps, (max_np + kMaxSplits - 1) / kMaxSplits);
    // keep the item count within the workspace: items <= pages_total/pps + seqs*Hkv
    {
        long long cap = (long long)max_items - (long long)num_seqs * num_kv_heads;
        if (cap < 1) cap = 1;
        const long long need = div_ceil_i64(pages_total, cap);
        if (pps < need) pps = (int)need;
        if (pps < 1) pps = 1;
    }
    // whole pages per wave: round automatic split sizes up to a multiple of min_pps
    if (forced_pps <= 0 && min_pps > 1) pps = (pps + min_pps - 1) / min_pps * min_pps;
    int carry_i = 0;
    for (int b0 = 0; b0 < num_seqs; b0 += nthr) {
        const int b = b0 + tid;
        const int it = (b < num_seqs) ? ((pl.aux[b] + pps - 1) / pps) * num_kv_heads : 0;
        int tot;
        const int ex = block_exclusive_scan(it, pl.red, &tot);
        if (b < num_seqs) pl.item_base[b] = carry_i + ex;
        carry_i += tot;
    }
    if (tid == 0) {
        pl.item_base[num_seqs] = carry_i;
        pl.q_off[num_seqs] = carry_q;
        pl.n_items = carry_i;
        pl.pps = pps;
    }
    __syncthreads();
}

// Sequence owning item `it` (largest b with item_base[b] <= it).
PA_DEVINLINE int item_seq(const Plan& pl, int num_seqs, int it) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pl.item_base[mid] <= it) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace pa
