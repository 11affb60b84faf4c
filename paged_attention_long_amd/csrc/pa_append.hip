// Writing a step's new K/V rows into the paged cache (quantise-on-write for
// fp8 caches).  Sequence b's new rows are its last q_len_b positions
// (seq_len_b counts them), so row i lands at logical position
// p = seq_len_b - q_len_b + i: page block_table[b][p / P], slot p % P, the
// same addressing the attention kernels read with (kv_offset).  A 16-bit
// cache receives the input bits; an fp8 E4M3FN cache receives the code
// nearest to x / s (s the KV head's K or V scale, the quotient rounded once
// in fp32), ties to the even code, magnitudes from 448 up saturated to 448,
// NaN kept as NaN, sign kept.  An int8 cache receives, per row (one token
// of one KV head), the scale s = amax / 127 over the row's D values (fp32)
// and per element the integer nearest to x / s (one fp32 division, ties to
// even) within [-127, 127], a NaN quotient stored as 0; the scale goes to
// the row's place in the row-scale pool.  The pages quantise their own int8
// cache on write in the same place of the step ("Dual MI50, part 2",
// section "Prefill: teach the fork's fast kernel to read the int8 cache").
//
// One thread per 8 elements (16 B in, 16 B or 8 B out).  A workgroup takes
// four consecutive rows (tokens) of a sequence; its items run over the 8-element
// chunks of a head row fastest, then over the four rows, then over the head
// rows (K of every KV head, then V), so a wave stores one head row of four
// consecutive slots, adjacent in the page.  A row's page comes from the block
// table through a multiply-high by the host's magic number for page_size / 16;
// the quotient x / s by a multiply with 1/s where that provably gives the
// same code (else by the division itself), and the fp8 code by the hardware's
// round-to-nearest-even conversion (with one row per workgroup, a division and
// an integer rounding per element: 50.5 us for 64 sequences x 256 rows x 8
// heads x 128; this way 32.4 us).  Every store is checked against the
// cache and the block table; rows whose position or page falls outside them
// are skipped.
#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kAppendThreads = 256;

// E4M3FN codes of two fp32 values (byte 0: x, byte 1: y): the hardware
// conversion rounds to nearest, ties to even, at any magnitude below 448;
// the median clamps larger magnitudes and infinity to +-448 first (they
// saturate), and NaN becomes sign | 0x7f by select.
PA_DEVINLINE uint32_t e4m3_pair(float x, float y) {
    uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(x, -448.0f, 448.0f),
                                                          __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f), 0, false) &
                 0xffffu;
    if (x != x) v = (v & 0xff00u) | ((__float_as_uint(x) >> 24) & 0x80u) | 0x7fu;
    if (y != y) v = (v & 0x00ffu) | ((((__float_as_uint(y) >> 24) & 0x80u) | 0x7fu) << 8);
    return v;
}

// x * fl(1/s) lies within 2.5 units in the last place of fl(x / s) when s
// and 1/s are normal, so their codes can differ only where a point half-way
// between two codes is that close: for magnitudes from 2^-6 up (normal codes)
// where the 20 bits below the kept mantissa are within 3 of 0x80000.  Such
// values, and smaller magnitudes (subnormal codes, zero), take the quotient.
PA_DEVINLINE bool e4m3_needs_quotient(float q) {
    const uint32_t a = __float_as_uint(q) & 0x7fffffffu;
    return a < 0x3c800000u || ((a & 0xfffffu) - 0x7fffdu) <= 6u;
}

// Likewise for the nearest integer: within 3 ulp of a half-integer.
PA_DEVINLINE bool int_needs_quotient(float q) {
    const float d = fabsf(fabsf(q - __builtin_rintf(q)) - 0.5f);
    const int eb = (int)(__float_as_uint(q) & 0x7f800000u) - (23 << 23);
    return d <= 3.0f * __uint_as_float((uint32_t)max(eb, 0));
}

// A normal, finite fp32 value (exponent field 1 .. 254).
PA_DEVINLINE bool f32_normal(float v) { return (__float_as_uint(v) & 0x7f800000u) - 0x00800000u < 0x7f000000u; }

// Maximum over the aligned group of N lanes (N = 8 or 16: one row's
// threads) that propagates NaN, through DPP moves inside 16-lane rows.
template <int N>
PA_DEVINLINE float group_max_nan(float x) {
    auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
    x = mx(x, dpp<kDppQuadXor1>(x));
    x = mx(x, dpp<kDppQuadXor2>(x));
    x = mx(x, dpp<kDppHalfMirror>(x));
    if constexpr (N >= 16) x = mx(x, dpp<kDppRowMirror>(x));
    if constexpr (N == 32) {
        const uint32_t u = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        x = mx(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}

// int8 code of the fp32 quotient q: nearest integer, ties to even, within
// [-127, 127]; NaN to 0.
PA_DEVINLINE uint32_t i8_code(float q) {
    if (q != q) return 0u;
    const float r = __builtin_rintf(fminf(fmaxf(q, -127.0f), 127.0f));
    return (uint32_t)((int)r & 0xff);
}

template <int IT>
PA_DEVINLINE float to_f32(uint32_t bits16) {
    if constexpr (IT == PA_DTYPE_BF16) return __uint_as_float(bits16 << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <int KVT, int IT, int CPR = 16>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
    const int b = blockIdx.x;
    __shared__ int red[kAppendThreads / kWave];
    // this sequence's first input row: sum of the earlier q_lens
    int part = 0;
    for (int s = threadIdx.x; s < b; s += kAppendThreads) part += max(a.q_lens[s], 0);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = part;
    __syncthreads();
    int q_off = 0;
#pragma unroll
    for (int w = 0; w < kAppendThreads / kWave; ++w) q_off += red[w];
    const int ql = a.q_lens[b], sl = a.seq_lens[b];
    if (ql <= 0 || ql > sl || q_off + ql > a.num_tokens) {
        if (a.checks && threadIdx.x == 0 && blockIdx.y == 0 && ql != 0)
            debug_flag(a.err_word, (ql < 0 || ql > sl) ? PA_CHECK_LENGTHS : PA_CHECK_TOKENS);
        return;
    }
    // 8-element chunks per head row (a power of two); an int8 row's CPR
    // threads are one aligned lane group (chunk indices start at the thread
    // index and step by the workgroup size) and share the row's page
    const int cpr = KVT == PA_DTYPE_INT8 ? CPR : a.head_dim / 8;
    const int lcpr = 31 - __builtin_clz(cpr);
    const int per_row = 2 * a.num_kv_heads * cpr;
    const int64_t row_elems = (int64_t)a.num_kv_heads * a.head_dim;
    // row i's page id (-1: outside the block table, -2: a page id outside
    // the pool; both skipped, and reported in the checked mode) and slot
    auto row_page = [&](int i, int& pid, int& slot) {
        const int p = sl - ql + i;
        // p / page_size as (p / 16) / (page_size / 16) by the host's magic number
        const int lp = a.cpp == 1 ? p >> 4
                       : p < (1 << 28) ? (int)(__umulhi((uint32_t)(p >> 4), a.cpp_magic) >> a.cpp_shift)
                                       : p / a.page_size;
        slot = p - lp * a.page_size;
        pid = -1;
        if (lp < a.bt_stride) {
            pid = a.block_table[(int64_t)b * a.bt_stride + lp];
            if (pid < 0 || pid >= a.num_pages) pid = -2;
        }
    };
    auto chunk_src = [&](int i, int cw) {
        const int ch = cw & (cpr - 1);
        const int hw = cw >> lcpr;
        const int which = hw >= a.num_kv_heads;
        const int g = hw - which * a.num_kv_heads;
        return static_cast<const uint16_t*>(which ? a.v_new : a.k_new) + (int64_t)(q_off + i) * row_elems +
               (int64_t)g * a.head_dim + ch * 8;
    };
    // converts and stores chunk cw (16 input bytes in `in`) of a row at page pid, slot slot
    auto put = [&](int cw, const uint4& in, int pid, int slot) {
        const int ch = cw & (cpr - 1);
        const int hw = cw >> lcpr;
        const int which = hw >= a.num_kv_heads;                     // 0: K, 1: V
        const int g = hw - which * a.num_kv_heads;
        const int64_t off = (int64_t)pid * a.page_stride + (int64_t)g * a.head_stride +
                            (int64_t)slot * a.token_stride + ch * 8;
        if constexpr (KVT == PA_DTYPE_INT8) {
            const uint32_t w[4] = {in.x, in.y, in.z, in.w};
            float x[8];
            float amax = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                x[k] = to_f32<IT>((w[k / 2] >> (16 * (k & 1))) & 0xffffu);
                amax = __builtin_elementwise_maximum(amax, fabsf(x[k]));
            }
            amax = group_max_nan<CPR>(amax);
            const float s = __fdiv_rn(amax, 127.0f);
            const float rs = __fdiv_rn(1.0f, s);
            const bool fast = f32_normal(s) && f32_normal(rs);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float q = x[k] * rs;
                if (!fast || int_needs_quotient(q)) q = __fdiv_rn(x[k], s);
                const uint32_t code = i8_code(q);
                if (k < 4) lo |= code << (8 * k);
                else hi |= code << (8 * (k - 4));
            }
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(which ? a.v_cache : a.k_cache) + off) = make_uint2(lo, hi);
            if (ch == 0)
                a.row_scale[which * a.rs_v + (int64_t)pid * a.rs_page + (int64_t)g * a.rs_head +
                            (int64_t)slot * a.rs_tok] = s;
        } else if constexpr (KVT != PA_DTYPE_FP8_E4M3) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(which ? a.v_cache : a.k_cache) + off) = in;
        } else {
            const float s = a.kv_scale[which * a.num_kv_heads + g];
            const float rs = __fdiv_rn(1.0f, s);
            const bool fast = f32_normal(s) && f32_normal(rs);
            const uint32_t w[4] = {in.x, in.y, in.z, in.w};
            float q[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float x = to_f32<IT>((w[k / 2] >> (16 * (k & 1))) & 0xffffu);
                q[k] = x * rs;
                if (!fast || e4m3_needs_quotient(q[k])) q[k] = __fdiv_rn(x, s);
            }
            const uint32_t lo = e4m3_pair(q[0], q[1]) | (e4m3_pair(q[2], q[3]) << 16);
            const uint32_t hi = e4m3_pair(q[4], q[5]) | (e4m3_pair(q[6], q[7]) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(which ? a.v_cache : a.k_cache) + off) = make_uint2(lo, hi);
        }
    };
    auto report = [&](int pid) {
        if (a.checks) debug_flag(a.err_word, pid == -1 ? PA_CHECK_TABLE : PA_CHECK_PAGE);
    };
    // A workgroup takes kRows consecutive rows.  Items run chunk fastest,
    // then row, then head row, so the kRows rows of one head row that a wave
    // stores (consecutive slots of a page) are adjacent in the cache.
    constexpr int kRows = 4;
    const int i0 = blockIdx.y * kRows;
    if (i0 >= ql) return;
    const int n_items = per_row * kRows;
    for (int it = threadIdx.x; it < n_items; it += kAppendThreads) {
        const int ch = it & (cpr - 1);
        const int r = (it >> lcpr) & (kRows - 1);
        const int hw = it >> (lcpr + 2);
        const int i = i0 + r;
        if (i >= ql) continue;
        int pid, slot;
        row_page(i, pid, slot);
        const int cw = (hw << lcpr) | ch;
        if (pid < 0) {
            if (cw == 0) report(pid);
            continue;
        }
        put(cw, *reinterpret_cast<const uint4*>(chunk_src(i, cw)), pid, slot);
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int kv_dtype, int in_dtype, int max_rows, hipStream_t stream) {
    // workgroups along a sequence's rows, four rows each
    const dim3 grid(a.num_seqs, (std::max(max_rows, 1) + 3) / 4);
    if (kv_dtype == PA_DTYPE_INT8) {
        const bool bf = in_dtype == PA_DTYPE_BF16;
        if (a.head_dim == 256) {
            if (bf) hipLaunchKernelGGL((append_kernel<PA_DTYPE_INT8, PA_DTYPE_BF16, 32>), grid, dim3(kAppendThreads), 0, stream, a);
            else hipLaunchKernelGGL((append_kernel<PA_DTYPE_INT8, PA_DTYPE_F16, 32>), grid, dim3(kAppendThreads), 0, stream, a);
        } else if (a.head_dim == 128) {
            if (bf) hipLaunchKernelGGL((append_kernel<PA_DTYPE_INT8, PA_DTYPE_BF16, 16>), grid, dim3(kAppendThreads), 0, stream, a);
            else hipLaunchKernelGGL((append_kernel<PA_DTYPE_INT8, PA_DTYPE_F16, 16>), grid, dim3(kAppendThreads), 0, stream, a);
        } else {
            if (bf) hipLaunchKernelGGL((append_kernel<PA_DTYPE_INT8, PA_DTYPE_BF16, 8>), grid, dim3(kAppendThreads), 0, stream, a);
            else hipLaunchKernelGGL((append_kernel<PA_DTYPE_INT8, PA_DTYPE_F16, 8>), grid, dim3(kAppendThreads), 0, stream, a);
        }
    } else if (kv_dtype == PA_DTYPE_FP8_E4M3) {
        if (in_dtype == PA_DTYPE_BF16)
            hipLaunchKernelGGL((append_kernel<PA_DTYPE_FP8_E4M3, PA_DTYPE_BF16>), grid, dim3(kAppendThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((append_kernel<PA_DTYPE_FP8_E4M3, PA_DTYPE_F16>), grid, dim3(kAppendThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL((append_kernel<PA_DTYPE_F16, PA_DTYPE_F16>), grid, dim3(kAppendThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace pa
