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
// Bandwidth-bound and tiny per row: one thread per 8 elements (16 B in,
// 16 B or 8 B out), workgroups along the sequence's rows.  Every store is
// checked against the cache and the block table; rows whose position or page
// falls outside them are skipped.
#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kAppendThreads = 256;

// E4M3FN code of an fp32 value by integer rounding of its bits: the
// mantissa is cut to 3 bits (exponent >= -6) or the significand is shifted
// to units of 2^-9 (subnormal codes), rounding to nearest, ties to even.
// Codes are ordered like the values they stand for, so a round-up that
// carries into the exponent lands on the next code.
PA_DEVINLINE uint32_t e4m3_code(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;         // >= 448 (and infinity): saturate
    if (a < 0x00800000u) return sign;                  // zero and fp32 subnormals (< 2^-126)
    const int e = (int)(a >> 23) - 127;
    uint32_t code;
    if (e >= -6) {
        const uint32_t m = a & 0x7fffffu;
        const uint32_t base = ((uint32_t)(e + 7) << 3) | (m >> 20);
        const uint32_t rem = m & 0xfffffu;
        code = base + ((rem > 0x80000u || (rem == 0x80000u && (base & 1u))) ? 1u : 0u);
    } else {
        const int sh = 14 - e;                         // significand in units of 2^-9
        if (sh >= 32) return sign;
        const uint32_t sig = (a & 0x7fffffu) | 0x800000u;
        const uint32_t base = sig >> sh;
        const uint32_t rem = sig & ((1u << sh) - 1u);
        const uint32_t half = 1u << (sh - 1);
        code = base + ((rem > half || (rem == half && (base & 1u))) ? 1u : 0u);
    }
    return sign | min(code, 0x7eu);
}

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
    // 8-element chunks per head row; an int8 row's CPR threads are one aligned
    // lane group (the loop's start and stride are multiples of CPR)
    const int cpr = KVT == PA_DTYPE_INT8 ? CPR : a.head_dim / 8;
    const int64_t per_side = (int64_t)ql * a.num_kv_heads * cpr;
    const int64_t stride = (int64_t)gridDim.y * kAppendThreads;
    for (int64_t c = (int64_t)blockIdx.y * kAppendThreads + threadIdx.x; c < 2 * per_side; c += stride) {
        const int which = c >= per_side;                           // 0: K, 1: V
        const int64_t r = c - which * per_side;
        const int ch = (int)(r % cpr);
        const int64_t rg = r / cpr;
        const int g = (int)(rg % a.num_kv_heads);
        const int i = (int)(rg / a.num_kv_heads);
        const int p = sl - ql + i;
        const int lp = p / a.page_size;
        // (an int8 row's threads share p and pid: they skip together)
        if (lp >= a.bt_stride) {
            if (a.checks) debug_flag(a.err_word, PA_CHECK_TABLE);
            continue;
        }
        const int pid = a.block_table[(int64_t)b * a.bt_stride + lp];
        if (pid < 0 || pid >= a.num_pages) {
            if (a.checks) debug_flag(a.err_word, PA_CHECK_PAGE);
            continue;
        }
        const uint16_t* src = static_cast<const uint16_t*>(which ? a.v_new : a.k_new) +
                              ((int64_t)(q_off + i) * a.num_kv_heads + g) * a.head_dim + ch * 8;
        const uint4 in = *reinterpret_cast<const uint4*>(src);
        const int64_t off = (int64_t)pid * a.page_stride + (int64_t)g * a.head_stride +
                            (int64_t)(p - lp * a.page_size) * a.token_stride + ch * 8;
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
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t code = i8_code(__fdiv_rn(x[k], s));
                if (k < 4) lo |= code << (8 * k);
                else hi |= code << (8 * (k - 4));
            }
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(which ? a.v_cache : a.k_cache) + off) = make_uint2(lo, hi);
            if (ch == 0)
                a.row_scale[which * a.rs_v + (int64_t)pid * a.rs_page + (int64_t)g * a.rs_head +
                            (int64_t)(p - lp * a.page_size) * a.rs_tok] = s;
        } else if constexpr (KVT != PA_DTYPE_FP8_E4M3) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(which ? a.v_cache : a.k_cache) + off) = in;
        } else {
            const float s = a.kv_scale[which * a.num_kv_heads + g];
            const uint32_t w[4] = {in.x, in.y, in.z, in.w};
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t bits = (w[k / 2] >> (16 * (k & 1))) & 0xffffu;
                const uint32_t code = e4m3_code(__fdiv_rn(to_f32<IT>(bits), s));
                if (k < 4) lo |= code << (8 * k);
                else hi |= code << (8 * (k - 4));
            }
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(which ? a.v_cache : a.k_cache) + off) = make_uint2(lo, hi);
        }
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int kv_dtype, int in_dtype, int max_rows, hipStream_t stream) {
    const int64_t chunks = 2LL * max_rows * a.num_kv_heads * (a.head_dim / 8);
    const int gy = (int)std::min<int64_t>(256, std::max<int64_t>(1, (chunks + kAppendThreads - 1) / kAppendThreads));
    const dim3 grid(a.num_seqs, gy);
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
