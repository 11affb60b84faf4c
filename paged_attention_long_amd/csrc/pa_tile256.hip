// Tile kernel on the matrix cores (gfx950 MFMA) for head_dim 256.
//
// Used for the row counts the VALU kernel does not take at this width (more
// than 64 query rows per KV head, i.e. chunked prefill).  The dense models of
// the pages' long-context prefill measurements have 256-wide heads
// ("Strix Halo dense cliff patch attribution", section "Which patch, and how
// I know").
//
// A work item is (sequence, KV head, block of 128 query rows, split of the
// key tiles).  Rows of one KV head are token-major (row = i*G + h), so the G
// query heads of consecutive new tokens share every K/V tile the item loads
// ("Dual MI50, part 2", section "Decode: a new kernel for the shape MTP
// actually runs"), and the big query block amortises each tile load ("Dual
// MI50, part 2", section "Prefill: teach the fork's fast kernel to read the
// int8 cache").  Four waves own 32 rows each.
//
// Per tile of 32 keys (two 16-token chunks gathered through the block table):
//   * every thread loads its share of the K and V rows two tiles ahead into
//     registers (16-byte loads, two register sets; one-byte caches are widened
//     exactly to 16 bits) while the current tile is computed, and writes the
//     next tile's rows into the other half of a two-tile LDS ring after it
//     (two tiles of compute hide the load latency, which one does not: 4.16
//     -> 3.97 ms on a 2,048-token chunk); rows are 512 B with their 16-byte
//     chunks XOR-swizzled by the row, so the operand reads below (one chunk
//     of many rows at once) spread over the banks;
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (A = 32 K rows, B = Q^T held in
//     registers, 16 steps over the head dim): each lane then holds 16 keys of
//     one query row;
//   * online softmax in fp32 against a lazily raised reference max (moved
//     only when a score passes it by 2^8); masked keys become -inf by select
//     and the V rows of dead keys are stored as zeros, so NaN in freed pages
//     never reaches a product;
//   * O^T += V^T P^T over eight 32-wide head-dim blocks; the V^T operands
//     come from the row-major V tile through the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16), gathered in the key order of P's packed pairs so
//     P stays where the score MFMA left it.  With 16-bit caches, while a row
//     has seen little weight, P's rounding to 16 bits is added back by a
//     second pass (hi/lo split of P).
// Splits are combined by the merge launch that follows (pa_merge.h).
#include "pa_common.h"
#include "pa_merge.h"
#include "pa_kernels.h"

#include <type_traits>

namespace pa {

namespace {

constexpr int kD = 256;
constexpr int kPage = 16;
constexpr int kNW = 4;                  // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kBM = 32 * kNW;           // query rows per item
constexpr int kBN = 32;                 // keys per tile
constexpr int kPPT = kBN / kPage;       // 16-token chunks per tile
constexpr int kKS = kD / 16;            // score steps over the head dim
constexpr int kDB = kD / 32;            // 32-wide head-dim blocks of O^T
constexpr int kRowBytes = kD * 2;       // one 16-bit K or V row in LDS
constexpr int kTile = kBN * kRowBytes;  // one K (or V) tile
constexpr float kTau = 8.0f;            // lazy max: rescale when a score passes the reference by 2^8
// P.V also runs on P's rounding error while a row's weight sum is below
// kSplitBelow times its largest weight.  Past that point the largest single
// weight is at most 1/kSplitBelow of the sum, so rounding it to 16 bits
// (relative 2^-9 for bf16) moves the output by at most 2^-9/8 |v| ~ 2.4e-4 |v|,
// and the other weights' rounding errors are independent of it.
constexpr float kSplitBelow = 8.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

template <int T>
PA_DEVINLINE f32x16_t mma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
    if constexpr (T == PA_DTYPE_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
}

template <int T>
PA_DEVINLINE uint32_t pack2(float x, float y) {
    if constexpr (T == PA_DTYPE_BF16) return f32x2_to_bf16x2(f32x2_t{x, y});
    else return f32x2_to_f16x2(f32x2_t{x, y});
}
template <int T>
PA_DEVINLINE float unpack_lo(uint32_t u) {
    if constexpr (T == PA_DTYPE_BF16) return bf16lo_to_f32(u);
    else return f16x2_to_f32(u).x;
}
template <int T>
PA_DEVINLINE float unpack_hi(uint32_t u) {
    if constexpr (T == PA_DTYPE_BF16) return bf16hi_to_f32(u);
    else return f16x2_to_f32(u).y;
}

// NaN-propagating maximum (IEEE maximum).
PA_DEVINLINE float fmax_nan(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// Eight one-byte cache codes (fp8 e4m3 or int8) to eight 16-bit values of
// type T, exactly (both 16-bit types hold every code's value).
template <int T, int KVT>
PA_DEVINLINE u32x4_t widen8(const u32x2_t& c) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if constexpr (KVT == PA_DTYPE_FP8_E4M3) {
            if constexpr (T == PA_DTYPE_BF16) {
                r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false));
                r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true));
            } else {
                r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.0f, false));
                r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.0f, true));
            }
        } else {
            uint32_t lo, hi;
            if constexpr (T == PA_DTYPE_BF16) i8x4_to_bf16x4(c[i], lo, hi);
            else i8x4_to_f16x4(c[i], lo, hi);
            r[2 * i] = lo;
            r[2 * i + 1] = hi;
        }
    }
    return r;
}

// Byte offset of 16-byte chunk c (0..31) of row r inside a tile.  The chunk's
// low four bits are XOR-ed with a key that puts the row's low two bits into
// the chunk's high two bits, so the 16 rows of a K operand read (one chunk
// each) and the 4 rows x 2 chunks of a transposing V read land in distinct
// banks (a 512-byte row spans the 64 banks twice).
PA_DEVINLINE int swz_key(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
PA_DEVINLINE int swz(int r, int c) { return r * kRowBytes + ((c ^ swz_key(r)) << 4); }

template <int KVT>
struct Elem {
    static constexpr bool BYTE = (KVT == PA_DTYPE_FP8_E4M3) || (KVT == PA_DTYPE_INT8);
    static constexpr int EB = BYTE ? 1 : 2;
    // 16-byte global loads per thread per K (or V) tile
    static constexpr int LOADS = kBN * kD * EB / 16 / kThreads;
    // 16-byte chunks per cached row
    static constexpr int CPR = kD * EB / 16;
};

template <int KVT, int QT>
__global__ __launch_bounds__(kThreads) void tile256_kernel(DecodeArgs a) {
    constexpr bool FP8 = (KVT == PA_DTYPE_FP8_E4M3);
    constexpr bool INT8 = (KVT == PA_DTYPE_INT8);
    constexpr bool BYTE = Elem<KVT>::BYTE;
    constexpr int EB = Elem<KVT>::EB;
    constexpr int NL = Elem<KVT>::LOADS;
    constexpr int CPR = Elem<KVT>::CPR;
    constexpr int PVT = BYTE ? PA_DTYPE_F16 : KVT;   // P.V operand type

    __shared__ Plan pl;
    extern __shared__ int dyn_lds[];
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[2][2][kTile];   // [ring slot][K, V]
    __shared__ __attribute__((aligned(16))) float tsc[2][2 * kBN];         // int8: [slot][K scales | V scales]
    __shared__ long long red_items[8][kNW];
    __shared__ int red_big[8][kNW];
    __shared__ long long redw[kNW], redq[kNW];
    __shared__ int redt[kNW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
    const int h32 = lane >> 5;
    const int l32 = lane & 31;

    // ---------------------------------------------------------------- plan
    // A sequence is in this launch if in_launch() says so.  Its rows form
    // ceil(rows / 128) row blocks; each row block's visible keys are cut into
    // 32-key tiles, grouped into `splits` splits (the same number for every
    // row block of the sequence).  Split sizes: of the candidates sized for
    // 1..4 rounds of the resident grid and four between the one-round lower
    // bound (work / t) and a size that surely fits one round (work / (t - row
    // blocks)), the one whose rounds x largest item is smallest, ties to the
    // fewer items.
    plan_bind(pl, dyn_lds, a.num_seqs);
    auto widest_tiles = [&](int sl, int ql) {
        const int rows = ql * a.group;
        const int nqt = (rows + kBM - 1) / kBM;
        int tub = 0;
        for (int q = max(0, nqt - 2); q < nqt; ++q) {
            const int r0 = q * kBM, r1 = min(rows, r0 + kBM) - 1;
            const int p0 = sl - ql + r0 / a.group, p1 = sl - ql + r1 / a.group;
            const int klo = a.window > 0 ? max(0, p0 - a.window + 1) : 0;
            const int pages = p1 / kPage - klo / kPage + 1;
            tub = max(tub, (pages + kPPT - 1) / kPPT);
        }
        return tub;
    };
    {
        long long work = 0, qtiles = 0;
        int max_tiles = 0, carry_q = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += kThreads) {
            const int b = b0 + tid;
            int ql = 0, nqt = 0, tub = 0;
            if (b < a.num_seqs) {
                const int sl = a.seq_lens[b];
                ql = checked_q_len(a, sl, a.q_lens[b]);
                pl.seq_len[b] = sl;
                pl.q_len[b] = ql;
                const int rows = ql * a.group;
                if (ql > 0 && in_launch(a, rows, sl - seq_visible_lo(sl, ql, a.window))) {
                    nqt = (rows + kBM - 1) / kBM;
                    tub = widest_tiles(sl, ql);
                }
            }
            int tot;
            const int ex = block_exclusive_scan(ql, pl.red, &tot);
            if (b < a.num_seqs) {
                pl.q_off[b] = carry_q + ex;
                if (a.checks && ql > 0 && (int64_t)carry_q + ex + ql > a.num_tokens) {
                    // rows past num_tokens: skipped (and so is every later sequence)
                    debug_flag(a.err_word, PA_CHECK_TOKENS);
                    pl.q_len[b] = 0;
                    nqt = 0;
                    tub = 0;
                }
                pl.aux[b] = tub;
                pl.item_base[b] = nqt;   // temporary
            }
            carry_q += tot;
            const long long w = wave_sum_i64((long long)nqt * tub), nq = wave_sum_i64(nqt);
            const int mt = wave_max_i32(tub);
            if (lane == 0) { redw[wid] = w; redq[wid] = nq; redt[wid] = mt; }
            __syncthreads();
            for (int ww = 0; ww < kNW; ++ww) {
                work += redw[ww];
                qtiles += redq[ww];
                max_tiles = max(max_tiles, redt[ww]);
            }
            __syncthreads();
        }
        work *= a.num_kv_heads;
        qtiles *= a.num_kv_heads;
        // lower bounds on tiles per split: at most kMaxSplits splits, items
        // within the partial workspace
        int tmin = max(1, (max_tiles + kMaxSplits - 1) / kMaxSplits);
        {
            long long cap = (long long)a.max_items - qtiles;
            if (cap < 1) cap = 1;
            tmin = max(tmin, (int)div_ceil_i64(work, cap));
        }
        int tps = tmin;
        if (a.forced_pps > 0) {
            tps = max(a.forced_pps, tmin);
        } else {
            const long long t = a.target_items > 0 ? a.target_items : 1;
            constexpr int NC = 8;
            const long long c_lo = max((long long)tmin, div_ceil_i64(work, t));
            const long long c_hi = min((long long)1 << 30, t > qtiles ? max(c_lo, div_ceil_i64(work, t - qtiles)) : c_lo);
            int cand[NC];
            long long items[NC];
            int big[NC];
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                cand[k] = k < 4 ? max(tmin, (int)div_ceil_i64(work, t * (k + 1))) : (int)(c_lo + (c_hi - c_lo) * (k - 3) / 4);
                items[k] = 0;
                big[k] = 0;
            }
            for (int b = tid; b < a.num_seqs; b += kThreads) {
                const int tub = pl.aux[b];
                if (tub > 0) {
#pragma unroll
                    for (int k = 0; k < NC; ++k) {
                        const int S = (tub + cand[k] - 1) / cand[k];
                        items[k] += (long long)pl.item_base[b] * S;
                        big[k] = max(big[k], (tub + S - 1) / S);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                const long long it_w = wave_sum_i64(items[k]);
                const int big_w = wave_max_i32(big[k]);
                if (lane == 0) { red_items[k][wid] = it_w; red_big[k][wid] = big_w; }
            }
            __syncthreads();
            long long best = -1, best_items = 0;
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                long long it_k = 0;
                int big_k = 0;
                for (int ww = 0; ww < kNW; ++ww) {
                    it_k += red_items[k][ww];
                    big_k = max(big_k, red_big[k][ww]);
                }
                const long long cost = div_ceil_i64(it_k * a.num_kv_heads, t) * big_k;
                if (best < 0 || cost < best || (cost == best && it_k < best_items)) {
                    best = cost;
                    best_items = it_k;
                    tps = cand[k];
                }
            }
        }
        int carry_i = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += kThreads) {
            const int b = b0 + tid;
            int it = 0;
            if (b < a.num_seqs) {
                const int S = (pl.aux[b] + tps - 1) / tps;
                it = pl.item_base[b] * a.num_kv_heads * S;
                pl.aux[b] = S;
            }
            int tot;
            const int ex = block_exclusive_scan(it, pl.red, &tot);
            if (b < a.num_seqs) pl.item_base[b] = carry_i + ex;
            carry_i += tot;
        }
        if (tid == 0) {
            pl.item_base[a.num_seqs] = carry_i;
            pl.q_off[a.num_seqs] = carry_q;
            pl.n_items = carry_i;
            pl.pps = tps;
        }
        __syncthreads();
    }
    const int n_items = pl.n_items;

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
    const int64_t page_bytes = a.page_stride * EB;
    const int64_t tok_bytes = a.token_stride * EB;

    // Transposing V reads (P.V operand; d = db*32 + l32, keys 4h32 .. +3 and
    // 8 + 4h32 .. +3 of a 16-key step): within each 16-lane group, source lane
    // s reads tile row 4h32 + s/4 (+8) at columns cq*16 + 4(s%4) .. +3 of
    // head-dim block db, and lane j of the group receives the 4 keys of column
    // cq*16 + j.  Byte offsets for step 0; step ts adds 16 rows (same swizzle key).
    uint32_t v_lane_off[2 * kDB];
    {
        const int s16 = lane & 15, cq = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int col = db * 32 + cq * 16 + 4 * (s16 & 3);
                const int row = 4 * h32 + (s16 >> 2) + 8 * hh;
                v_lane_off[2 * db + hh] = (uint32_t)(swz(row, col >> 3) + (col & 7) * 2);
            }
    }

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        // ------------------------------------------------------------ item geometry (uniform)
        const int b = __builtin_amdgcn_readfirstlane(item_seq(pl, a.num_seqs, it));
        const int seq_len = __builtin_amdgcn_readfirstlane(pl.seq_len[b]);
        const int q_len = __builtin_amdgcn_readfirstlane(pl.q_len[b]);
        const int q_off = __builtin_amdgcn_readfirstlane(pl.q_off[b]);
        const int S = __builtin_amdgcn_readfirstlane(pl.aux[b]);
        const int lo = seq_visible_lo(seq_len, q_len, a.window);
        const int local = it - __builtin_amdgcn_readfirstlane(pl.item_base[b]);
        const int per_qt = a.num_kv_heads * S;
        const int qt = local / per_qt;
        const int rem = local - qt * per_qt;
        const int g = rem / S;
        const int split = rem - g * S;
        const int rows_all = q_len * a.group;
        const int row0 = qt * kBM;
        const int rows = min(kBM, rows_all - row0);
        const int pos_first = seq_len - q_len + row0 / a.group;
        const int pos_last = seq_len - q_len + (row0 + rows - 1) / a.group;
        const int klo = a.window > 0 ? max(0, pos_first - a.window + 1) : 0;
        const int pg_first = klo / kPage;
        const int pg_end = pos_last / kPage + 1;
        const int n_tiles = (pg_end - pg_first + kPPT - 1) / kPPT;
        const int tpsb = (widest_tiles(seq_len, q_len) + S - 1) / S;
        const int t_begin = min(n_tiles, split * tpsb);
        const int t_end = min(n_tiles, t_begin + tpsb);
        const float kscale = FP8 ? a.kv_scale[g] : 1.0f;
        const float vscale = FP8 ? a.kv_scale[a.num_kv_heads + g] : 1.0f;
        const float s2 = a.scale * kLog2e * kscale;
        const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
        const bool direct = (S == 1);
        const int64_t head_off = (int64_t)g * a.head_stride * EB;

        // ------------------------------------------------------------ this lane's query row
        const int row_l = wid * 32 + l32;
        const int row_g = row0 + row_l;
        const bool row_ok = row_l < rows;
        const int tok_i = row_ok ? row_g / a.group : 0;
        const int pos_r = row_ok ? seq_len - q_len + tok_i : -1;
        const int lo_r = (a.window > 0) ? pos_r - a.window + 1 : 0;
        // the wave's rows: a tile inside every row's visible range needs no mask
        const int w_row0 = row0 + wid * 32;
        const int w_rows = max(0, min(32, rows - wid * 32));
        const int w_pmin = seq_len - q_len + w_row0 / a.group;
        const int w_pmax = seq_len - q_len + (w_row0 + max(w_rows, 1) - 1) / a.group;
        const int w_lomax = (a.window > 0) ? w_pmax - a.window + 1 : 0;

        u32x4_t qreg[kKS];
        {
            const int h = g * a.group + (row_ok ? row_g - tok_i * a.group : 0);
            const uint16_t* qp = qbase + ((int64_t)(q_off + tok_i) * a.num_q_heads + h) * kD + 8 * h32;
#pragma unroll
            for (int s = 0; s < kKS; ++s) {
                if (row_ok) qreg[s] = load_b128_cached(qp + 16 * s);
                else { qreg[s][0] = 0; qreg[s][1] = 0; qreg[s][2] = 0; qreg[s][3] = 0; }
            }
        }

        f32x16_t o_acc[kDB];
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o_acc[db][i] = 0.f;
        float m_run = kNegInf, m_true = kNegInf, l_exact = 0.f;
        float neg_m = 0.f, split_thr = kSplitBelow;

        // ------------------------------------------------------------ tile staging
        // Tile t covers 16-token chunks pg_first + t*2 and + 1; a chunk past
        // the visible range reads the last visible one (in bounds) and its
        // keys are dead.  Key k of a tile is live iff it lies in [lo, seq_len).
        auto key_pos = [&](int t, int key) { return (pg_first + t * kPPT) * kPage + key; };
        auto key_live = [&](int t, int key) {
            const int j = key_pos(t, key);
            return (j >= lo) && (j < seq_len) && (pg_first + t * kPPT + key / kPage < pg_end);
        };
        using Raw = u32x4_t;
        Raw kr[2][NL], vr[2][NL];
        float fsc[2] = {0.f, 0.f};
        auto tile_load = [&](int t, auto b_c) {
            constexpr int B = decltype(b_c)::value;
            int pid[kPPT];
#pragma unroll
            for (int p = 0; p < kPPT; ++p)
                pid[p] = chunk_page(bt, __builtin_amdgcn_readfirstlane(min(pg_first + t * kPPT + p, pg_end - 1)), a);
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int idx = i * kThreads + tid;
                const int key = idx / CPR, c = idx % CPR;
                const int64_t off = (int64_t)pid[key / kPage] * page_bytes + head_off + (int64_t)(key % kPage) * tok_bytes +
                                    c * 16;
                kr[B][i] = load_b128(kbase + off);
                vr[B][i] = load_b128(vbase + off);
            }
            if constexpr (INT8) {
                if (tid < 2 * kBN) {
                    const int key = tid % kBN;
                    const int p = pid[key / kPage];
                    fsc[B] = __builtin_nontemporal_load(a.row_scale + (int64_t)p * a.rs_page + (int64_t)g * a.rs_head +
                                                     (int64_t)(key % kPage) * a.rs_tok + (tid >= kBN ? a.rs_v : 0));
                }
            }
        };
        auto tile_store = [&](int slot, int t, auto b_c) {
            constexpr int B = decltype(b_c)::value;
            uint8_t* kt = tiles[slot][0];
            uint8_t* vt = tiles[slot][1];
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int idx = i * kThreads + tid;
                const int key = idx / CPR, c = idx % CPR;
                const bool live = key_live(t, key);
                if constexpr (BYTE) {
                    // 16 codes -> two 16-byte chunks of 16-bit values
                    const u32x2_t k0{kr[B][i][0], kr[B][i][1]}, k1{kr[B][i][2], kr[B][i][3]};
                    const u32x2_t v0{vr[B][i][0], vr[B][i][1]}, v1{vr[B][i][2], vr[B][i][3]};
                    *reinterpret_cast<u32x4_t*>(kt + swz(key, 2 * c)) = widen8<QT, KVT>(k0);
                    *reinterpret_cast<u32x4_t*>(kt + swz(key, 2 * c + 1)) = widen8<QT, KVT>(k1);
                    const u32x4_t z{0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4_t*>(vt + swz(key, 2 * c)) = live ? widen8<PVT, KVT>(v0) : z;
                    *reinterpret_cast<u32x4_t*>(vt + swz(key, 2 * c + 1)) = live ? widen8<PVT, KVT>(v1) : z;
                } else {
                    *reinterpret_cast<u32x4_t*>(kt + swz(key, c)) = kr[B][i];
                    *reinterpret_cast<u32x4_t*>(vt + swz(key, c)) = live ? vr[B][i] : u32x4_t{0u, 0u, 0u, 0u};
                }
            }
            if constexpr (INT8) {
                // a dead key's V scale (maybe NaN) is stored as 0
                if (tid < 2 * kBN) tsc[slot][tid] = (tid >= kBN && !key_live(t, tid - kBN)) ? 0.f : fsc[B];
            }
        };

        // ------------------------------------------------------------ one tile
        auto compute_tile = [&](int t, int slot) {
            const uint8_t* kt = tiles[slot][0];
            const uint32_t vt32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)tiles[slot][1];
            // S^T = K Q^T over the 16 head-dim steps
            f32x16_t sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
            for (int s0 = 0; s0 < kKS; s0 += 8) {
                u32x4_t kf[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const u32x4_t*>(kt + swz(l32, 2 * (s0 + s) + h32));
#pragma unroll
                for (int s = 0; s < 8; ++s) sacc = mma32<QT>(kf[s], qreg[s0 + s], sacc);
            }
            // score i of this lane is key 8*(i/4) + 4*h32 + i%4 of the tile
            float vs[16];
            if constexpr (INT8) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 kk = *reinterpret_cast<const float4*>(&tsc[slot][8 * q + 4 * h32]);
                    const float4 vv = *reinterpret_cast<const float4*>(&tsc[slot][kBN + 8 * q + 4 * h32]);
                    sacc[4 * q] *= kk.x; sacc[4 * q + 1] *= kk.y; sacc[4 * q + 2] *= kk.z; sacc[4 * q + 3] *= kk.w;
                    vs[4 * q] = vv.x; vs[4 * q + 1] = vv.y; vs[4 * q + 2] = vv.z; vs[4 * q + 3] = vv.w;
                }
            }
            const int key0 = key_pos(t, 0);
            const bool full = (key0 >= w_lomax) && (key0 + kBN - 1 <= w_pmin) && (key0 >= lo) &&
                              (key0 + kBN <= seq_len) && (pg_first + (t + 1) * kPPT <= pg_end);
            if (!full) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = key0 + 8 * (i / 4) + 4 * h32 + (i % 4);
                    const bool vis = (j <= pos_r) && (j >= lo_r) && (j >= lo) && (j < seq_len);
                    sacc[i] = vis ? sacc[i] : kNegInf;
                }
            }
            // tile max of the row (the other 16 keys are in lane l ^ 32); lazy rescale
            float tmax = kNegInf;
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmax_nan(tmax, sacc[i]);
            {
                const f32x2_t p = xor_pair<32>(tmax);
                tmax = fmax_nan(p.x, p.y) * s2;
            }
            if (wave_any(tmax > m_true)) {
                m_true = fmax_nan(m_true, tmax);
                if (wave_any(tmax > m_run + kTau)) {
                    const float mn = m_true;
                    const float al = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - mn);
                    m_run = mn;
                    neg_m = (m_run == kNegInf) ? 0.f : -m_run;
                    l_exact *= al;
#pragma unroll
                    for (int db = 0; db < kDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) o_acc[db][i] *= al;
                }
                split_thr = kSplitBelow * ((m_run == kNegInf) ? 1.f : fast_exp2(m_true - m_run));
            }
            // P, packed as the B operand of two 16-key steps: step ts holds
            // scores 8ts .. 8ts+7 of this lane
            u32x4_t pb[2], plo[2];
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float p0 = fast_exp2(fmaf(sacc[i], s2, neg_m));
                const float p1 = fast_exp2(fmaf(sacc[i + 1], s2, neg_m));
                sacc[i] = p0;
                sacc[i + 1] = p1;
                l_exact += p0 + p1;
                if constexpr (INT8) pb[i / 8][(i % 8) / 2] = pack2<PVT>(p0 * vs[i], p1 * vs[i + 1]);
                else pb[i / 8][(i % 8) / 2] = pack2<PVT>(p0, p1);
            }
            // 16-bit caches: add P's rounding error back while the row's weight
            // sum is small against its largest weight (one-byte caches carry a
            // far larger error of their own)
            const bool split_p = !BYTE && wave_any(l_exact < split_thr);
            if (split_p) {
#pragma unroll
                for (int i = 0; i < 16; i += 2)
                    plo[i / 8][(i % 8) / 2] = pack2<PVT>(sacc[i] - unpack_lo<PVT>(pb[i / 8][(i % 8) / 2]),
                                                         sacc[i + 1] - unpack_hi<PVT>(pb[i / 8][(i % 8) / 2]));
            }
            // O^T += V^T P^T
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) {
                i16x4_t vf[2 * kDB];
#pragma unroll
                for (int k = 0; k < 2 * kDB; ++k)
                    vf[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4_t*)(uintptr_t)(vt32 + v_lane_off[k] + ts * 16 * kRowBytes));
#pragma unroll
                for (int db = 0; db < kDB; ++db) {
                    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, vf[2 * db]);
                    const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, vf[2 * db + 1]);
                    const u32x4_t va{lo2[0], lo2[1], hi2[0], hi2[1]};
                    o_acc[db] = mma32<PVT>(va, pb[ts], o_acc[db]);
                    if (split_p) o_acc[db] = mma32<PVT>(va, plo[ts], o_acc[db]);
                }
            }
        };

        if (t_begin < t_end) {
            using B0 = std::integral_constant<int, 0>;
            using B1 = std::integral_constant<int, 1>;
            tile_load(t_begin, B0{});
            if (t_begin + 1 < t_end) tile_load(t_begin + 1, B1{});
            tile_store(0, t_begin, B0{});
            __syncthreads();
            for (int t = t_begin; t < t_end; t += 2) {
                if (t + 2 < t_end) tile_load(t + 2, B0{});
                compute_tile(t, 0);
                if (t + 1 < t_end) tile_store(1, t + 1, B1{});
                __syncthreads();
                if (t + 1 >= t_end) break;
                if (t + 3 < t_end) tile_load(t + 3, B1{});
                compute_tile(t + 1, 1);
                if (t + 2 < t_end) tile_store(0, t + 2, B0{});
                __syncthreads();
            }
        }

        // ------------------------------------------------------------ finish the rows
        float LE;
        {
            const f32x2_t p = xor_pair<32>(l_exact);
            LE = p.x + p.y;
        }
        if (row_ok) {
            const float inv = (LE > 0.f) ? 1.0f / LE : 0.f;
            float* op;
            float sc;
            MergeTarget tgt{a.out, a.lse, a.num_q_heads, a.group, vscale};
            if (direct) {
                const int64_t orow = out_row(tgt, q_off, g, row_g);
                op = a.out + orow * kD;
                sc = inv * vscale;
                if (a.lse != nullptr && h32 == 0) a.lse[orow] = (LE > 0.f) ? (m_run + fast_log2(LE)) * kLn2 : kNegInf;
            } else {
                const int64_t slot = (int64_t)(it + a.item_off) * kBM + row_l;
                op = a.ws_o + slot * kD;
                sc = inv;
                if (h32 == 0) a.ws_lse[slot] = (LE > 0.f) ? m_run + fast_log2(LE) : kNegInf;
            }
            // O^T element i of block db is head-dim db*32 + 8*(i/4) + 4*h32 + i%4
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<float4*>(op + db * 32 + 8 * q + 4 * h32) =
                        make_float4(o_acc[db][4 * q] * sc, o_acc[db][4 * q + 1] * sc, o_acc[db][4 * q + 2] * sc,
                                    o_acc[db][4 * q + 3] * sc);
        }
        if (!direct && split == 0 && tid == 0)
            publish_merge(a, MergeDesc{it + a.item_off, S, rows, kBM, q_off, g, row0, vscale});
        __syncthreads();
    }
}

template <int KVT, int QT>
hipError_t launch_t(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((tile256_kernel<KVT, QT>), dim3(grid), dim3(kThreads), plan_lds_bytes(a.num_seqs), st, a);
    return hipGetLastError();
}

template <int KVT, int QT>
int blocks_t(size_t dyn) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, tile256_kernel<KVT, QT>, kThreads, dyn);
    return (e == hipSuccess && n > 0) ? n : 1;
}

// f(kvt, qt) with the kernel's template arguments as integral constants.
template <typename F>
bool with_tile256(int kv_dtype, int q_dtype, F&& f) {
    using I = std::integral_constant<int, PA_DTYPE_INT8>;
    using E = std::integral_constant<int, PA_DTYPE_FP8_E4M3>;
    using H = std::integral_constant<int, PA_DTYPE_F16>;
    using B = std::integral_constant<int, PA_DTYPE_BF16>;
    const bool bq = q_dtype == PA_DTYPE_BF16;
    switch (kv_dtype) {
        case PA_DTYPE_F16: return f(H{}, H{}), true;
        case PA_DTYPE_BF16: return f(B{}, B{}), true;
        case PA_DTYPE_FP8_E4M3: return bq ? (f(E{}, B{}), true) : (f(E{}, H{}), true);
        case PA_DTYPE_INT8: return bq ? (f(I{}, B{}), true) : (f(I{}, H{}), true);
        default: return false;
    }
}

}  // namespace

int tile256_rows_per_item() { return kBM; }

int tile256_blocks_per_cu(int kv_dtype, int q_dtype, int max_num_seqs) {
    int n = 1;
    with_tile256(kv_dtype, q_dtype, [&](auto kvt, auto qt) {
        n = blocks_t<decltype(kvt)::value, decltype(qt)::value>(plan_lds_bytes(max_num_seqs));
    });
    return n;
}

hipError_t launch_tile256(const DecodeArgs& a, int kv_dtype, int q_dtype, int grid, hipStream_t stream) {
    hipError_t e = hipErrorInvalidValue;
    with_tile256(kv_dtype, q_dtype, [&](auto kvt, auto qt) {
        e = launch_t<decltype(kvt)::value, decltype(qt)::value>(a, grid, stream);
    });
    return e;
}

}  // namespace pa
