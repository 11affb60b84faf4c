// Tile kernel on the matrix cores (gfx950 MFMA) for chunked prefill and for
// verification-width query blocks.
//
// A work item is (sequence, KV head, block of BM query rows, split of the
// KV tiles).  Query rows of one KV head are token-major (row = i*G + h), so
// a row block holds the G query heads of consecutive new tokens and every
// K/V tile it loads is reused by all of them (grouped-query sharing, as in
// "Dual MI50, part 2", section "Decode: a new kernel for the shape MTP
// actually runs"), and large query tiles amortise each tile load ("Dual MI50,
// part 2", section "Prefill: teach the fork's fast kernel to read the int8
// cache": going from 16 to 64 query rows per tile was 1.8x).
//
// Per tile of BN keys (BN/16 pages gathered through the block table):
//   * K is staged row-major in LDS, V transposed (V^T[d][key]) so that the
//     key dimension, which P.V contracts, is contiguous for the MFMA operand;
//   * S^T = K Q^T with v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q^T
//     held in registers for the whole item): each lane then holds 16 keys of
//     one query row, so the row max / sum need one cross-half exchange;
//   * online softmax in fp32 with an exact running max (a row's largest
//     weight is exactly 1); masked keys are set to -inf by select and dead
//     keys' K and V are zeroed when staged, so NaN in freed pages never
//     reaches a product;
//   * P^T is rounded to the MFMA input type in registers and O^T = V^T P^T is
//     accumulated in fp32; the output is normalised by the sum of the rounded
//     weights (a weighted mean with exactly normalised weights), the lse by
//     the sum of the fp32 weights; at verification widths, which are bound
//     by memory, a second MFMA adds the rounding error of P;
//   * the next tile's global loads are issued before the current tile is
//     computed (register prefetch) and written to LDS after it.
// fp8 (E4M3FN) K is widened to the query's type and fp8 V to fp16 while
// staging; both conversions are exact.  Splits are merged by the last
// workgroup to finish (pa_merge.h).
#include "pa_common.h"
#include "pa_merge.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kPage = 16;
constexpr float kSplitBelow = 32.0f;   // weight sum below which P.V also runs on P's rounding error

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int T>
PA_DEVINLINE f32x16_t mma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
    if constexpr (T == PA_DTYPE_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
}

// Round two floats to the 16-bit type T (RNE) and pack.
template <int T>
PA_DEVINLINE uint32_t pack2(float x, float y) {
    if constexpr (T == PA_DTYPE_BF16) return f32x2_to_bf16x2(f32x2_t{x, y});
    else return f32x2_to_f16x2(f32x2_t{x, y});
}
// The two packed values back as floats (exact).
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
template <int T>
PA_DEVINLINE float unpack_sum(uint32_t u) {
    return unpack_lo<T>(u) + unpack_hi<T>(u);
}

template <int D, int KVT, int QT, int WR>
struct Cfg {
    static constexpr int WK = 4 / WR;                      // wave groups along keys
    static constexpr int BN = (WR == 4) ? 64 : 32;         // keys per tile
    static constexpr int PPT = BN / kPage;                 // pages per tile
    static constexpr int BM = 32 * WR;                     // query rows per item
    static constexpr int NT = 64 * WR;                     // threads per wave group
    static constexpr int KS = D / 16;                      // QK k-steps over the head dim
    static constexpr int DB = D / 32;                      // 32-wide head-dim blocks of O^T
    static constexpr int NB = BN / 32;                     // 32-key blocks of S^T
    static constexpr int TS = BN / 16;                     // 16-key k-steps of P.V
    static constexpr int KROW = D + 8;                     // K tile row stride in LDS (elements)
    static constexpr int VROW = BN + 8;                    // V^T tile row stride in LDS (elements)
    static constexpr int EB = (KVT == PA_DTYPE_FP8_E4M3) ? 1 : 2;
    static constexpr int KCH = BN * (D / 8) / NT;          // 8-element K chunks per thread
    static constexpr int VUN = (BN / 4) * (D / 8) / NT;    // (4 keys x 8 elements) V units per thread
    static constexpr int PVT = (KVT == PA_DTYPE_FP8_E4M3) ? PA_DTYPE_F16 : KVT;  // P.V operand type
    // Verification widths are bound by memory, so P.V runs twice there: on the
    // rounded weights and on their rounding error (near-exact P).
    static constexpr bool PSPLIT = (WR == 1);
    static_assert(KCH >= 1 && VUN >= 1, "tile too small for the thread count");
    static constexpr int GROUP_LDS = (BN * KROW + D * VROW) * 2;   // bytes per wave group
};

template <int KVT>
struct Raw;
template <>
struct Raw<PA_DTYPE_F16> { using T = u32x4_t; };
template <>
struct Raw<PA_DTYPE_BF16> { using T = u32x4_t; };
template <>
struct Raw<PA_DTYPE_FP8_E4M3> { using T = u32x2_t; };

// Eight raw cache elements -> four packed pairs of type T (exact).
template <int KVT, int T>
PA_DEVINLINE u32x4_t widen8(const typename Raw<KVT>::T& c) {
    if constexpr (KVT == PA_DTYPE_FP8_E4M3) {
        u32x4_t r;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x2_t lo = fp8x2_to_f32(c[i], false);
            const f32x2_t hi = fp8x2_to_f32(c[i], true);
            if constexpr (T == PA_DTYPE_BF16) {
                r[2 * i] = f32x2_to_bf16x2(lo);
                r[2 * i + 1] = f32x2_to_bf16x2(hi);
            } else {
                r[2 * i] = f32x2_to_f16x2(lo);
                r[2 * i + 1] = f32x2_to_f16x2(hi);
            }
        }
        return r;
    } else {
        return c;
    }
}

template <int KVT>
PA_DEVINLINE typename Raw<KVT>::T load_raw(const uint8_t* p) {
    if constexpr (KVT == PA_DTYPE_FP8_E4M3) return load_b64(p);
    else return load_b128(p);
}

template <int KVT>
PA_DEVINLINE typename Raw<KVT>::T zero_raw() {
    typename Raw<KVT>::T z;
    if constexpr (KVT == PA_DTYPE_FP8_E4M3) { z[0] = 0; z[1] = 0; }
    else { z[0] = 0; z[1] = 0; z[2] = 0; z[3] = 0; }
    return z;
}

// Per-item geometry shared by all waves.
struct ItemGeom {
    int b, g, qt, split;
    SeqInfo si;
    int row0;            // first row (of the KV head's rows) of this item
    int rows;            // valid rows in this item (<= BM)
    int pg_first;        // first logical page of tile 0
    int pg_end;          // one past the last page with visible keys
    int n_tiles;         // tiles of this row block
    int t_begin, t_end;  // tiles of this split
    int splits;
};

template <int D, int KVT, int QT, int WR>
__global__ __launch_bounds__(256) void mfma_attn_kernel(DecodeArgs a) {
    using C = Cfg<D, KVT, QT, WR>;
    using RawT = typename Raw<KVT>::T;
    constexpr int BM = C::BM, BN = C::BN, PPT = C::PPT;

    __shared__ Plan pl;
    __shared__ int flag;
    __shared__ __attribute__((aligned(16))) uint8_t tiles[C::WK * C::GROUP_LDS];
    __shared__ float red_m[4][32];   // per wave: row max / sum exchange for the WK merge
    __shared__ float red_l[4][32];
    __shared__ float red_e[4][32];
    extern __shared__ int dyn_lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
    const int gi = wid / WR;            // wave group (own KV tile stream)
    const int rb = wid % WR;            // row block of this wave
    const int gtid = tid - gi * C::NT;  // thread index inside the group
    const int h32 = lane >> 5;          // lane half
    const int l32 = lane & 31;

    uint16_t* Ks = reinterpret_cast<uint16_t*>(tiles + gi * C::GROUP_LDS);
    uint16_t* Vt = Ks + BN * C::KROW;

    // ---------------------------------------------------------------- plan
    // A sequence is in this launch if q_len*G lies in [rows_lo, rows_hi].
    // Its rows form ceil(rows/BM) row blocks; each row block's visible keys
    // are cut into tiles of BN keys; tiles are grouped into `splits` splits
    // of `tps` tiles (the same for every row block of the sequence).
    plan_bind(pl, dyn_lds, a.num_seqs);
    {
        const int nthr = blockDim.x;
        long long work = 0;
        long long qtiles = 0;
        int max_tiles = 0;
        int carry_q = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += nthr) {
            const int b = b0 + tid;
            int ql = 0, nqt = 0, tub = 0;
            if (b < a.num_seqs) {
                const int sl = a.seq_lens[b];
                ql = a.q_lens[b];
                pl.seq_len[b] = sl;
                pl.q_len[b] = ql;
                const int rows = ql * a.group;
                if (ql > 0 && rows >= a.rows_lo && rows <= a.rows_hi) {
                    nqt = (rows + BM - 1) / BM;
                    // widest key range over the row blocks: the last full or the last block
                    for (int q = max(0, nqt - 2); q < nqt; ++q) {
                        const int r0 = q * BM, r1 = min(rows, r0 + BM) - 1;
                        const int p0 = sl - ql + r0 / a.group, p1 = sl - ql + r1 / a.group;
                        const int klo = a.window > 0 ? max(0, p0 - a.window + 1) : 0;
                        const int pages = p1 / kPage - klo / kPage + 1;
                        tub = max(tub, (pages + PPT - 1) / PPT);
                    }
                }
                pl.aux[b] = tub;
                pl.item_base[b] = nqt;   // temporary
            }
            int tot;
            const int ex = block_exclusive_scan(ql, pl.red, &tot);
            if (b < a.num_seqs) pl.q_off[b] = carry_q + ex;
            carry_q += tot;
            long long w = (long long)nqt * tub;
            int mt = tub;
            long long nq = nqt;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                w += __shfl_xor(w, o, 64);
                nq += __shfl_xor(nq, o, 64);
                mt = max(mt, __shfl_xor(mt, o, 64));
            }
            __shared__ long long redw[8], redq[8];
            if (lane == 0) { redw[wid] = w; redq[wid] = nq; pl.red[16 + wid] = mt; }
            __syncthreads();
            for (int ww = 0; ww < (int)(blockDim.x / 64); ++ww) {
                work += redw[ww];
                qtiles += redq[ww];
                max_tiles = max(max_tiles, pl.red[16 + ww]);
            }
            __syncthreads();
        }
        work *= a.num_kv_heads;
        qtiles *= a.num_kv_heads;
        int tps;
        if (a.forced_pps > 0) {
            tps = a.forced_pps;
        } else {
            const long long t = a.target_items > 0 ? a.target_items : 1;
            tps = (int)((work + t - 1) / t);
        }
        tps = max(tps, (max_tiles + kMaxSplits - 1) / kMaxSplits);
        {
            long long cap = (long long)a.max_items - qtiles;
            if (cap < 1) cap = 1;
            const long long need = (work + cap - 1) / cap;
            if (tps < need) tps = (int)need;
            if (tps < 1) tps = 1;
        }
        int carry_i = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += nthr) {
            const int b = b0 + tid;
            int it = 0;
            if (b < a.num_seqs) {
                const int nqt = pl.item_base[b];
                const int S = (pl.aux[b] + tps - 1) / tps;
                it = nqt * a.num_kv_heads * S;
                pl.aux[b] = S;   // splits per (sequence, KV head, row block)
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
    const int64_t page_bytes = a.page_stride * C::EB;

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        // ------------------------------------------------------------ item geometry
        ItemGeom ig;
        ig.b = item_seq(pl, a.num_seqs, it);
        ig.si.seq_len = pl.seq_len[ig.b];
        ig.si.q_len = pl.q_len[ig.b];
        ig.si.q_off = pl.q_off[ig.b];
        ig.si.lo = seq_visible_lo(ig.si.seq_len, ig.si.q_len, a.window);
        ig.splits = pl.aux[ig.b];
        {
            const int local = it - pl.item_base[ig.b];
            const int per_qt = a.num_kv_heads * ig.splits;
            ig.qt = local / per_qt;
            const int rem = local - ig.qt * per_qt;
            ig.g = rem / ig.splits;
            ig.split = rem - ig.g * ig.splits;
        }
        // every field is the same in all lanes; keep it in scalar registers
        ig.b = __builtin_amdgcn_readfirstlane(ig.b);
        ig.g = __builtin_amdgcn_readfirstlane(ig.g);
        ig.qt = __builtin_amdgcn_readfirstlane(ig.qt);
        ig.split = __builtin_amdgcn_readfirstlane(ig.split);
        ig.splits = __builtin_amdgcn_readfirstlane(ig.splits);
        ig.si.seq_len = __builtin_amdgcn_readfirstlane(ig.si.seq_len);
        ig.si.q_len = __builtin_amdgcn_readfirstlane(ig.si.q_len);
        ig.si.q_off = __builtin_amdgcn_readfirstlane(ig.si.q_off);
        ig.si.lo = __builtin_amdgcn_readfirstlane(ig.si.lo);
        const int rows_all = ig.si.q_len * a.group;
        ig.row0 = ig.qt * BM;
        ig.rows = min(BM, rows_all - ig.row0);
        const int pos_first = ig.si.seq_len - ig.si.q_len + ig.row0 / a.group;
        const int pos_last = ig.si.seq_len - ig.si.q_len + (ig.row0 + ig.rows - 1) / a.group;
        const int klo = a.window > 0 ? max(0, pos_first - a.window + 1) : 0;
        ig.pg_first = klo / kPage;
        ig.pg_end = pos_last / kPage + 1;
        ig.n_tiles = (ig.pg_end - ig.pg_first + PPT - 1) / PPT;
        {
            // tiles per split of this sequence (same for every row block)
            const int rows_b = rows_all;
            const int nqt = (rows_b + BM - 1) / BM;
            int tub = 0;
            for (int q = max(0, nqt - 2); q < nqt; ++q) {
                const int r0 = q * BM, r1 = min(rows_b, r0 + BM) - 1;
                const int p0 = ig.si.seq_len - ig.si.q_len + r0 / a.group;
                const int p1 = ig.si.seq_len - ig.si.q_len + r1 / a.group;
                const int kl = a.window > 0 ? max(0, p0 - a.window + 1) : 0;
                const int pages = p1 / kPage - kl / kPage + 1;
                tub = max(tub, (pages + PPT - 1) / PPT);
            }
            const int tpsb = (tub + ig.splits - 1) / ig.splits;
            ig.t_begin = min(ig.n_tiles, ig.split * tpsb);
            ig.t_end = min(ig.n_tiles, ig.t_begin + tpsb);
        }
        const float kscale = (KVT == PA_DTYPE_FP8_E4M3) ? a.kv_scale[ig.g] : 1.0f;
        const float vscale = (KVT == PA_DTYPE_FP8_E4M3) ? a.kv_scale[a.num_kv_heads + ig.g] : 1.0f;
        const float s2 = a.scale * kLog2e * kscale;
        const int32_t* bt = a.block_table + (int64_t)ig.b * a.bt_stride;
        const bool direct = (ig.splits == 1);

        // ------------------------------------------------------------ this lane's query row
        const int row_l = rb * 32 + l32;               // row within the item
        const int row_g = ig.row0 + row_l;             // row within the KV head
        const bool row_ok = row_l < ig.rows;
        const int tok_i = row_ok ? row_g / a.group : 0;
        const int pos_r = row_ok ? ig.si.seq_len - ig.si.q_len + tok_i : -1;
        const int lo_r = (a.window > 0) ? pos_r - a.window + 1 : 0;
        // rows of this wave: position range, for the "tile needs no mask" test
        const int w_row0 = ig.row0 + rb * 32;
        const int w_rows = max(0, min(32, ig.rows - rb * 32));
        const int w_pmin = ig.si.seq_len - ig.si.q_len + w_row0 / a.group;
        const int w_pmax = ig.si.seq_len - ig.si.q_len + (w_row0 + max(w_rows, 1) - 1) / a.group;
        const int w_lomax = (a.window > 0) ? w_pmax - a.window + 1 : 0;

        u32x4_t qreg[C::KS];
        {
            const int h = ig.g * a.group + (row_ok ? row_g - tok_i * a.group : 0);
            const uint16_t* qp = qbase + ((int64_t)(ig.si.q_off + tok_i) * a.num_q_heads + h) * D + 8 * h32;
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                if (row_ok) qreg[s] = load_b128_cached(qp + 16 * s);
                else { qreg[s][0] = 0; qreg[s][1] = 0; qreg[s][2] = 0; qreg[s][3] = 0; }
            }
        }

        f32x16_t o_acc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o_acc[db][i] = 0.f;
        float m_run = kNegInf;
        float l_run = 0.f;      // sum of the rounded weights that multiplied V (output normalisation)
        float l_exact = 0.f;    // sum of the fp32 weights (lse)

        // ------------------------------------------------------------ staging
        // The PPT page ids of a tile are the same for the whole workgroup:
        // they are read with scalar loads one tile ahead of the K/V loads.
        RawT kraw[C::KCH];
        RawT vraw[C::VUN][4];
        // K chunk c: key ch / (D/8), element (ch % (D/8)) * 8 (a wave reads whole rows).
        // V unit u: keys 4*(un % (BN/4)) .. +3, element (un / (BN/4)) * 8 (keys fastest, so
        // the transposed LDS writes of a wave fall in distinct banks).
        // Loads are unconditional so the wait counts stay exact: a page past
        // the visible range reads the last visible page's id, and dead keys
        // (outside [lo, seq_len) or past that page) are zeroed when stored.
        auto load_pids = [&](int t, int (&pid)[PPT]) {
#pragma unroll
            for (int p = 0; p < PPT; ++p) {
                const int pg = min(ig.pg_first + t * PPT + p, ig.pg_end - 1);
                pid[p] = bt[pg];
            }
        };
        auto key_live = [&](int t, int key) -> bool {
            const int pg = ig.pg_first + t * PPT + key / kPage;
            const int j = pg * kPage + key % kPage;
            return pg < ig.pg_end && j >= ig.si.lo && j < ig.si.seq_len;
        };
        const int64_t head_off = kv_offset(0, ig.g, 0, a.page_stride, a.head_stride, a.token_stride) * C::EB;
        auto key_off = [&](const int (&pid)[PPT], int key) -> int64_t {
            return (int64_t)pid[key / kPage] * page_bytes + head_off + (int64_t)(key % kPage) * a.token_stride * C::EB;
        };
        uint32_t live_k = 0, live_v = 0;      // live masks of the staged chunks
        auto load_tile = [&](int t, const int (&pid)[PPT]) {
            live_k = 0;
            live_v = 0;
#pragma unroll
            for (int c = 0; c < C::KCH; ++c) {
                const int ch = gtid + c * C::NT;
                const int key = ch / (D / 8), e = (ch % (D / 8)) * 8;
                kraw[c] = load_raw<KVT>(kbase + key_off(pid, key) + e * C::EB);
                live_k |= key_live(t, key) ? (1u << c) : 0u;
            }
#pragma unroll
            for (int u = 0; u < C::VUN; ++u) {
                const int un = gtid + u * C::NT;
                const int k4 = (un % (BN / 4)) * 4, e = (un / (BN / 4)) * 8;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    vraw[u][q] = load_raw<KVT>(vbase + key_off(pid, k4 + q) + e * C::EB);
                    live_v |= key_live(t, k4 + q) ? (1u << (4 * u + q)) : 0u;
                }
            }
        };
        auto store_tile = [&]() {
#pragma unroll
            for (int c = 0; c < C::KCH; ++c) {
                const int ch = gtid + c * C::NT;
                const int key = ch / (D / 8), e = (ch % (D / 8)) * 8;
                const RawT r = (live_k >> c) & 1u ? kraw[c] : zero_raw<KVT>();
                *reinterpret_cast<u32x4_t*>(Ks + key * C::KROW + e) = widen8<KVT, QT>(r);
            }
#pragma unroll
            for (int u = 0; u < C::VUN; ++u) {
                const int un = gtid + u * C::NT;
                const int k4 = (un % (BN / 4)) * 4, e = (un / (BN / 4)) * 8;
                u32x4_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = widen8<KVT, C::PVT>((live_v >> (4 * u + q)) & 1u ? vraw[u][q] : zero_raw<KVT>());
                // transpose 4 keys x 8 elements into V^T[e + x][k4 .. k4 + 3]
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    // element pair (2x, 2x+1) of each key
                    const uint32_t lo01 = __builtin_amdgcn_perm(w[1][x], w[0][x], 0x05040100u);
                    const uint32_t lo23 = __builtin_amdgcn_perm(w[3][x], w[2][x], 0x05040100u);
                    const uint32_t hi01 = __builtin_amdgcn_perm(w[1][x], w[0][x], 0x07060302u);
                    const uint32_t hi23 = __builtin_amdgcn_perm(w[3][x], w[2][x], 0x07060302u);
                    *reinterpret_cast<u32x2_t*>(Vt + (e + 2 * x) * C::VROW + k4) = u32x2_t{lo01, lo23};
                    *reinterpret_cast<u32x2_t*>(Vt + (e + 2 * x + 1) * C::VROW + k4) = u32x2_t{hi01, hi23};
                }
            }
        };

        // ------------------------------------------------------------ tile loop
        const int my_first = ig.t_begin + gi;
        const int n_iter = (ig.t_end - ig.t_begin + C::WK - 1) / C::WK;
        int pid_next[PPT];                     // page ids of the tile after the one in flight
        if (n_iter > 0) {
            int pid0[PPT];
            load_pids(my_first, pid0);
            load_tile(my_first, pid0);
            load_pids(my_first + C::WK, pid_next);
        }
        for (int iter = 0; iter < n_iter; ++iter) {
            const int t = my_first + iter * C::WK;
            const bool have = t < ig.t_end;
            __syncthreads();                  // previous tile's LDS reads are done
            if (have) store_tile();
            __syncthreads();
            const int tn = t + C::WK;
            if (iter + 1 < n_iter) load_tile(tn, pid_next);   // in flight while this tile is computed
            load_pids(tn + C::WK, pid_next);
            if (!have) continue;

            // S^T = K Q^T: NB blocks of 32 keys x 32 rows
            f32x16_t sacc[C::NB];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[nb][i] = 0.f;
#pragma unroll
                for (int s = 0; s < C::KS; ++s) {
                    const u32x4_t kf =
                        *reinterpret_cast<const u32x4_t*>(Ks + (nb * 32 + l32) * C::KROW + 16 * s + 8 * h32);
                    sacc[nb] = mma32<QT>(kf, qreg[s], sacc[nb]);
                }
            }
            // scale, mask, tile max
            const int key0 = (ig.pg_first + t * PPT) * kPage;   // position of the tile's first key
            const bool full = (key0 >= w_lomax) && (key0 + BN - 1 <= w_pmin) && (key0 >= ig.si.lo) &&
                              (key0 + BN <= ig.si.seq_len) && (ig.pg_first + (t + 1) * PPT <= ig.pg_end);
            float tmax = kNegInf;
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = sacc[nb][i] * s2;
                    if (!full) {
                        const int j = key0 + nb * 32 + 8 * (i / 4) + 4 * h32 + (i % 4);
                        const bool vis = (j <= pos_r) && (j >= lo_r) && (j >= ig.si.lo) && (j < ig.si.seq_len);
                        x = vis ? x : kNegInf;
                    }
                    sacc[nb][i] = x;
                    tmax = fmaxf(tmax, x);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            // exact running max: the largest weight of a row is exactly 1, so a
            // row dominated by one key loses nothing to the rounding of P
            if (wave_any(tmax > m_run)) {
                const float mn = fmaxf(m_run, tmax);
                const float al = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - mn);
                // rows whose max did not move keep al == 1 (mn == m_run)
                m_run = mn;
                l_run *= al;
                l_exact *= al;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o_acc[db][i] *= al;
            }
            // P^T (rounded to the P.V type) and O^T += V^T P^T
            u32x4_t pb[C::TS];
#pragma unroll
            for (int ts = 0; ts < C::TS; ++ts) {
                const int nb = ts / 2, i0 = 8 * (ts % 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x0 = sacc[nb][i0 + 2 * j], x1 = sacc[nb][i0 + 2 * j + 1];
                    const float p0 = (x0 == kNegInf) ? 0.f : fast_exp2(x0 - m_run);
                    const float p1 = (x1 == kNegInf) ? 0.f : fast_exp2(x1 - m_run);
                    sacc[nb][i0 + 2 * j] = p0;
                    sacc[nb][i0 + 2 * j + 1] = p1;
                    l_exact += p0 + p1;
                    pb[ts][j] = pack2<C::PVT>(p0, p1);
                    l_run += unpack_sum<C::PVT>(pb[ts][j]);
                }
            }
            // While a row has few effective keys (small weight sum), rounding P
            // to 8 or 11 bits is visible in the output: add a second P.V on the
            // rounding error.  Always on at verification widths (memory-bound).
            const bool split = C::PSPLIT || wave_any(l_exact < kSplitBelow);
#pragma unroll
            for (int ts = 0; ts < C::TS; ++ts) {
                const int nb = ts / 2, i0 = 8 * (ts % 2);
                u32x4_t pl2;
                if (split) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pl2[j] = pack2<C::PVT>(sacc[nb][i0 + 2 * j] - unpack_lo<C::PVT>(pb[ts][j]),
                                               sacc[nb][i0 + 2 * j + 1] - unpack_hi<C::PVT>(pb[ts][j]));
                        l_run += unpack_sum<C::PVT>(pl2[j]);
                    }
                }
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    const uint16_t* vr = Vt + (db * 32 + l32) * C::VROW + 16 * ts + 4 * h32;
                    const u32x2_t va = *reinterpret_cast<const u32x2_t*>(vr);
                    const u32x2_t vb = *reinterpret_cast<const u32x2_t*>(vr + 8);
                    const u32x4_t vf = {va[0], va[1], vb[0], vb[1]};
                    o_acc[db] = mma32<C::PVT>(vf, pb[ts], o_acc[db]);
                    if (split) o_acc[db] = mma32<C::PVT>(vf, pl2, o_acc[db]);
                }
            }
        }

        // ------------------------------------------------------------ finish the row
        // each row lives in lanes l32 and l32 + 32 (same m_run); sum their l
        float L = l_run + __shfl_xor(l_run, 32, 64);
        float LE = l_exact + __shfl_xor(l_exact, 32, 64);
        float M = m_run;
        if (C::WK > 1) {
            // combine the WK wave groups (same rows, disjoint tiles) through LDS
            __syncthreads();
            if (h32 == 0) { red_m[wid][l32] = M; red_l[wid][l32] = L; red_e[wid][l32] = LE; }
            __syncthreads();
            float Mx = kNegInf;
#pragma unroll
            for (int w = 0; w < C::WK; ++w) Mx = fmaxf(Mx, red_m[w * WR + rb][l32]);
            const float al = (M == kNegInf) ? 0.f : fast_exp2(M - Mx);
            float Lx = 0.f, LEx = 0.f;
#pragma unroll
            for (int w = 0; w < C::WK; ++w) {
                const float mw = red_m[w * WR + rb][l32];
                const float f = (mw == kNegInf) ? 0.f : fast_exp2(mw - Mx);
                Lx += red_l[w * WR + rb][l32] * f;
                LEx += red_e[w * WR + rb][l32] * f;
            }
            // reuse the tile LDS as a [WK][32][D] fp32 reduction buffer per row block
            __syncthreads();
            float* accbuf = reinterpret_cast<float*>(tiles);
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d = db * 32 + 8 * jj + 4 * h32;
                    float4 v = make_float4(o_acc[db][4 * jj] * al, o_acc[db][4 * jj + 1] * al, o_acc[db][4 * jj + 2] * al,
                                           o_acc[db][4 * jj + 3] * al);
                    *reinterpret_cast<float4*>(accbuf + ((gi * WR + rb) * 32 + l32) * D + d) = v;
                }
            __syncthreads();
            if (gi == 0) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d = db * 32 + 8 * jj + 4 * h32;
                        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
                        for (int w = 0; w < C::WK; ++w) {
                            const float4 v = *reinterpret_cast<const float4*>(accbuf + ((w * WR + rb) * 32 + l32) * D + d);
                            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
                        }
                        o_acc[db][4 * jj] = s.x; o_acc[db][4 * jj + 1] = s.y;
                        o_acc[db][4 * jj + 2] = s.z; o_acc[db][4 * jj + 3] = s.w;
                    }
            }
            M = Mx;
            L = Lx;
            LE = LEx;
        }
        if (gi == 0 && row_ok) {
            const float inv = (L > 0.f) ? 1.0f / L : 0.f;
            MergeTarget tgt{a.out, a.lse, a.num_q_heads, a.group, vscale};
            if (direct) {
                const int64_t orow = out_row(tgt, ig.si.q_off, ig.g, row_g);
                float* op = a.out + orow * D;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d = db * 32 + 8 * jj + 4 * h32;
                        const float sc = inv * vscale;
                        *reinterpret_cast<float4*>(op + d) =
                            make_float4(o_acc[db][4 * jj] * sc, o_acc[db][4 * jj + 1] * sc, o_acc[db][4 * jj + 2] * sc,
                                        o_acc[db][4 * jj + 3] * sc);
                    }
                if (a.lse != nullptr && h32 == 0) a.lse[orow] = (LE > 0.f) ? (M + fast_log2(LE)) * kLn2 : kNegInf;
            } else {
                const int64_t slot = (int64_t)it * BM + row_l;
                float* op = a.ws_o + slot * D;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d = db * 32 + 8 * jj + 4 * h32;
                        *reinterpret_cast<float4*>(op + d) =
                            make_float4(o_acc[db][4 * jj] * inv, o_acc[db][4 * jj + 1] * inv, o_acc[db][4 * jj + 2] * inv,
                                        o_acc[db][4 * jj + 3] * inv);
                    }
                if (h32 == 0) a.ws_lse[slot] = (LE > 0.f) ? M + fast_log2(LE) : kNegInf;
            }
        }
        if (!direct) {
            const int64_t first_item = it - ig.split;
            int* ctr = a.counters + ((int64_t)ig.b * a.num_kv_heads + ig.g) * a.counter_stride + ig.qt;
            if (arrive_last(ctr, ig.splits, &flag)) {
                __syncthreads();
                MergeTarget tgt{a.out, a.lse, a.num_q_heads, a.group, vscale};
                merge_splits<D>(a.ws_o, a.ws_lse, first_item, ig.splits, ig.rows, BM, tgt, ig.si.q_off, ig.g,
                                *reinterpret_cast<MergeShared*>(tiles), ig.row0);
            }
        }
        __syncthreads();
    }
}

}  // namespace

template <int D, int KVT, int QT, int WR>
static hipError_t launch_t(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((mfma_attn_kernel<D, KVT, QT, WR>), dim3(grid), dim3(256), plan_lds_bytes(a.num_seqs), st, a);
    return hipGetLastError();
}

template <int WR>
static hipError_t launch_wr(const DecodeArgs& a, int kvt, int qt, int grid, hipStream_t st) {
    if (kvt == PA_DTYPE_F16) return launch_t<128, PA_DTYPE_F16, PA_DTYPE_F16, WR>(a, grid, st);
    if (kvt == PA_DTYPE_BF16) return launch_t<128, PA_DTYPE_BF16, PA_DTYPE_BF16, WR>(a, grid, st);
    if (qt == PA_DTYPE_BF16) return launch_t<128, PA_DTYPE_FP8_E4M3, PA_DTYPE_BF16, WR>(a, grid, st);
    return launch_t<128, PA_DTYPE_FP8_E4M3, PA_DTYPE_F16, WR>(a, grid, st);
}

int mfma_rows_per_item(int wr) { return 32 * wr; }

hipError_t launch_mfma_attn(const DecodeArgs& a, int head_dim, int kv_dtype, int q_dtype, int wr, int grid,
                            hipStream_t stream) {
    if (head_dim != 128) return hipErrorInvalidValue;
    if (wr == 4) return launch_wr<4>(a, kv_dtype, q_dtype, grid, stream);
    return launch_wr<1>(a, kv_dtype, q_dtype, grid, stream);
}

}  // namespace pa
