// Tile kernel on the matrix cores (gfx950 MFMA) for chunked prefill and for
// verification-width query blocks.
//
// A work item is (sequence, KV head, block of BM query rows, split of the
// KV tiles).  Query rows of one KV head are token-major (row = i*G + h), so a
// row block holds the G query heads of consecutive new tokens and every K/V
// tile it loads is reused by all of them (grouped-query sharing, "Dual MI50,
// part 2", section "Decode: a new kernel for the shape MTP actually runs"),
// and big query tiles amortise each tile load ("Dual MI50, part 2", section
// "Prefill: teach the fork's fast kernel to read the int8 cache": 16 to 64
// query rows per tile was 1.8x there).
//
// Two shapes share the code:
//   * WR = 8 (prefill): eight waves own 32 rows each (BM = 256), two per
//     SIMD, and share 32-key tiles in a six-slot LDS ring, filled six tiles
//     ahead by asynchronous global->LDS loads (16-bit caches) or by the waves
//     themselves, each widening an eighth of a tile exactly to 16 bits
//     through registers (one-byte caches; int8 row scales beside the slot); a
//     software pipeline puts the scores of tile k+1 on the matrix cores,
//     reads tile k's V fragments while they run, turns tile k's scores into
//     P on the VALU and runs P.V of tile k, then reads tile k+2's K
//     fragments while P.V runs; the second wave of each SIMD issues its P.V
//     after the per-tile barrier, a phase behind the first;
//   * WR = 1 (verification widths and few-row sequences, <= 64 rows per KV
//     head): each wave owns the same 32 rows and streams its own 32-key
//     tiles, so the tile loop has no workgroup barrier; the four waves'
//     softmax states are merged at the end.  16-bit tiles are staged through
//     registers into the wave's LDS tile; fp8 tiles go by asynchronous loads
//     into two raw staging slots and both operands are read raw (K by 64-bit
//     reads, V by 8-bit transposing reads) and widened in registers.
//
// Per tile of BN keys (BN/16 pages gathered through the block table):
//   * LDS rows have their 16-byte chunks XOR-swizzled by the row index, so
//     that the operand reads (one chunk of many rows at once) are free of
//     bank conflicts;
//   * S^T = K Q^T with v_mfma_f32_32x32x16 (A = K rows, B = Q^T held in
//     registers): each lane then holds 16 keys of one query row;
//   * V^T operands come straight from the row-major V tile through the
//     gfx950 transposing LDS reads (ds_read_b64_tr_b16, or _tr_b8 on raw
//     fp8): the 8-byte pieces of several key rows come back as several keys
//     of one head-dim column;
//   * online softmax in fp32 against a lazily raised reference max (moved
//     only when a score passes it by 2^8, so weights stay <= 256 and the
//     accumulators are rarely rescaled); masked keys are set to -inf by
//     select and dead keys' V rows are zeroed in LDS, so NaN in freed pages
//     never reaches a product;
//   * P^T is rounded to the MFMA input type and output and lse are
//     normalised by the fp32 weight sum; with 16-bit caches at verification
//     widths, and while a row has few effective keys, a second MFMA adds P's
//     rounding error, so rows dominated by a few keys keep full precision.
// Splits are combined by the merge launch that follows (pa_merge.h).
#include "pa_common.h"
#include "pa_merge.h"
#include "pa_kernels.h"

#include <type_traits>
#include <utility>

namespace pa {

namespace {

constexpr int kPage = 16;
// P.V also runs on P's rounding error while a row's weight sum is below
// kSplitBelow times its largest weight.  Past that point the largest single
// weight is at most 1/kSplitBelow of the sum, so rounding it to 16 bits
// (relative 2^-9 for bf16) moves the output by at most 2^-9/8 |v| ~ 2.4e-4 |v|,
// and the other weights' rounding errors are independent of it.
constexpr float kSplitBelow = 8.0f;
constexpr float kTau = 8.0f;           // lazy max: rescale when a score passes the reference by 2^8
constexpr int kRowBytes = 256;         // one K or V row in LDS: 128 16-bit elements

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
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

// Maximum that propagates NaN (IEEE maximum): gfx950 issues it as one
// three-operand instruction with no canonicalising of its inputs.
PA_DEVINLINE float fmax_nan(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// max(x[l], x[l ^ 32]) for every lane l (NaN-propagating)
PA_DEVINLINE float half_swap_max(float x) {
    const f32x2_t p = xor_pair<32>(x);
    return fmax_nan(p.x, p.y);
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// waits for every asynchronous tile load still in flight (they write LDS).
// Callers make the data they hand over complete themselves (the LDS read
// helpers wait inside their asm blocks; tile loads are waited for by count).
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
PA_DEVINLINE void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] in bits 3:0, expcnt in 6:4,
// lgkmcnt in 11:8, vmcnt[5:4] in 15:14); a field at its maximum is not waited on.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// Asynchronous 16-byte load per lane into LDS: lane l's bytes land at
// lds + 16*l (gfx950 global_load_lds_dwordx4).  The body exists only in the
// device compilation pass (the host pass never runs kernel code).
PA_DEVINLINE void async_load16(const void* src, lds_void_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#else
    (void)src;
    (void)lds;
#endif
}

// Asynchronous 4-byte load per lane into LDS: lane l's dword lands at
// lds + 4*l (global_load_lds_dword).
PA_DEVINLINE void async_load4(const void* src, lds_void_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
#else
    (void)src;
    (void)lds;
#endif
}

// Byte offset of 16-byte chunk c of row r inside a tile.  Rows are 256 B (one
// full pass over the banks), so the chunk index is XOR-ed with a row key that
// puts the row's low two bits into the chunk's high two bits: the K operand
// read (16 rows, one chunk each) and the transposing V read (4 consecutive
// rows x 4 consecutive chunks per 32 lanes) both land in distinct banks.
PA_DEVINLINE int swz_key(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
PA_DEVINLINE int swz(int r, int c) { return r * kRowBytes + ((c ^ swz_key(r)) << 4); }

// Eight transposing 64-bit LDS reads (ds_read_b64_tr_b16) at addr[k] + OFF,
// completed inside the block.  Inline asm because the compiler cannot tell
// which LDS object the transposing-read builtin touches and would make it
// wait for every asynchronous tile load in flight, including the prefetch
// into the other buffer.  Outputs are early-clobber: each read lands while
// later addresses are still being consumed.
// Eight 128-bit LDS reads at addr[k] + OFF, completed inside the block (the
// pipelined path manages its asynchronous-load waits itself).
template <int OFF>
PA_DEVINLINE void lds_read_b128_x8(const uint32_t (&addr)[8], u32x4_t (&r)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\t"
        "ds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\t"
        "ds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%16\n\t"
        "ds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %14 offset:%16\n\t"
        "ds_read_b128 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7]), "i"(OFF)
        : "memory");
}

// Raw fp8 K operand fragments of staging slot SLOT (slots 8 KB apart): eight
// 64-bit reads at ka[s], completed inside the block.  These reads (and the V
// reads below) are invisible to the compiler's wait insertion, so the caller
// orders them after the asynchronous loads that fill the slot.
#define PA_RAW_K_READS(OFF)                                                                          \
    asm volatile("ds_read_b64 %0, %8 offset:" #OFF "\n\t"                                           \
                 "ds_read_b64 %1, %9 offset:" #OFF "\n\t"                                           \
                 "ds_read_b64 %2, %10 offset:" #OFF "\n\t"                                          \
                 "ds_read_b64 %3, %11 offset:" #OFF "\n\t"                                          \
                 "ds_read_b64 %4, %12 offset:" #OFF "\n\t"                                          \
                 "ds_read_b64 %5, %13 offset:" #OFF "\n\t"                                          \
                 "ds_read_b64 %6, %14 offset:" #OFF "\n\t"                                          \
                 "ds_read_b64 %7, %15 offset:" #OFF "\n\t"                                          \
                 "s_waitcnt lgkmcnt(0)"                                                              \
                 : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),     \
                   "=&v"(k[6]), "=&v"(k[7])                                                          \
                 : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), \
                   "v"(ka[7])                                                                        \
                 : "memory")
template <int SLOT>
PA_DEVINLINE void lds_read_raw_k(const uint32_t (&ka)[8], u32x2_t (&k)[8]) {
    static_assert(SLOT == 0 || SLOT == 1, "two staging slots");
    if constexpr (SLOT == 0) PA_RAW_K_READS(0);
    else PA_RAW_K_READS(8192);
}
#undef PA_RAW_K_READS

// Raw fp8 V^T operand fragments of slot SLOT by 8-bit transposing reads
// (ds_read_b64_tr_b8: within 16 lanes, the 8-byte pieces of lanes 2r, 2r+1
// form row r of an 8 x 16-byte block and lane j receives byte j of every
// row).  v[ts * 4 + db] for 16-key step ts and 32-column block db: va[db]
// addresses the block's rows of step 0, step 1 is 2 KB further; V is 4 KB
// into the slot.  Completed inside the block.
#define PA_RAW_V_READS(O0, O1)                                                                       \
    asm volatile("ds_read_b64_tr_b8 %0, %8 offset:" #O0 "\n\t"                                      \
                 "ds_read_b64_tr_b8 %1, %9 offset:" #O0 "\n\t"                                      \
                 "ds_read_b64_tr_b8 %2, %10 offset:" #O0 "\n\t"                                     \
                 "ds_read_b64_tr_b8 %3, %11 offset:" #O0 "\n\t"                                     \
                 "ds_read_b64_tr_b8 %4, %8 offset:" #O1 "\n\t"                                      \
                 "ds_read_b64_tr_b8 %5, %9 offset:" #O1 "\n\t"                                      \
                 "ds_read_b64_tr_b8 %6, %10 offset:" #O1 "\n\t"                                     \
                 "ds_read_b64_tr_b8 %7, %11 offset:" #O1 "\n\t"                                     \
                 "s_waitcnt lgkmcnt(0)"                                                              \
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),     \
                   "=&v"(v[6]), "=&v"(v[7])                                                          \
                 : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])                                    \
                 : "memory")
template <int SLOT>
PA_DEVINLINE void lds_read_raw_vt(const uint32_t (&va)[4], u32x2_t (&v)[8]) {
    static_assert(SLOT == 0 || SLOT == 1, "two staging slots");
    if constexpr (SLOT == 0) PA_RAW_V_READS(4096, 6144);
    else PA_RAW_V_READS(12288, 14336);
}
#undef PA_RAW_V_READS

// One 128-bit LDS store at addr + OFF.  Inline asm for the same reason as the
// reads: the compiler's alias tracking can lose the LDS object of such stores
// and wait for every asynchronous load in flight.  A store takes its data at
// issue; the caller orders later reads.
template <int OFF>
PA_DEVINLINE void lds_store_b128(uint32_t addr, const u32x4_t& d) {
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(d), "i"(OFF) : "memory");
}

// Sixteen 128-bit LDS reads: addr[k] (into r0) and addr[k] + OFF (into r1),
// completed inside the block.
template <int OFF>
PA_DEVINLINE void lds_read_b128_x16(const uint32_t (&addr)[8], u32x4_t (&r0)[8], u32x4_t (&r1)[8]) {
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %17\n\t"
        "ds_read_b128 %2, %18\n\t"
        "ds_read_b128 %3, %19\n\t"
        "ds_read_b128 %4, %20\n\t"
        "ds_read_b128 %5, %21\n\t"
        "ds_read_b128 %6, %22\n\t"
        "ds_read_b128 %7, %23\n\t"
        "ds_read_b128 %8, %16 offset:%24\n\t"
        "ds_read_b128 %9, %17 offset:%24\n\t"
        "ds_read_b128 %10, %18 offset:%24\n\t"
        "ds_read_b128 %11, %19 offset:%24\n\t"
        "ds_read_b128 %12, %20 offset:%24\n\t"
        "ds_read_b128 %13, %21 offset:%24\n\t"
        "ds_read_b128 %14, %22 offset:%24\n\t"
        "ds_read_b128 %15, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0[0]), "=&v"(r0[1]), "=&v"(r0[2]), "=&v"(r0[3]), "=&v"(r0[4]), "=&v"(r0[5]), "=&v"(r0[6]),
          "=&v"(r0[7]), "=&v"(r1[0]), "=&v"(r1[1]), "=&v"(r1[2]), "=&v"(r1[3]), "=&v"(r1[4]), "=&v"(r1[5]),
          "=&v"(r1[6]), "=&v"(r1[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7]), "i"(OFF)
        : "memory");
}

// Sixteen transposing 64-bit LDS reads at addr[k] + OFF0 (into r0) and
// addr[k] + OFF1 (into r1), completed inside the block.
template <int OFF0, int OFF1>
PA_DEVINLINE void lds_read_tr16_x16(const uint32_t (&addr)[8], u32x2_t (&r0)[8], u32x2_t (&r1)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %2, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%25\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
        "ds_read_b64_tr_b16 %12, %20 offset:%25\n\t"
        "ds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0[0]), "=&v"(r0[1]), "=&v"(r0[2]), "=&v"(r0[3]), "=&v"(r0[4]), "=&v"(r0[5]), "=&v"(r0[6]),
          "=&v"(r0[7]), "=&v"(r1[0]), "=&v"(r1[1]), "=&v"(r1[2]), "=&v"(r1[3]), "=&v"(r1[4]), "=&v"(r1[5]),
          "=&v"(r1[6]), "=&v"(r1[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7]), "i"(OFF0), "i"(OFF1)
        : "memory");
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
PA_DEVINLINE void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
PA_DEVINLINE void static_for(F&& f) { static_for_impl(f, std::make_integer_sequence<int, N>{}); }

template <int OFF>
PA_DEVINLINE void lds_read_tr16_x8(const uint32_t (&addr)[8], u32x2_t (&r)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7]), "i"(OFF)
        : "memory");
}

template <int WR>
constexpr int tile_threads() { return WR == 8 ? 512 : 256; }

template <int D, int KVT, int QT, int WR>
struct Cfg {
    static_assert(D == 128, "the tile kernel is built for head_dim 128");
    static constexpr int NW = (WR == 8) ? 8 : 4;           // waves per workgroup
    static constexpr int NTH = 64 * NW;                    // threads per workgroup
    static_assert(NTH == tile_threads<WR>(), "launch bounds");
    static constexpr int WK = NW / WR;                     // wave groups along keys
    static_assert(WR == 1 || WR == 8, "items of 32 rows (four key streams) or 256 rows (eight waves)");
    static constexpr int BN = 32;                          // keys per tile
    static constexpr int PPT = BN / kPage;                 // pages per tile
    static constexpr int BM = 32 * WR;                     // query rows per item
    static constexpr int NT = 64 * WR;                     // threads per wave group
    static constexpr int KS = D / 16;                      // QK k-steps over the head dim
    static constexpr int DB = D / 32;                      // 32-wide head-dim blocks of O^T
    static constexpr int NB = BN / 32;                     // 32-key blocks of S^T
    static constexpr int TS = BN / 16;                     // 16-key k-steps of P.V
    static constexpr bool FP8 = (KVT == PA_DTYPE_FP8_E4M3);
    static constexpr bool INT8 = (KVT == PA_DTYPE_INT8);   // int8 codes with a fp32 scale per row
    static constexpr bool BYTE = FP8 || INT8;              // one-byte cache elements
    static constexpr int EB = BYTE ? 1 : 2;
    static constexpr int PVT = BYTE ? PA_DTYPE_F16 : KVT;  // P.V operand type
    // memory-bound 16-bit caches: P.V always on the split P (fp8 caches never
    // split P: their own error is far larger than P's f16 rounding)
    static constexpr bool PSPLIT = (WR == 1) && !BYTE;
    static constexpr int TILE = BN * kRowBytes;            // bytes of one K (or V) tile in LDS
    static constexpr int GROUP_LDS = 2 * TILE;             // a wave group's K and V tile in LDS
    static constexpr int DMA_PER_WAVE = BN * kRowBytes / 1024 / WR;   // 1 KB async loads per wave per tile
    // fp8 at WR = 1: raw tiles reach LDS by asynchronous loads into two
    // staging slots per wave (K then V, 8 KB a slot); both operands are read
    // raw (V by 8-bit transposing reads) and widened in registers at their
    // matrix ops.  RAW_DMA 1 KB loads per wave per tile (K and V).
    static constexpr bool FSTAGE = BYTE && (WR == 1);
    // V through registers (32-row one-byte items): V rows are loaded one
    // step ahead into registers and written into the staging slot when their
    // step begins, K alone takes the asynchronous path (which tops out lower
    // than register loads, so the two paths together move more)
    static constexpr bool VREG = FSTAGE && FP8;   // (int8's scale registers leave no room)
    static constexpr int RAW_TILE = BN * D;                // bytes of one raw fp8 K (or V) tile
    // int8: one more 4-byte load per lane and tile brings the tile's K and V
    // row scales into LDS
    static constexpr int RAW_DMA = (VREG ? 1 : 2) * RAW_TILE / 1024 + (INT8 ? 1 : 0);
    static constexpr int STAGE_LDS = FSTAGE ? WK * 2 * 2 * RAW_TILE : 16;
    // 256-row items on 16-bit caches run a software pipeline: K tiles in a
    // ring of NKB buffers, V tiles in a ring of NVB, loads issued LEAD tiles
    // ahead; the item's page ids are staged in LDS (PID_CAP of them).  The
    // loop is unrolled over the ring, so buffer offsets are immediates.
    // One-byte caches join it with register-staged tiles: each wave brings
    // its eighth of a tile through registers, widens it exactly to 16 bits
    // and stores it into the ring slot (int8: with its rows' K and V scales
    // into the slot's scale array).
    static constexpr bool PIPE = (WR == 8);
    static constexpr int NKB = 6, NVB = 6, LEAD = 6;
    static constexpr int PID_CAP = PIPE ? 4096 : (WR == 1 ? 1024 : 1);
    static constexpr int TILES_LDS = PIPE ? (NKB + NVB) * TILE : (FSTAGE ? 16 : WK * GROUP_LDS);
    // int8 row scales of a tile: BN K scales then BN V scales, per staging
    // slot (FSTAGE) or per wave group's LDS tile
    static constexpr int SC_FLOATS = INT8 ? (PIPE ? NKB : FSTAGE ? WK * 2 : WK) * 2 * BN : 4;
};

template <int KVT>
struct Raw;
template <>
struct Raw<PA_DTYPE_F16> { using T = u32x4_t; };
template <>
struct Raw<PA_DTYPE_BF16> { using T = u32x4_t; };
template <>
struct Raw<PA_DTYPE_FP8_E4M3> { using T = u32x2_t; };
template <>
struct Raw<PA_DTYPE_INT8> { using T = u32x2_t; };

// Eight fp8 e4m3 values to eight 16-bit values, exactly (both targets hold
// every e4m3 value): the gfx950 scaled conversion with scale 1 turns two fp8
// bytes of a word (low or high half) into a packed pair in one instruction.
template <int T>
PA_DEVINLINE u32x4_t widen_fp8x8(const u32x2_t& c) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if constexpr (T == PA_DTYPE_BF16) {
            r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false));
            r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true));
        } else {
            r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.0f, false));
            r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.0f, true));
        }
    }
    return r;
}

// Eight one-byte cache codes to eight 16-bit values of type T, exactly.
template <int T, int KVT>
PA_DEVINLINE u32x4_t widen8(const u32x2_t& c) {
    if constexpr (KVT == PA_DTYPE_FP8_E4M3) {
        return widen_fp8x8<T>(c);
    } else {
        u32x4_t r;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t lo, hi;
            if constexpr (T == PA_DTYPE_BF16) i8x4_to_bf16x4(c[i], lo, hi);
            else i8x4_to_f16x4(c[i], lo, hi);
            r[2 * i] = lo;
            r[2 * i + 1] = hi;
        }
        return r;
    }
}

struct ItemGeom {
    int b, g, qt, split, splits;
    SeqInfo si;
    int row0, rows;
    int pg_first, pg_end;
    int n_tiles, t_begin, t_end;
};

template <int D, int KVT, int QT, int WR>
__global__ __launch_bounds__(tile_threads<WR>()) void tile_attn_kernel(DecodeArgs a) {
    using C = Cfg<D, KVT, QT, WR>;
    constexpr int BM = C::BM, BN = C::BN, PPT = C::PPT;

    __shared__ Plan pl;
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[C::TILES_LDS];
    __shared__ __attribute__((aligned(16))) int ipid[C::PID_CAP];
    __shared__ __attribute__((aligned(1024))) uint8_t stage[C::STAGE_LDS];
    __shared__ __attribute__((aligned(16))) float tscale[C::SC_FLOATS];
    __shared__ float red_m[4][32];
    __shared__ float red_e[4][32];
    __shared__ long long redw[8], redq[8];
    __shared__ long long red_items[4][8];
    __shared__ int red_big[4][8];
    extern __shared__ int dyn_lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
    const int gi = wid / WR;             // wave group (own K/V tile stream)
    const int rb = wid % WR;             // row block of this wave
    const int wig = wid % WR;            // wave index inside its group
    const int gtid = tid - gi * C::NT;   // thread index inside the group
    const int h32 = lane >> 5;
    const int l32 = lane & 31;
    // Transposing V reads (PV operand, d = db*32 + l32, keys 16ts + 4h32 .. +3
    // and 16ts + 8 + 4h32 .. +3): within each 16-lane group source lane s
    // reads tile row 4h32 + s/4 (+8) at columns cq*16 + 4(s%4) .. +3 of d block
    // db; lane j of the group receives 4 keys of column j.  Byte offsets for
    // ts = 0 (read 2db, then 2db+1 for the +8 rows).
    uint32_t v_lane_off[8];
    {
        const int s16 = lane & 15, cq = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int col = db * 32 + cq * 16 + 4 * (s16 & 3);
                const int row = 4 * h32 + (s16 >> 2) + 8 * hh;
                v_lane_off[2 * db + hh] = (uint32_t)(swz(row, col >> 3) + (col & 7) * 2);
            }
    }

    // the LDS tile of wave group gi (outside the pipelined paths): K then V
    auto kbuf = [&](int) { return tiles + gi * 2 * C::TILE; };
    auto vbuf = [&](int) { return tiles + gi * 2 * C::TILE + C::TILE; };

    // ---------------------------------------------------------------- plan
    // A sequence is in this launch if in_launch() says so.  Its
    // rows form ceil(rows/BM) row blocks; each row block's visible keys are cut
    // into tiles of BN keys; tiles are grouped into `splits` splits (the same
    // number for every row block of the sequence).
    plan_bind(pl, dyn_lds, a.num_seqs);
    auto widest_tiles = [&](int sl, int ql) {
        const int rows = ql * a.group;
        const int nqt = (rows + BM - 1) / BM;
        int tub = 0;
        for (int q = max(0, nqt - 2); q < nqt; ++q) {
            const int r0 = q * BM, r1 = min(rows, r0 + BM) - 1;
            const int p0 = sl - ql + r0 / a.group, p1 = sl - ql + r1 / a.group;
            const int klo = a.window > 0 ? max(0, p0 - a.window + 1) : 0;
            const int pages = p1 / kPage - klo / kPage + 1;
            tub = max(tub, (pages + PPT - 1) / PPT);
        }
        return tub;
    };
    {
        const int nthr = blockDim.x;
        long long work = 0, qtiles = 0;
        int max_tiles = 0, carry_q = 0;
        // row blocks and widest tile count of a sequence (0, 0 if not in this launch)
        auto seq_stats = [&](int sl, int ql, int& nqt, int& tub) {
            nqt = 0;
            tub = 0;
            const int rows = ql * a.group;
            if (ql > 0 && in_launch(a, rows, sl - seq_visible_lo(sl, ql, a.window))) {
                nqt = (rows + BM - 1) / BM;
                tub = widest_tiles(sl, ql);
            }
        };
        // A single sequence (verification, prefill) is planned with uniform
        // scalar code: no scans or reductions across the workgroup.
        const bool one = a.num_seqs == 1;
        int one_nqt = 0, one_tub = 0;
        if (one) {
            const int sl = a.seq_lens[0];
            int ql = checked_q_len(a, sl, a.q_lens[0]);
            if (a.checks && ql > a.num_tokens) {
                debug_flag(a.err_word, PA_CHECK_TOKENS);
                ql = 0;
            }
            seq_stats(sl, ql, one_nqt, one_tub);
            if (tid == 0) {
                pl.seq_len[0] = sl;
                pl.q_len[0] = ql;
                pl.q_off[0] = 0;
            }
            carry_q = ql;
            work = (long long)one_nqt * one_tub;
            qtiles = one_nqt;
            max_tiles = one_tub;
        }
        for (int b0 = 0; !one && b0 < a.num_seqs; b0 += nthr) {
            const int b = b0 + tid;
            int ql = 0, nqt = 0, tub = 0;
            if (b < a.num_seqs) {
                const int sl = a.seq_lens[b];
                ql = checked_q_len(a, sl, a.q_lens[b]);
                pl.seq_len[b] = sl;
                pl.q_len[b] = ql;
                seq_stats(sl, ql, nqt, tub);
                pl.aux[b] = tub;
                pl.item_base[b] = nqt;   // temporary
            }
            int tot;
            const int ex = block_exclusive_scan(ql, pl.red, &tot);
            if (b < a.num_seqs) pl.q_off[b] = carry_q + ex;
            if (a.checks && b < a.num_seqs && ql > 0 && (int64_t)carry_q + ex + ql > a.num_tokens) {
                // rows past num_tokens: skipped (and so is every later sequence)
                debug_flag(a.err_word, PA_CHECK_TOKENS);
                pl.q_len[b] = 0;
                pl.aux[b] = 0;
                pl.item_base[b] = 0;
                nqt = 0;
                tub = 0;
            }
            carry_q += tot;
            const long long w = wave_sum_i64((long long)nqt * tub), nq = wave_sum_i64(nqt);
            const int mt = wave_max_i32(tub);
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
        // Lower bounds on tiles per split: at most kMaxSplits splits, items
        // within the partial workspace.
        int tmin = max(1, (max_tiles + kMaxSplits - 1) / kMaxSplits);
        {
            long long cap = (long long)a.max_items - qtiles;
            if (cap < 1) cap = 1;
            tmin = max(tmin, (int)div_ceil_i64(work, cap));
        }
        int tps;
        const long long t_grid = a.target_items > 0 ? a.target_items : 1;
        if (a.forced_pps > 0) {
            tps = max(a.forced_pps, tmin);
        } else if (WR == 1 && qtiles * 8 <= t_grid) {
            // Few row blocks (32-row items): the size that surely fits one
            // round (below) is within t / (t - row blocks) <= 8/7 of the
            // one-round lower bound work / t, so it is taken without costing
            // the candidates (their evaluation takes every workgroup a few
            // microseconds).
            const long long c = min(div_ceil_i64(work, t_grid - qtiles), (long long)1 << 30);
            tps = (max(tmin, (int)c) + C::WK - 1) / C::WK * C::WK;
        } else {
            // The grid is one round of resident workgroups (t of them) and each
            // takes items it, it + t, ...  Try splits sized for 1..3 rounds and,
            // for a batch, a size that surely fits one round (work / (t - row
            // blocks): a sequence's items are fewer than tiles / size + 1 per
            // row block; the size for one round by work alone can overshoot the
            // grid by a few items and take two), and keep the one whose rounds x
            // largest item is smallest (split sizes are equalised within a
            // sequence).  An item's tiles are shared by the WK waves of its
            // workgroup, so an item takes ceil(tiles / WK) wave steps:
            // candidates are rounded up to a multiple of WK (the same steps,
            // fewer items and partials) and costed in wave steps.
            const long long t = a.target_items > 0 ? a.target_items : 1;
            auto round_wk = [](int c) { return (c + C::WK - 1) / C::WK * C::WK; };
            auto wave_steps = [](int tiles) { return (tiles + C::WK - 1) / C::WK; };
            constexpr int NC = 4;
            int cand[NC];
            long long items[NC];
            int big[NC];
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                cand[k] = one ? tmin : round_wk(max(tmin, (int)div_ceil_i64(work, t * (k + 1))));
                if (k == NC - 1 && !one && t > qtiles)
                    cand[k] = round_wk(max(tmin, (int)min(div_ceil_i64(work, t - qtiles), (long long)1 << 30)));
                items[k] = 0;
                big[k] = 0;
            }
            // one pass over the sequences for all candidates
            long long best = -1;
            tps = tmin;
            if (one) {
                // lane k evaluates candidate k (the divisions run once, side by
                // side); the smallest cost wins, ties to the fewer rounds
                long long cost = 0;
                int ck = tmin;
                if (lane < NC) {
                    ck = round_wk(max(tmin, (int)div_ceil_i64(work, t * (lane + 1))));
                    const int S = one_tub > 0 ? (one_tub + ck - 1) / ck : 0;
                    const long long it_k = (long long)one_nqt * S;
                    const int big_k = S > 0 ? (one_tub + S - 1) / S : 0;
                    cost = div_ceil_i64(it_k * a.num_kv_heads, t) * wave_steps(big_k);
                }
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)cost, k);
                    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((unsigned long long)cost >> 32), k);
                    const long long c_k = (long long)(((unsigned long long)hi << 32) | lo);
                    if (best < 0 || c_k < best) { best = c_k; tps = __builtin_amdgcn_readlane(ck, k); }
                }
            }
            for (int b = tid; !one && b < a.num_seqs; b += nthr) {
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
            for (int k = 0; !one && k < NC; ++k) {
                const long long it_w = wave_sum_i64(items[k]);
                const int big_w = wave_max_i32(big[k]);
                if (lane == 0) { red_items[k][wid] = it_w; red_big[k][wid] = big_w; }
            }
            if (!one) __syncthreads();
#pragma unroll
            for (int k = 0; !one && k < NC; ++k) {
                long long it_k = 0;
                int big_k = 0;
                for (int ww = 0; ww < (int)(blockDim.x / 64); ++ww) {
                    it_k += red_items[k][ww];
                    big_k = max(big_k, red_big[k][ww]);
                }
                const long long cost = div_ceil_i64(it_k * a.num_kv_heads, t) * wave_steps(big_k);
                if (best < 0 || cost < best) { best = cost; tps = cand[k]; }
            }
        }
        int carry_i = 0;
        if (one) {
            const int S = (one_tub + tps - 1) / tps;
            carry_i = one_nqt * a.num_kv_heads * S;
            if (tid == 0) {
                pl.aux[0] = S;
                pl.item_base[0] = 0;
            }
        }
        for (int b0 = 0; !one && b0 < a.num_seqs; b0 += nthr) {
            const int b = b0 + tid;
            int it = 0;
            if (b < a.num_seqs) {
                const int nqt = pl.item_base[b];
                const int S = (pl.aux[b] + tps - 1) / tps;
                it = nqt * a.num_kv_heads * S;
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
    const int64_t page_bytes = a.page_stride * C::EB;
    const int64_t tok_bytes = a.token_stride * C::EB;

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        // ------------------------------------------------------------ item geometry (uniform)
        ItemGeom ig;
        ig.b = __builtin_amdgcn_readfirstlane(item_seq(pl, a.num_seqs, it));
        ig.si.seq_len = __builtin_amdgcn_readfirstlane(pl.seq_len[ig.b]);
        ig.si.q_len = __builtin_amdgcn_readfirstlane(pl.q_len[ig.b]);
        ig.si.q_off = __builtin_amdgcn_readfirstlane(pl.q_off[ig.b]);
        ig.si.lo = seq_visible_lo(ig.si.seq_len, ig.si.q_len, a.window);
        ig.splits = __builtin_amdgcn_readfirstlane(pl.aux[ig.b]);
        {
            const int local = it - __builtin_amdgcn_readfirstlane(pl.item_base[ig.b]);
            const int per_qt = a.num_kv_heads * ig.splits;
            ig.qt = local / per_qt;
            const int rem = local - ig.qt * per_qt;
            ig.g = rem / ig.splits;
            ig.split = rem - ig.g * ig.splits;
        }
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
            const int tub = widest_tiles(ig.si.seq_len, ig.si.q_len);
            const int tpsb = (tub + ig.splits - 1) / ig.splits;
            ig.t_begin = min(ig.n_tiles, ig.split * tpsb);
            ig.t_end = min(ig.n_tiles, ig.t_begin + tpsb);
        }
        // the scales are read-only and uniform: scalar loads (a vector load
        // would sit in the same in-order counter as the tile loads issued next)
        const __attribute__((address_space(4))) float* ksc = (const __attribute__((address_space(4))) float*)a.kv_scale;
        const float kscale = C::FP8 ? ksc[ig.g] : 1.0f;
        const float vscale = C::FP8 ? ksc[a.num_kv_heads + ig.g] : 1.0f;
        const float s2 = a.scale * kLog2e * kscale;
        const int32_t* bt = a.block_table + (int64_t)ig.b * a.bt_stride;
        const bool direct = (ig.splits == 1);
        const int64_t head_off = kv_offset(0, ig.g, 0, a.page_stride, a.head_stride, a.token_stride) * C::EB;

        // ------------------------------------------------------------ this lane's query row
        const int row_l = rb * 32 + l32;
        const int row_g = ig.row0 + row_l;
        const bool row_ok = row_l < ig.rows;
        const int tok_i = row_ok ? row_g / a.group : 0;
        const int pos_r = row_ok ? ig.si.seq_len - ig.si.q_len + tok_i : -1;
        const int lo_r = (a.window > 0) ? pos_r - a.window + 1 : 0;
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
        float m_run = kNegInf, m_true = kNegInf, l_exact = 0.f;
        // Derived from m_run and m_true, refreshed only when one of them moves:
        // the exponent offset -m_run (0 while a row has seen no visible key)
        // and the split threshold kSplitBelow * 2^(m_true - m_run).
        float neg_m = 0.f, split_thr = kSplitBelow;

        // ------------------------------------------------------------ tile staging
        // Tile t covers logical pages pg_first + t*PPT ...; a page past the
        // visible range reads the last visible page (in bounds) and its keys
        // are dead.  Key k of a tile is live iff it lies in [lo, seq_len).
        // The block table is read-only while the kernel runs: read it through
        // the constant address space so the wave-uniform page ids come from
        // scalar loads, which do not wait behind the asynchronous tile loads.
        const __attribute__((address_space(4))) int32_t* bt_c =
            (const __attribute__((address_space(4))) int32_t*)bt;
        auto tile_pid = [&](int t, int p) {
            const int pg = __builtin_amdgcn_readfirstlane(min(ig.pg_first + t * PPT + p, ig.pg_end - 1));
            return chunk_page(bt_c, pg, a);
        };
        auto key_pos = [&](int t, int key) { return (ig.pg_first + t * PPT) * kPage + key; };
        auto row_src = [&](const uint8_t* base, const int (&pid)[PPT], int key) -> const uint8_t* {
            return base + (int64_t)pid[key / kPage] * page_bytes + head_off + (int64_t)(key % kPage) * tok_bytes;
        };
        // 16-bit caches: 1 KB loads of tile rows (asynchronous into LDS on the
        // pipelined path, through registers at 32-row items).  Load i of a
        // group covers tile rows 4i .. 4i+3; lane l fills row 4i + l/16,
        // physical chunk l%16, which holds logical chunk (l%16) ^ (row & 15).
        // Per-lane byte offset inside its page for load ii (constant per item).
        uint32_t dma_off[C::DMA_PER_WAVE];
#pragma unroll
        for (int ii = 0; ii < C::DMA_PER_WAVE; ++ii) {
            const int row = 4 * (ii * WR + wig) + (lane >> 4);
            const int c = (lane & 15) ^ swz_key(row);
            dma_off[ii] = (uint32_t)(head_off + (int64_t)(row % kPage) * tok_bytes + c * 16);
        }
        // WR = 1: the item's page ids are staged in LDS when they fit (set
        // before the tile loop), so a tile's loads do not wait behind a
        // scalar block-table load that missed its cache.
        bool pid_staged = false;
        auto tile_pids = [&](int t, int (&pid)[PPT]) {
            if constexpr (WR == 1) {
                static_assert(PPT == 2, "tiles of two pages");
                if (pid_staged) {
                    const int2 w = *reinterpret_cast<const int2*>(ipid + (t - ig.t_begin) * PPT);
                    pid[0] = __builtin_amdgcn_readfirstlane(w.x);
                    pid[1] = __builtin_amdgcn_readfirstlane(w.y);
                    return;
                }
            }
#pragma unroll
            for (int p = 0; p < PPT; ++p) pid[p] = tile_pid(t, p);
        };
        // int8 row scales: the scale of key slot `slot` of virtual page pid
        // (K; V is rs_v further)
        auto row_scale_ptr = [&](int pid, int slot) {
            return a.row_scale + (int64_t)pid * a.rs_page + (int64_t)ig.g * a.rs_head + (int64_t)slot * a.rs_tok;
        };
        // int8: the wave group's scale array (32-row items: the tile's K
        // scales, then its V scales)
        float* tsc_group = tscale + (C::FSTAGE ? 0 : gi * 2 * BN);
        // fp8 staging (FSTAGE): async load i of a raw K or V tile covers rows
        // 8i .. 8i+7 (128 B each), lane l row 8i + l/8.  Rows are stored with
        // 16-byte unit u at position u ^ (row & 7), so the operand reads (one
        // unit of many rows at once) spread over the banks: lane l brings unit
        // (l%8) ^ ((l/8) & 7).  A wave's two slots: [K 4 KB | V 4 KB] each.
        uint32_t raw_off[C::FSTAGE ? 4 : 1];
        if constexpr (C::FSTAGE) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * i + (lane >> 3);
                raw_off[i] = (uint32_t)(head_off + (int64_t)(row % kPage) * tok_bytes +
                                        (((lane & 7) ^ ((lane >> 3) & 7)) << 4));
            }
        }
        // VREG: one tile's V rows in registers, in the staging layout (load i,
        // lane l: the 16 bytes the asynchronous path would put at i*1024 + 16*l)
        u32x4_t vreg[C::VREG ? 4 : 1];
        auto v_load = [&](int t) {
            if constexpr (C::VREG) {
                int pid[PPT];
                tile_pids(t, pid);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vreg[i] = load_b128(vbase + (int64_t)pid[(8 * i) / kPage] * page_bytes + raw_off[i]);
            }
        };
        auto v_store = [&](auto slot_c) {
            if constexpr (C::VREG) {
                const uint32_t v32 = (uint32_t)(uintptr_t)(lds_void_t*)(stage + gi * 4 * C::RAW_TILE +
                                                                       decltype(slot_c)::value * 2 * C::RAW_TILE +
                                                                       C::RAW_TILE) + 16 * lane;
                lds_store_b128<0>(v32, vreg[0]);
                lds_store_b128<1024>(v32, vreg[1]);
                lds_store_b128<2048>(v32, vreg[2]);
                lds_store_b128<3072>(v32, vreg[3]);
            }
        };
        auto raw_dma = [&](auto slot_c, int t) {
            if constexpr (C::FSTAGE) {
                uint8_t* st = stage + gi * 4 * C::RAW_TILE + decltype(slot_c)::value * 2 * C::RAW_TILE;
                int pid[PPT];
                tile_pids(t, pid);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t pb = (int64_t)pid[(8 * i) / kPage] * page_bytes;
                    async_load16(kbase + pb + raw_off[i], (lds_void_t*)(st + i * 1024));
                    if constexpr (!C::VREG)
                        async_load16(vbase + pb + raw_off[i], (lds_void_t*)(st + C::RAW_TILE + i * 1024));
                }
                if constexpr (C::INT8) {
                    // lanes 0..31: K scales of keys 0..31; lanes 32..63: their V scales
                    const int key = lane & 31;
                    const float* src = row_scale_ptr(pid[key / kPage], key % kPage) + (lane >= 32 ? a.rs_v : 0);
                    async_load4(src, (lds_void_t*)(tscale + (gi * 2 + decltype(slot_c)::value) * 2 * BN));
                }
            }
        };
        // Zero the V rows of dead keys (only tiles that touch a range edge).
        auto zero_dead_v_in = [&](int t, uint8_t* vb) {
            const int k0 = key_pos(t, 0);
            const bool edge = (k0 < ig.si.lo) || (k0 + BN > ig.si.seq_len) || (ig.pg_first + (t + 1) * PPT > ig.pg_end);
            if (!edge) return false;
            for (int e = gtid; e < BN * 16; e += C::NT) {
                const int key = e >> 4, c = e & 15;
                const int j = k0 + key;
                const bool live = (j >= ig.si.lo) && (j < ig.si.seq_len) && (ig.pg_first + t * PPT + key / kPage < ig.pg_end);
                if (!live) *reinterpret_cast<u32x4_t*>(vb + swz(key, c)) = u32x4_t{0u, 0u, 0u, 0u};
            }
            return true;
        };
        auto zero_dead_v = [&](int t, int buf) { return zero_dead_v_in(t, vbuf(buf)); };
        // Synchronise the wave group after LDS writes (WR == 1: one wave).
        auto group_sync = [&]() {
            if constexpr (WR == 1) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wave's LDS writes are done
            else __syncthreads();
        };

        // ------------------------------------------------------------ pieces of one tile
        // Scores stay unscaled (s2 > 0 preserves the order): the reference max
        // m_run is kept in scaled units and p = 2^(s*s2 - m_run) is one fma and
        // one exp.  Masked keys become -inf by select (only tiles that touch a
        // range edge or the causal diagonal).
        auto mask_scores = [&](int t, f32x16_t (&S)[C::NB]) {
            const int key0 = key_pos(t, 0);
            const bool full = (key0 >= w_lomax) && (key0 + BN - 1 <= w_pmin) && (key0 >= ig.si.lo) &&
                              (key0 + BN <= ig.si.seq_len) && (ig.pg_first + (t + 1) * PPT <= ig.pg_end);
            if (!full) {
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int j = key0 + nb * 32 + 8 * (i / 4) + 4 * h32 + (i % 4);
                        const bool vis = (j <= pos_r) && (j >= lo_r) && (j >= ig.si.lo) && (j < ig.si.seq_len);
                        S[nb][i] = vis ? S[nb][i] : kNegInf;
                    }
            }
        };
        // Row max of the tile; lazy rescale: the reference max m_run moves (to
        // the exact max) only when a score passes it by 2^kTau, so p <= 2^kTau
        // and the accumulators are rescaled a handful of times per row.
        auto raise_max = [&](const f32x16_t (&S)[C::NB]) {
            float tmax = kNegInf;
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmax = fmax_nan(tmax, S[nb][i]);
            tmax = half_swap_max(tmax) * s2;
            // m_true <= m_run + kTau holds on entry, so a rescale needs a new maximum
            if (wave_any(tmax > m_true)) {
                m_true = fmax_nan(m_true, tmax);
                if (wave_any(tmax > m_run + kTau)) {
                    const float mn = m_true;
                    const float al = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - mn);
                    m_run = mn;
                    neg_m = (m_run == kNegInf) ? 0.f : -m_run;
                    l_exact *= al;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) o_acc[db][i] *= al;
                }
                split_thr = kSplitBelow * ((m_run == kNegInf) ? 1.f : fast_exp2(m_true - m_run));
            }
        };
        // int8: the 16 row scales of this lane's keys in a tile (key
        // nb*32 + 8*(i/4) + 4*h32 + i%4 for score i of block nb) from the
        // tile's scale array in LDS.
        auto lane_scales = [&](const float* base, float (&out)[C::NB][16]) {
            asm volatile("" ::: "memory");   // after the waits for the array's loads and stores
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(base + nb * 32 + 8 * q + 4 * h32);
                    out[nb][4 * q] = v.x; out[nb][4 * q + 1] = v.y; out[nb][4 * q + 2] = v.z; out[nb][4 * q + 3] = v.w;
                }
        };
        // int8: each key's own K scale multiplies its score (before masking,
        // which replaces a dead key's NaN by select).
        auto apply_kscale = [&](f32x16_t (&S)[C::NB], const float* ksc) {
            float k[C::NB][16];
            lane_scales(ksc, k);
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) S[nb][i] *= k[nb][i];
        };
        // P = 2^(s*s2 - m_run) rounded to the P.V operand type; while a row has
        // few effective keys (weight sum small against its largest weight) the
        // rounding error of P goes into pl as a second operand.  int8: the
        // weight that meets V is p times the key's V scale (vsc; 0 for dead
        // keys), the normaliser sums p.
        auto exp_pack = [&](f32x16_t (&S)[C::NB], u32x4_t (&pb)[C::TS], u32x4_t (&pl)[C::TS],
                            const float* vsc = nullptr) {
            // a row that has seen no visible key yet keeps m_run = -inf; its p are 0
            const float nm = neg_m;
            float vs[C::INT8 ? C::NB : 1][16];
            if constexpr (C::INT8) lane_scales(vsc, vs);
#pragma unroll
            for (int ts = 0; ts < C::TS; ++ts) {
                const int nb = ts / 2, i0 = 8 * (ts % 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = fast_exp2(fmaf(S[nb][i0 + 2 * j], s2, nm));
                    const float p1 = fast_exp2(fmaf(S[nb][i0 + 2 * j + 1], s2, nm));
                    S[nb][i0 + 2 * j] = p0;
                    S[nb][i0 + 2 * j + 1] = p1;
                    l_exact += p0 + p1;
                    if constexpr (C::INT8)
                        pb[ts][j] = pack2<C::PVT>(p0 * vs[nb][i0 + 2 * j], p1 * vs[nb][i0 + 2 * j + 1]);
                    else
                        pb[ts][j] = pack2<C::PVT>(p0, p1);
                }
            }
            // one-byte caches: P's f16 rounding (relative 2^-11) stays far
            // inside the error the cache format already carries, so no split
            const bool split = C::PSPLIT || (!C::BYTE && wave_any(l_exact < split_thr));
            if (split) {
#pragma unroll
                for (int ts = 0; ts < C::TS; ++ts) {
                    const int nb = ts / 2, i0 = 8 * (ts % 2);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pl[ts][j] = pack2<C::PVT>(S[nb][i0 + 2 * j] - unpack_lo<C::PVT>(pb[ts][j]),
                                                  S[nb][i0 + 2 * j + 1] - unpack_hi<C::PVT>(pb[ts][j]));
                }
            }
            return split;
        };
        // O^T += V^T P^T; V^T operands by transposing reads.  Row 16ts + r0 has
        // the same swizzle key for every ts, so one set of eight lane addresses
        // serves the whole tile with ts in the offset.
        // One pass of O^T += V^T P^T over a tile (P as TS packed key steps);
        // va holds this lane's read addresses, OFF the tile's offset from them.
        auto pv_frags = [&](const uint32_t (&va)[8], auto off_c, const u32x4_t (&p)[C::TS]) {
            constexpr int OFF = decltype(off_c)::value;
            // V fragments of key steps 2u and 2u+1 in one batch of reads
            static_assert(C::TS % 2 == 0, "key steps come in pairs");
            static_for<C::TS / 2>([&](auto u_c) {
                constexpr int u = decltype(u_c)::value;
                u32x2_t r0[8], r1[8];
                lds_read_tr16_x16<OFF + (2 * u) * 16 * kRowBytes, OFF + (2 * u + 1) * 16 * kRowBytes>(va, r0, r1);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const u32x2_t(&r)[8] = h ? r1 : r0;
                        o_acc[db] = mma32<C::PVT>(u32x4_t{r[2 * db][0], r[2 * db][1], r[2 * db + 1][0], r[2 * db + 1][1]},
                                                  p[2 * u + h], o_acc[db]);
                    }
            });
        };
        // P's rounding error, when it is used, takes a second pass over the V
        // fragments (re-read from LDS): one branch per tile, and the plain pass
        // holds no extra registers.
        auto pv = [&](uint32_t vb32, const u32x4_t (&pb)[C::TS], const u32x4_t (&pl)[C::TS], bool split) {
            uint32_t va[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) va[k] = vb32 + v_lane_off[k];
            pv_frags(va, std::integral_constant<int, 0>{}, pb);
            if (split) pv_frags(va, std::integral_constant<int, 0>{}, pl);
        };

        // ------------------------------------------------------------ compute one tile
        auto compute_tile = [&](int t, const uint8_t* kb, const uint8_t* vb) {
            // S^T = K Q^T: all K fragments of the tile are read first, then the
            // MFMAs run back to back (the scheduling barriers keep the reads
            // grouped instead of one read / wait / MFMA at a time).
            u32x4_t kf[C::NB][C::KS];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int s = 0; s < C::KS; ++s)
                    kf[nb][s] = *reinterpret_cast<const u32x4_t*>(kb + swz(nb * 32 + l32, 2 * s + h32));
            f32x16_t sacc[C::NB];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[nb][i] = 0.f;
#pragma unroll
                for (int s = 0; s < C::KS; ++s) sacc[nb] = mma32<QT>(kf[nb][s], qreg[s], sacc[nb]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, C::NB * C::KS, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, C::NB * C::KS, 0);   // MFMAs
            if constexpr (C::INT8) apply_kscale(sacc, tsc_group);
            mask_scores(t, sacc);
            raise_max(sacc);
            u32x4_t pb[C::TS], pl[C::TS];
            const bool split = exp_pack(sacc, pb, pl, C::INT8 ? tsc_group + BN : nullptr);
            pv((uint32_t)(uintptr_t)(lds_void_t*)vb, pb, pl, split);
        };

        // ------------------------------------------------------------ tile loop
        const int my_first = ig.t_begin + gi;
        const int n_iter = (ig.t_end - ig.t_begin + C::WK - 1) / C::WK;
        if constexpr (WR == 1) {
            // every tile a wave loads (clamped to the item's last) is staged
            const int n_pid = (ig.t_end - ig.t_begin) * PPT;
            pid_staged = n_pid <= C::PID_CAP;
            const int pid0 = ig.pg_first + ig.t_begin * PPT;
            if (pid_staged)
                for (int k = tid; k < n_pid; k += blockDim.x) ipid[k] = chunk_page(bt, min(pid0 + k, ig.pg_end - 1), a);
            __syncthreads();
        }
        if constexpr (C::PIPE) {
            // Iteration k holds tile k's scores (cur) and tile k+1's K
            // fragments (kf).  In order: the scores of tile k+1 go to the
            // matrix cores; tile k's V fragments are read from LDS (the read
            // waits while those MFMAs run); the VALU turns tile k's scores into
            // P; P.V of tile k goes to the matrix cores; past the barrier that
            // certifies tile k+2 for every wave (and frees tile k's buffers),
            // tile k+LEAD is requested into them and tile k+2's K fragments
            // are read (that read waits while P.V runs).  Tile k's K and V sit
            // in buffer k % NKB from its load (issued at iteration k - LEAD)
            // until its V fragments are read in iteration k.  The second wave
            // of each SIMD (waves NW/2 ..) issues its P.V after the barrier.
            // Page ids of the item's tiles and of the LEAD + 1 tiles prefetched
            // or fetched past its end (those read the last visible page: in
            // bounds, unused), staged in LDS when they fit; otherwise scalar
            // loads per tile.
            const int n_pid = (ig.t_end - ig.t_begin + C::LEAD + 1) * PPT;
            const bool staged = n_pid <= C::PID_CAP;
            const int pid0 = ig.pg_first + ig.t_begin * PPT;
            if (staged)
                for (int k = tid; k < n_pid; k += blockDim.x) ipid[k] = chunk_page(bt, min(pid0 + k, ig.pg_end - 1), a);
            __syncthreads();
            // tiles t_begin + k with k in [k_live, k_live + n_live) have no dead V rows
            int k_live, n_live;
            {
                const int kb0 = ig.pg_first * kPage;
                const int key_b = min(ig.si.seq_len, ig.pg_end * kPage);
                const int t_lo = ig.si.lo <= kb0 ? 0 : (ig.si.lo - kb0 + BN - 1) / BN;
                const int t_hi = key_b < kb0 ? 0 : (key_b - kb0) / BN;
                k_live = t_lo - ig.t_begin;
                n_live = max(0, t_hi - t_lo);
            }
            const uint32_t ring32 = (uint32_t)(uintptr_t)(lds_void_t*)tiles;
            // page ids of tile k (its two pages), fetched a step before the
            // loads that use them so the fetch's round trip is off the path
            // between the barrier and the loads
            auto pid_fetch = [&](int k) -> int2 {
                static_assert(PPT == 2, "tiles of two pages");
                if (staged) return *reinterpret_cast<const int2*>(ipid + k * PPT);
                const int t = min(ig.t_begin + k, ig.t_end - 1);
                return make_int2(tile_pid(t, 0), tile_pid(t, 1));
            };
            // one-byte caches: wave wig brings tile rows 4 wig .. 4 wig + 3
            // (8 bytes of K and of V per lane, 8-element chunk lane % 16 of
            // row 4 wig + lane / 16) through register set R, then stores them
            // widened to 16 bits at their swizzled place in the tile's slot
            // (int8: lanes 0-7 also bring the K (lanes 0-3) and V (4-7) row
            // scales of the wave's four rows; a dead key's V scale is stored as 0)
            [[maybe_unused]] u32x2_t rk[2], rv[2];
            [[maybe_unused]] float rsc[2] = {0.f, 0.f};
            [[maybe_unused]] uint32_t boff = 0, lds_off = 0;
            const int skey = 4 * wig + (lane & 3);   // int8: the key of this lane's scale
            if constexpr (C::BYTE) {
                const int key = 4 * wig + (lane >> 4), c8 = lane & 15;
                boff = (uint32_t)(head_off + (int64_t)(key % kPage) * tok_bytes + c8 * 8);
                lds_off = (uint32_t)swz(key, c8);
            }
            auto reg_load = [&](auto r_c, int2 w) {
                constexpr int R = decltype(r_c)::value;
                static_assert(PPT == 2 && C::NW == 8, "rows 0-15 come from the first page, 16-31 the second");
                const int pid = __builtin_amdgcn_readfirstlane(wig < 4 ? w.x : w.y);
                const int64_t pb = (int64_t)pid * page_bytes;
                rk[R] = load_b64(kbase + pb + boff);
                rv[R] = load_b64(vbase + pb + boff);
                if constexpr (C::INT8) {
                    if (lane < 8)
                        rsc[R] = __builtin_nontemporal_load(row_scale_ptr(pid, skey % kPage) + (lane >= 4 ? a.rs_v : 0));
                }
            };
            auto reg_store = [&](auto r_c, int k) {
                constexpr int R = decltype(r_c)::value;
                uint8_t* kb = tiles + (k % C::NKB) * C::TILE;
                uint8_t* vb = tiles + (C::NKB + k % C::NVB) * C::TILE;
                *reinterpret_cast<u32x4_t*>(kb + lds_off) = widen8<QT, KVT>(rk[R]);
                *reinterpret_cast<u32x4_t*>(vb + lds_off) = widen8<C::PVT, KVT>(rv[R]);
                if constexpr (C::INT8) {
                    if (lane < 8) {
                        const int j = key_pos(ig.t_begin + k, skey);
                        const bool live = (j >= ig.si.lo) && (j < ig.si.seq_len) &&
                                          (ig.pg_first + (ig.t_begin + k) * PPT + skey / kPage < ig.pg_end);
                        tscale[(k % C::NKB) * 2 * BN + (lane >= 4 ? BN : 0) + skey] =
                            (lane >= 4 && !live) ? 0.f : rsc[R];
                    }
                }
            };
            auto dma_pipe = [&](int k, int2 w) {
                const int pid[PPT] = {__builtin_amdgcn_readfirstlane(w.x), __builtin_amdgcn_readfirstlane(w.y)};
                uint8_t* kb = tiles + (k % C::NKB) * C::TILE;
                uint8_t* vb = tiles + (C::NKB + k % C::NVB) * C::TILE;
#pragma unroll
                for (int ii = 0; ii < C::DMA_PER_WAVE; ++ii) {
                    const int i = ii * WR + wig;
                    const int64_t pb = (int64_t)pid[(4 * i) / kPage] * page_bytes;
                    async_load16(kbase + pb + dma_off[ii], (lds_void_t*)(kb + i * 1024));
                    async_load16(vbase + pb + dma_off[ii], (lds_void_t*)(vb + i * 1024));
                }
            };
            // This lane's LDS read addresses at ring offset 0: K fragments (row
            // l32, chunks 2*s8 + h32) and the transposing V reads.  A buffer's
            // offset from them is an immediate of the read instructions.
            static_assert(C::NB == 1 && C::NKB == C::NVB && C::TS == 2, "one 32-key block per tile, rings of equal length");
            uint32_t ka[8], va[8];
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) ka[s8] = ring32 + (uint32_t)swz(l32, 2 * s8 + h32);
#pragma unroll
            for (int k = 0; k < 8; ++k) va[k] = ring32 + (uint32_t)(C::NKB * C::TILE) + v_lane_off[k];
            // S^T of a tile = K Q^T: eight MFMAs accumulate over the head dimension.
            auto qk_mma = [&](const u32x4_t (&kf)[C::KS], f32x16_t (&S)[C::NB]) {
#pragma unroll
                for (int i = 0; i < 16; ++i) S[0][i] = 0.f;
#pragma unroll
                for (int s8 = 0; s8 < C::KS; ++s8) S[0] = mma32<QT>(kf[s8], qreg[s8], S[0]);
            };
            // O^T += V^T P^T over one tile from V fragments already in registers
            // (r0: key step 0, r1: key step 1)
            auto pv_mma = [&](const u32x2_t (&r0)[8], const u32x2_t (&r1)[8], const u32x4_t (&p)[C::TS]) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const u32x2_t(&r)[8] = h ? r1 : r0;
                        o_acc[db] = mma32<C::PVT>(u32x4_t{r[2 * db][0], r[2 * db][1], r[2 * db + 1][0], r[2 * db + 1][1]},
                                                  p[h], o_acc[db]);
                    }
            };
            // dead V rows of tile k (range edges only) are zeroed in its buffer
            auto zero_dead_v_pipe = [&](int k) {
                if ((unsigned)(k - k_live) < (unsigned)n_live) return false;
                const int t = ig.t_begin + k;
                const int k0 = key_pos(t, 0);
                uint8_t* vb = tiles + (C::NKB + k % C::NVB) * C::TILE;
                for (int e = tid; e < BN * 16; e += blockDim.x) {
                    const int key = e >> 4, c = e & 15;
                    const int j = k0 + key;
                    const bool live = (j >= ig.si.lo) && (j < ig.si.seq_len) && (ig.pg_first + t * PPT + key / kPage < ig.pg_end);
                    if (!live) *reinterpret_cast<u32x4_t*>(vb + swz(key, c)) = u32x4_t{0u, 0u, 0u, 0u};
                }
                return true;
            };
            // The second wave of each SIMD (waves 4-7) issues its P.V after the
            // barrier instead of before it, so between two barriers the two
            // waves of a SIMD are a phase apart: one's matrix ops meet the
            // other's LDS reads and softmax.
            const bool late_pv = wid >= C::NW / 2;
            const int n_it = ig.t_end - ig.t_begin;
            if (n_it > 0) {
                static_assert(C::LEAD == C::NKB, "tile k+LEAD reuses tile k's buffers");
                using R0 = std::integral_constant<int, 0>;
                using R1 = std::integral_constant<int, 1>;
                int2 pid_nx;
                if constexpr (C::BYTE) {
                    // tiles 0 and 1 stored, 2 and 3 in registers (tile t in set t % 2)
                    reg_load(R0{}, pid_fetch(0));
                    reg_load(R1{}, pid_fetch(1));
                    reg_store(R0{}, 0);
                    reg_store(R1{}, 1);
                    reg_load(R0{}, pid_fetch(2));
                    reg_load(R1{}, pid_fetch(3));
                    pid_nx = pid_fetch(4);
                    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wave's stores are done
                    barrier_no_fence();
                } else {
#pragma unroll
                    for (int k = 0; k < C::LEAD; ++k) dma_pipe(k, pid_fetch(k));
                    pid_nx = pid_fetch(C::LEAD);
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm((C::LEAD - 2) * 2 * C::DMA_PER_WAVE));   // tiles 0 and 1 landed
                    __syncthreads();
                }
                {
                    const bool z0 = zero_dead_v_pipe(0);
                    const bool z1 = zero_dead_v_pipe(1);
                    if (z0 || z1) __syncthreads();
                }
                u32x4_t kf[C::KS];
                f32x16_t S0[C::NB], S1[C::NB];
                lds_read_b128_x8<0>(ka, kf);
                qk_mma(kf, S0);
                lds_read_b128_x8<C::TILE>(ka, kf);
                auto step = [&](auto j_c, int k, f32x16_t (&cur)[C::NB], f32x16_t (&nxt)[C::NB]) {
                    constexpr int J = decltype(j_c)::value;
                    constexpr int VOFF = J * C::TILE;                             // V of tile k
                    constexpr int KOFF = ((J + 2) % C::NKB) * C::TILE;            // K of tile k+2
                    qk_mma(kf, nxt);                                              // scores of tile k+1
                    __builtin_amdgcn_sched_barrier(0);
                    u32x2_t vr0[8], vr1[8];
                    lds_read_tr16_x16<VOFF, VOFF + 16 * kRowBytes>(va, vr0, vr1);
                    [[maybe_unused]] const float* tsc_k = tscale + (J % C::NKB) * 2 * BN;   // int8: tile k's scales
                    if constexpr (C::INT8) apply_kscale(cur, tsc_k);
                    mask_scores(ig.t_begin + k, cur);
                    raise_max(cur);
                    u32x4_t pb[C::TS], pl[C::TS];
                    const bool split = exp_pack(cur, pb, pl, C::INT8 ? tsc_k + BN : nullptr);
                    if (!late_pv) {
                        pv_mma(vr0, vr1, pb);
                        if (split) pv_mma(vr0, vr1, pl);
                    }
                    if constexpr (C::BYTE) {
                        // tile k+2 (in registers since iteration k-2) into the
                        // slot tile k-4 held; tile k+4 requested into its set
                        using RJ = std::integral_constant<int, J % 2>;
                        reg_store(RJ{}, k + 2);
                        reg_load(RJ{}, pid_nx);
                        pid_nx = pid_fetch(k + 5);
                        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wave's stores are done
                        barrier_no_fence();                       // ... and every wave's
                        if (zero_dead_v_pipe(k + 2)) __syncthreads();
                    } else {
                        // tile k+2 landed for this wave (tile k+3 may still be in
                        // flight) ...
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm((C::LEAD - 3) * 2 * C::DMA_PER_WAVE));
                        // ... and for every wave; every wave has read tile k's V
                        // (and, an iteration earlier, its K): its buffers take tile k+LEAD
                        barrier_no_fence();
                        if (zero_dead_v_pipe(k + 2)) __syncthreads();
                        dma_pipe(k + C::LEAD, pid_nx);
                        pid_nx = pid_fetch(k + C::LEAD + 1);
                    }
                    if (late_pv) {
                        pv_mma(vr0, vr1, pb);
                        if (split) pv_mma(vr0, vr1, pl);
                    }
                    lds_read_b128_x8<KOFF>(ka, kf);
                    __builtin_amdgcn_sched_barrier(0);
                };
                // the loop is unrolled over the ring (offsets are immediates)
                using I0 = std::integral_constant<int, 0>;
                using I1 = std::integral_constant<int, 1>;
                using I2 = std::integral_constant<int, 2>;
                using I3 = std::integral_constant<int, 3>;
                using I4 = std::integral_constant<int, 4>;
                using I5 = std::integral_constant<int, 5>;
                static_assert(C::NKB == 6, "the loop below is unrolled six times");
                int k = 0;
                for (; k + 6 <= n_it; k += 6) {
                    step(I0{}, k, S0, S1);
                    step(I1{}, k + 1, S1, S0);
                    step(I2{}, k + 2, S0, S1);
                    step(I3{}, k + 3, S1, S0);
                    step(I4{}, k + 4, S0, S1);
                    step(I5{}, k + 5, S1, S0);
                }
                if (k < n_it) step(I0{}, k, S0, S1);
                if (k + 1 < n_it) step(I1{}, k + 1, S1, S0);
                if (k + 2 < n_it) step(I2{}, k + 2, S0, S1);
                if (k + 3 < n_it) step(I3{}, k + 3, S1, S0);
                if (k + 4 < n_it) step(I4{}, k + 4, S0, S1);
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // the clamped prefetches past the end
                __syncthreads();
            }
        } else if constexpr (!C::BYTE) {
            // Register-staged tiles (32-row items, 16-bit caches): the next tile's K and V rows are in flight
            // in registers while this one is computed from the wave's LDS
            // buffer; then they are written there and the tile after is
            // requested.  Every load is issued, past the end too (clamped).
            static_assert(WR == 1, "one wave per tile stream");
            u32x4_t rk[C::DMA_PER_WAVE], rv[C::DMA_PER_WAVE];
            auto reg_load = [&](int t) {
                int pid[PPT];
                tile_pids(t, pid);
#pragma unroll
                for (int ii = 0; ii < C::DMA_PER_WAVE; ++ii) {
                    const int64_t pb = (int64_t)pid[(4 * ii) / kPage] * page_bytes;
                    rk[ii] = load_b128(kbase + pb + dma_off[ii]);
                    rv[ii] = load_b128(vbase + pb + dma_off[ii]);
                }
            };
            const uint32_t kb32 = (uint32_t)(uintptr_t)(lds_void_t*)kbuf(0);
            auto reg_store = [&]() {
#pragma unroll
                for (int ii = 0; ii < C::DMA_PER_WAVE; ++ii)
                {
                    lds_store_b128<0>(kb32 + ii * 1024 + lane * 16, rk[ii]);
                    lds_store_b128<C::TILE>(kb32 + ii * 1024 + lane * 16, rv[ii]);
                }
            };
            if (n_iter > 0) {
                reg_load(min(my_first, ig.t_end - 1));
                for (int itn = 0; itn < n_iter; ++itn) {
                    const int t = my_first + itn * C::WK;
                    reg_store();
                    reg_load(min(t + C::WK, ig.t_end - 1));
                    if (t < ig.t_end) {
                        if (zero_dead_v(t, 0)) group_sync();
                        compute_tile(t, kbuf(0), vbuf(0));
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
        } else if constexpr (C::FSTAGE) {
            // Tile k of this wave (tile my_first + k*WK) sits in staging slot
            // k % 2, loaded two tiles ahead; its K and V operand fragments are
            // read raw and widened in registers right at their matrix ops, so
            // the slot is free once the tile is done.  The small LDS footprint
            // leaves room for two workgroups per CU, whose waves hide each
            // other's latencies.  Every load is issued, past the end too
            // (clamped to the last tile: in bounds, unused); an odd count ends
            // with one uncomputed step.
            if (n_iter > 0) {
                using I0 = std::integral_constant<int, 0>;
                using I1 = std::integral_constant<int, 1>;
                static_assert(C::NB == 1 && C::TS == 2 && C::DB == 4 && C::RAW_TILE == 4096, "raw read offsets");
                uint8_t* st = stage + gi * 4 * C::RAW_TILE;
                const uint32_t st32 = (uint32_t)(uintptr_t)(lds_void_t*)st;
                // K fragment s of lane (l32, h32): row l32, unit s, half h32
                uint32_t ka[8];
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) ka[s8] = st32 + l32 * 128 + ((s8 ^ (l32 & 7)) << 4) + h32 * 8;
                // V^T fragment (ts, db): in each 16 lanes, lanes 2r, 2r+1 point
                // at the two halves of unit 2db + (lane/16)%2 of key row kr(r) of
                // step 0, where kr(r) = 4 (lane/32) + r for r < 4 and
                // 4 (lane/32) + r + 4 above (the key order of P's packed pairs)
                uint32_t va[4];
                {
                    const int s16 = lane & 15, r = s16 >> 1, hh = s16 & 1, g16 = lane >> 4;
                    const int krow = 4 * (g16 >> 1) + (r < 4 ? r : r + 4);
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        const int u = 2 * db + (g16 & 1);
                        va[db] = st32 + krow * 128 + ((u ^ (krow & 7)) << 4) + hh * 8;
                    }
                }
                auto tile_of = [&](int k) { return my_first + k * C::WK; };
                // issue order: K(0), V(0), K(1); a step k finds K(k), V(k) and
                // K(k+1) in flight and waits for the first two
                raw_dma(I0{}, min(tile_of(0), ig.t_end - 1));
                v_load(min(tile_of(0), ig.t_end - 1));
                raw_dma(I1{}, min(tile_of(1), ig.t_end - 1));
                u32x4_t pb[C::TS], pl[C::TS];
                auto fstep = [&](auto j_c, int k) {
                    constexpr int J = decltype(j_c)::value;
                    const int t = tile_of(k);
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::RAW_DMA));   // slot J's tile is the older in flight
                    if constexpr (C::VREG) {
                        // this tile's V rows into the slot (the stores take their
                        // data at issue), then the next tile's V rows go out
                        v_store(j_c);
                        v_load(min(tile_of(k + 1), ig.t_end - 1));
                    }
                    if (t < ig.t_end) {
                        // dead keys' V rows (range edges only) are zeroed in the slot
                        {
                            const int k0 = key_pos(t, 0);
                            const bool edge = (k0 < ig.si.lo) || (k0 + BN > ig.si.seq_len) ||
                                              (ig.pg_first + (t + 1) * PPT > ig.pg_end);
                            if (edge) {
                                uint8_t* vrows = st + J * 2 * C::RAW_TILE + C::RAW_TILE;
                                for (int e = gtid; e < BN * 8; e += C::NT) {
                                    const int key = e >> 3, c = e & 7;
                                    const int j = k0 + key;
                                    const bool live = (j >= ig.si.lo) && (j < ig.si.seq_len) &&
                                                      (ig.pg_first + t * PPT + key / kPage < ig.pg_end);
                                    if (!live) *reinterpret_cast<u32x4_t*>(vrows + key * 128 + c * 16) = u32x4_t{0u, 0u, 0u, 0u};
                                    // int8: a dead key's V scale (maybe NaN) becomes 0
                                    if constexpr (C::INT8)
                                        if (!live && c == 0) tscale[(gi * 2 + J) * 2 * BN + BN + key] = 0.f;
                                }
                                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                            }
                        }
                        u32x2_t kr[8];
                        lds_read_raw_k<J>(ka, kr);
                        f32x16_t S[C::NB];
#pragma unroll
                        for (int i = 0; i < 16; ++i) S[0][i] = 0.f;
#pragma unroll
                        for (int s8 = 0; s8 < C::KS; ++s8) S[0] = mma32<QT>(widen8<QT, KVT>(kr[s8]), qreg[s8], S[0]);
                        const float* tsc_slot = tscale + (gi * 2 + J) * 2 * BN;
                        if constexpr (C::INT8) apply_kscale(S, tsc_slot);
                        mask_scores(t, S);
                        raise_max(S);
                        exp_pack(S, pb, pl, C::INT8 ? tsc_slot + BN : nullptr);
                        u32x2_t vr[8];
                        lds_read_raw_vt<J>(va, vr);
#pragma unroll
                        for (int ts = 0; ts < C::TS; ++ts)
#pragma unroll
                            for (int db = 0; db < C::DB; ++db)
                                o_acc[db] = mma32<C::PVT>(widen8<C::PVT, KVT>(vr[ts * 4 + db]), pb[ts], o_acc[db]);
                    }
                    raw_dma(j_c, min(tile_of(k + 2), ig.t_end - 1));   // the slot's reads are complete
                    __builtin_amdgcn_wave_barrier();
                };
                for (int k = 0; k < n_iter; k += 2) {
                    fstep(I0{}, k);
                    fstep(I1{}, k + 1);
                }
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // the clamped loads past the end
            }
        } else {
            static_assert(C::PIPE || WR == 1, "items of 32 or 256 rows");
        }

        // ------------------------------------------------------------ finish the rows
        float LE = l_exact + __shfl_xor(l_exact, 32, 64);
        float L = LE;
        float M = m_run;
        MergeTarget tgt{a.out, a.lse, a.num_q_heads, a.group, vscale};
        if constexpr (C::WK > 1) {
            // The waves of the group streamed different tiles of the same rows:
            // bring their accumulators to a common max through LDS, then every
            // thread finishes 16 columns of one row (row tid/8).
            static_assert(WR == 1, "key-split waves are used with 32-row items only");
            __syncthreads();
            if (h32 == 0) { red_m[wid][l32] = M; red_e[wid][l32] = LE; }
            __syncthreads();
            float Mx = kNegInf;
#pragma unroll
            for (int w = 0; w < C::WK; ++w) Mx = fmaxf(Mx, red_m[w][l32]);
            const float al = (M == kNegInf) ? 0.f : fast_exp2(M - Mx);
            // [WK][32][D]; the 16-byte chunks of row r are XOR-ed with r so that
            // the 32 rows a half-wave writes at once (512 B apart) do not all
            // land in the same bank
            // (the fp8 staging path exchanges through its staging slots)
            static_assert(C::WK * 32 * D * 4 <= (C::FSTAGE ? C::STAGE_LDS : C::TILES_LDS),
                          "accumulator exchange fits the tile buffers");
            static_assert(D / 4 == 32, "32 chunks per row");
            float* accbuf = reinterpret_cast<float*>(C::FSTAGE ? stage : tiles);
            auto acc_at = [&](int row, int col) { return accbuf + row * D + (((col >> 2) ^ (row & 31)) << 2); };
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d = db * 32 + 8 * jj + 4 * h32;
                    *reinterpret_cast<float4*>(acc_at(wid * 32 + l32, d)) =
                        make_float4(o_acc[db][4 * jj] * al, o_acc[db][4 * jj + 1] * al, o_acc[db][4 * jj + 2] * al,
                                    o_acc[db][4 * jj + 3] * al);
                }
            __syncthreads();
            const int r = tid >> 3;
            const int c0 = (tid & 7) * 16;
            float Mr = kNegInf;
#pragma unroll
            for (int w = 0; w < C::WK; ++w) Mr = fmaxf(Mr, red_m[w][r]);
            float LEr = 0.f;
#pragma unroll
            for (int w = 0; w < C::WK; ++w) {
                const float mw = red_m[w][r];
                LEr += (mw == kNegInf) ? 0.f : red_e[w][r] * fast_exp2(mw - Mr);
            }
            float4 sum[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) sum[q] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < C::WK; ++w)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(acc_at(w * 32 + r, c0 + 4 * q));
                    sum[q].x += v.x; sum[q].y += v.y; sum[q].z += v.z; sum[q].w += v.w;
                }
            if (r < ig.rows) {
                const float inv = (LEr > 0.f) ? 1.0f / LEr : 0.f;
                float* op;
                float sc;
                if (direct) {
                    const int64_t orow = out_row(tgt, ig.si.q_off, ig.g, ig.row0 + r);
                    op = a.out + orow * D + c0;
                    sc = inv * vscale;
                    if (a.lse != nullptr && c0 == 0) a.lse[orow] = (LEr > 0.f) ? (Mr + fast_log2(LEr)) * kLn2 : kNegInf;
                } else {
                    const int64_t slot = (int64_t)(it + a.item_off) * BM + r;
                    op = a.ws_o + slot * D + c0;
                    sc = inv;
                    if (c0 == 0) a.ws_lse[slot] = (LEr > 0.f) ? Mr + fast_log2(LEr) : kNegInf;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<float4*>(op + 4 * q) =
                        make_float4(sum[q].x * sc, sum[q].y * sc, sum[q].z * sc, sum[q].w * sc);
            }
        } else if (row_ok) {
            const float inv = (L > 0.f) ? 1.0f / L : 0.f;
            if (direct) {
                const int64_t orow = out_row(tgt, ig.si.q_off, ig.g, row_g);
                float* op = a.out + orow * D;
                const float sc = inv * vscale;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d = db * 32 + 8 * jj + 4 * h32;
                        *reinterpret_cast<float4*>(op + d) =
                            make_float4(o_acc[db][4 * jj] * sc, o_acc[db][4 * jj + 1] * sc, o_acc[db][4 * jj + 2] * sc,
                                        o_acc[db][4 * jj + 3] * sc);
                    }
                if (a.lse != nullptr && h32 == 0) a.lse[orow] = (LE > 0.f) ? (M + fast_log2(LE)) * kLn2 : kNegInf;
            } else {
                const int64_t slot = (int64_t)(it + a.item_off) * BM + row_l;
                float* op = a.ws_o + slot * D;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d = db * 32 + 8 * jj + 4 * h32;
                        *reinterpret_cast<float4*>(op + d) =
                            make_float4(o_acc[db][4 * jj] * inv, o_acc[db][4 * jj + 1] * inv,
                                        o_acc[db][4 * jj + 2] * inv, o_acc[db][4 * jj + 3] * inv);
                    }
                if (h32 == 0) a.ws_lse[slot] = (LE > 0.f) ? M + fast_log2(LE) : kNegInf;
            }
        }
        if (!direct && ig.split == 0 && tid == 0)
            publish_merge(a, MergeDesc{it + a.item_off, ig.splits, ig.rows, BM, ig.si.q_off, ig.g, ig.row0, vscale});
        __syncthreads();
    }
}

}  // namespace

template <int D, int KVT, int QT, int WR>
static hipError_t launch_t(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((tile_attn_kernel<D, KVT, QT, WR>), dim3(grid), dim3(Cfg<D, KVT, QT, WR>::NTH),
                       plan_lds_bytes(a.num_seqs), st, a);
    return hipGetLastError();
}

template <int D, int KVT, int QT, int WR>
static int blocks_per_cu_t(size_t dyn_lds) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, tile_attn_kernel<D, KVT, QT, WR>,
                                                                      Cfg<D, KVT, QT, WR>::NTH, dyn_lds);
    return (e == hipSuccess && n > 0) ? n : 1;
}

// Instantiations by rows per item: 32-row items (WR = 1) and 256-row items
// (WR = 8) for every cache type.  f(tag) is called with the kernel's template arguments as types.
template <int KVT, int QT, int WR>
struct KernelTag {
    static constexpr int kvt = KVT, qt = QT, wr = WR;
};

template <typename F>
static bool with_kernel(int kv_dtype, int q_dtype, int wr, F&& f) {
    const bool fp8 = kv_dtype == PA_DTYPE_FP8_E4M3;
    if (kv_dtype == PA_DTYPE_INT8 && (wr == 1 || wr == 8)) {
        if (q_dtype == PA_DTYPE_BF16) {
            if (wr == 1) return f(KernelTag<PA_DTYPE_INT8, PA_DTYPE_BF16, 1>{}), true;
            return f(KernelTag<PA_DTYPE_INT8, PA_DTYPE_BF16, 8>{}), true;
        }
        if (wr == 1) return f(KernelTag<PA_DTYPE_INT8, PA_DTYPE_F16, 1>{}), true;
        return f(KernelTag<PA_DTYPE_INT8, PA_DTYPE_F16, 8>{}), true;
    }
    if (wr == 1) {
        if (kv_dtype == PA_DTYPE_F16) return f(KernelTag<PA_DTYPE_F16, PA_DTYPE_F16, 1>{}), true;
        if (kv_dtype == PA_DTYPE_BF16) return f(KernelTag<PA_DTYPE_BF16, PA_DTYPE_BF16, 1>{}), true;
        if (q_dtype == PA_DTYPE_BF16) return f(KernelTag<PA_DTYPE_FP8_E4M3, PA_DTYPE_BF16, 1>{}), true;
        return f(KernelTag<PA_DTYPE_FP8_E4M3, PA_DTYPE_F16, 1>{}), true;
    }
    if (wr == 8 && fp8) {
        if (q_dtype == PA_DTYPE_BF16) return f(KernelTag<PA_DTYPE_FP8_E4M3, PA_DTYPE_BF16, 8>{}), true;
        return f(KernelTag<PA_DTYPE_FP8_E4M3, PA_DTYPE_F16, 8>{}), true;
    }
    if (wr == 8 && !fp8) {
        if (kv_dtype == PA_DTYPE_F16) return f(KernelTag<PA_DTYPE_F16, PA_DTYPE_F16, 8>{}), true;
        return f(KernelTag<PA_DTYPE_BF16, PA_DTYPE_BF16, 8>{}), true;
    }
    return false;
}

int mfma_rows_per_item(int wr) { return 32 * wr; }

int mfma_blocks_per_cu(int kv_dtype, int q_dtype, int wr, int max_num_seqs) {
    const size_t dyn = plan_lds_bytes(max_num_seqs);
    int n = 1;
    with_kernel(kv_dtype, q_dtype, wr, [&](auto tag) {
        using T = decltype(tag);
        n = blocks_per_cu_t<128, T::kvt, T::qt, T::wr>(dyn);
    });
    return n;
}

hipError_t launch_mfma_attn(const DecodeArgs& a, int head_dim, int kv_dtype, int q_dtype, int wr, int grid,
                            hipStream_t stream) {
    if (head_dim != 128) return hipErrorInvalidValue;
    hipError_t e = hipErrorInvalidValue;
    with_kernel(kv_dtype, q_dtype, wr, [&](auto tag) {
        using T = decltype(tag);
        e = launch_t<128, T::kvt, T::qt, T::wr>(a, grid, stream);
    });
    return e;
}

}  // namespace pa
