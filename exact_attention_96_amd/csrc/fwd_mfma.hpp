// Fused attention forward on the gfx950 matrix cores (bf16 / fp16 inputs).
//
// Decomposition ("Understand FlashAttention", section "FlashAttention": outer
// loop over row blocks of Q, inner loop over column blocks of K and V).  One
// workgroup owns one (batch*head, query tile) pair of BR = 256 query rows;
// each of its 8 waves owns 32 rows.  The inner loop walks keys in units of
// BU = 64 and for each unit applies the update of that page's section
// "两块情况的完整推导" (steps 5-7): row max, rescale of the running sum and of
// the unnormalised output, P V; after the last unit it divides by the row sum
// (step 8) and writes the row log-sum-exp (appendix "附：数值稳定的logsumexp(L)推导").
//
// Ping-pong.  Waves w and w + 4 share a SIMD.  Waves 0-3 and waves 4-7 form two
// groups that alternate between a matrix phase (the MFMAs of one unit: S of
// unit u and P V of unit u - 1) and a softmax phase (exponentials of unit u on
// the vector ALU); the second group runs one phase behind, and a workgroup
// barrier separates phases.  So on every SIMD one wave feeds the matrix core
// while the other computes exponentials.  During its softmax phase a wave also
// reads the K fragments of its next unit from LDS into registers, so that the
// score MFMAs of a matrix phase start without waiting for LDS; only the V^T
// reads remain in the matrix phase, issued ahead of the P V MFMAs.
//
// Data movement.  K and V units go from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging) into two rings of four stages;
// the load group of unit u + 3 is issued at the start of step u and its
// completion is awaited (explicit vmcnt counts) only at the barriers that
// precede its first reader.  Rows keep their row-major layout with each
// 16-byte chunk placed at chunk index XOR a row-dependent swizzle, which makes
// every fragment read below free of LDS bank conflicts.  Fragment addresses are
// computed once; stage, key half and key chunk are immediate offsets.
//
// First product, transposed: S^T = K Q^T with v_mfma_f32_32x32x16.  Q^T is the
// B operand, held in registers for the whole loop.  Its accumulator gives
// every lane one query row (lane % 32) and 16 keys, so row max and row sum
// are in-lane reductions plus one exchange with lane ^ 32 (permlane32 swap).
// The K rows of each 32-key block are stored in the order sigma(r) = r with
// bits 2 and 3 swapped; then accumulator registers 8h .. 8h+7 of lane half g
// hold the consecutive keys 16h + 8g .. 16h + 8g + 7, which is exactly the B
// operand layout of the second product O^T = V^T P^T: P goes from the softmax
// to the matrix core without leaving registers, and the per-row rescale of O^T
// is a per-lane multiply.  The V^T A operand comes from the row-major V unit
// through ds_read_b64_tr_b16 (each 16-lane group transposes a 4 x 16 block).
//
// Softmax arithmetic.  t = s * c with c = scale * log2(e); p = 2^(t - m) against
// a reference m that only moves when needed: each lane adds its 32 fp32 values
// of p for the unit, and that sum bounds every one of them, so while no lane's
// sum exceeds 2^16 the values are in range and no row max is computed at all.
// Otherwise (the first unit, or a row whose max grew well past m) the unit's row
// max is taken, m moves to it, O~ and the row sum are rescaled and p is recomputed.
// This changes no result: softmax is invariant to the shift (same page,
// "数值稳定的 Softmax").  The bound keeps every p finite after its rounding for the
// P V product: 2^16 for bf16 (8 exponent bits), 2^15 for fp16, whose largest finite
// value is 65504 (a p in [65520, 65536] would round to inf).  The row sum adds the fp32 probabilities before their
// rounding to the input type, so lse keeps fp32 accuracy (a sum of bf16-rounded
// terms would cost ~2^-9 relative in l).
#pragma once

#include <type_traits>

#include "addr.hpp"
#include "common.hpp"

namespace attn {

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int Nq, Nk;      // query and key sequence lengths
    int off;         // causal diagonal offset: key j is visible to query i iff j <= i + off (Nk - Nq)
    int n_qtiles;    // ceil(Nq / BR)
    int total;       // B * H * n_qtiles
    float c;         // scale * log2(e)
    // Optional bit mask (kernels instantiated with MASK only): bit j % 64 of word
    // j / 64 of row i is 1 iff key j is visible to query i.  Head (b, h) uses mask
    // head m = b * mask_sb + h * mask_sh, which starts at word m * Nq * mask_w; rows
    // are mask_w = ceil(Nk / 64) words apart.
    const uint64_t *mask;
    long long mask_sb, mask_sh;
    int mask_w;
    int H;
    // Optional tile summary of the mask (matrix-core kernels only): for mask head m
    // and query tile t of kMaskTileRows rows, tiles_w words starting at word
    // (m * tiles_nt + t) * tiles_w; bit u % 64 of word u / 64 is 1 iff some row of
    // the tile sees a key of unit u (keys 64 u .. 64 u + 63).  NULL: no summary.
    const uint64_t *tiles;
    int tiles_w, tiles_nt;
    // Persistent kernel only: grid size, jobs per head, heads, and whether the jobs of
    // the heads congruent to x mod 8 go to the workgroups on XCD x.
    int p_grid, p_jph, p_nbh, p_xcd;
};

// Query rows per tile of the mask summary (the matrix-core kernel's query tile).
constexpr int kMaskTileRows = 256;
// Keys per unit of the mask summary.
constexpr int kMaskUnitKeys = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
    typedef bf16x8_t v8;
    typedef bf16x2_t v2;
    static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // round a pair to bf16 (nearest even), packed low | high << 16
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        const f32x2_t v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, v2));
    }
};

template <> struct Mfma<_Float16> {
    typedef f16x8_t v8;
    typedef f16x2_t v2;
    static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        const f32x2_t v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, v2));
    }
};

// Lane id (0..63) computed where it is used: volatile, so the compiler neither hoists
// it nor keeps values derived from it live across the key loop (where it would
// spill them, and a spill reload waits for every load in flight, DMA included).
__device__ __forceinline__ uint32_t lane_id_here() {
    uint32_t x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

// Swap bits 2 and 3 of a row index inside a 32-row block (an involution).
__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float lane_swap32_max(float x) {
    // v_permlane32_swap: returns (x of lanes 0..31 in both halves, x of lanes 32..63 in both halves)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_swap32_add(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
// V^T reads issued before the first score MFMA of a matrix phase (interleaved timings on
// three boards: 0 beats 2 by ~0.4 %, 8 by ~1.5 %; 12 and 16 lose 16 % and 40 %)
constexpr int kGemmFirstReads = 0;

// Scheduling groups: N single MFMAs, each followed by up to PER of the LEFT
// remaining LDS reads.
template <int N, int PER, int LEFT>
__device__ __forceinline__ void sched_mfma_reads() {
    if constexpr (N > 0) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if constexpr (LEFT > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LEFT < PER ? LEFT : PER, 0);
        sched_mfma_reads<N - 1, PER, (LEFT > PER ? LEFT - PER : 0)>();
    }
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from global memory (base + voff) straight into LDS at
// lds + 16 * lane (global_load_lds_dwordx4; base and lds wave-uniform).  Issued
// from inline assembly so that the compiler does not order later LDS reads
// after it: completion is tracked with explicit vmcnt waits.  M0 carries the LDS
// address and is written here; nothing else in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; see above
__device__ __forceinline__ void dma_to_lds16(const void *base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
// The same with 4 bytes per lane (LDS at lds + 4 * lane).  base must be
// wave-uniform; it is passed through readfirstlane so that it lives in SGPRs.
__device__ __forceinline__ void dma_to_lds4(const void *base, uint32_t voff, uint32_t lds) {
    // (readfirstlane moves a signed int: the words are joined by addr_join, which widens
    // them as unsigned; a sign-extended low word once faulted the GPU on a mask base with
    // bit 31 set)
    const uint64_t b = reinterpret_cast<uintptr_t>(base);
    const int lo = __builtin_amdgcn_readfirstlane(addr_lo_word(b));
    const int hi = __builtin_amdgcn_readfirstlane(addr_hi_word(b));
    const uint64_t u = addr_join(lo, hi);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff),
                 "s"(reinterpret_cast<const void *>(u)), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

// Kernel variants.  kFwdPlain: at most one unit per wave needs the masked
// softmax (equal lengths, or a causal offset Nk - Nq that is a multiple of 32):
// straight-line code, the register budget of the hot path.  kFwdOffset: any
// causal offset; the wave's masked units (one or two) run in a loop.  kFwdBits:
// keys are also hidden by a caller's bit mask (FwdArgs::mask), read per unit
// through an LDS ring of its own that rides in the K/V load groups; every unit
// takes the masked softmax.
constexpr int kFwdPlain = 0, kFwdOffset = 1, kFwdBits = 2;

template <typename T, int D, bool CAUSAL, int MODE = kFwdPlain>
struct MfmaFwd {
    static constexpr bool MASK = MODE == kFwdBits;
    static constexpr int NW = 8;                     // waves per workgroup, two per SIMD
    static constexpr int BR = NW * 32;               // query rows per workgroup, 32 per wave
    static constexpr int BU = 64;                    // keys per unit (one matrix phase)
    static constexpr int STAGES = 4;                 // LDS ring depth, for K and for V
    static constexpr int THREADS = NW * 64;
    static constexpr int CH = D / 8;                 // 16-byte chunks per row
    static constexpr int ROWB = D * 2;               // bytes per K/V row
    static constexpr int UNIT_B = BU * ROWB;         // bytes per K or V unit
    static constexpr int V_BASE = STAGES * UNIT_B;   // V ring follows the K ring
    static constexpr int MUNIT_B = BR * 8;           // mask bits of one unit: a 64-bit word per row
    static constexpr int M_BASE = 2 * STAGES * UNIT_B;  // mask ring follows the V ring
    static constexpr int LIST_BASE = M_BASE + STAGES * MUNIT_B;  // unit list (MASK) follows the mask ring
    static constexpr int LIST_CAP = 4096;            // units of the list: Nk <= 262144 with a summary
    static constexpr int LDS_B = MASK ? LIST_BASE + 4 * LIST_CAP : M_BASE;
    static_assert(!MASK || (BR == kMaskTileRows && BU == kMaskUnitKeys), "summary tiles are query tiles and units");
    static constexpr int LOADS = BU * CH / 64 / NW;  // 16-byte-per-lane DMA loads per wave, unit and tensor
    static constexpr int KVLOADS = 2 * LOADS;        // K and V loads per wave in one load group
    static constexpr int GROUP = KVLOADS + (MASK ? 1 : 0);  // plus one 4-byte mask load per wave
    static_assert(!MASK || MUNIT_B == NW * 64 * 4, "one 4-byte mask load per lane covers a unit");
    static constexpr int DB = D / 32;                // 32-row blocks of O^T
    static constexpr int DC = D / 16;                // k-steps of the first product
    // bound on a lane's fp32 sum of p for one unit, hence on every p: 2^16 for bf16; 2^15
    // for fp16, so that no p rounds past fp16's largest finite value (65504)
    static constexpr float kSumBound = std::is_same<T, _Float16>::value ? 32768.0f : 65536.0f;
    static_assert(LOADS >= 1 && LOADS * 64 * NW == BU * CH, "unit loads split evenly over the waves");
    static_assert(LDS_B <= 160 * 1024, "LDS budget");
    static_assert(STAGES >= 3, "waits assume at least three ring stages");
    typedef Mfma<T> M;
    typedef typename M::v8 v8;

    // chunk swizzles (see the bank analysis in the header comment of this file)
    static __device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

    static __device__ __forceinline__ v8 as_v8(u32x4_t x) { return __builtin_bit_cast(v8, x); }

    typedef uint32_t Packed[2][2][4];  // P of one unit: [32-key half][16-key B operand][pair]

    // State a wave carries across units.
    struct State {
        v8 qf[DC];               // Q^T fragments of the wave's 32 rows
        f32x16_t acc[DB];        // unnormalised O^T
        float m_ref;             // reference row max (log2 domain)
        float lsum;              // this lane's share of the row sum
        uint32_t kaddr[DC];      // LDS address of this lane's K fragment for k-step cc (stage 0)
        uint32_t vaddr[DB];      // LDS address of this lane's V^T fragment for d block db (stage 0)
        float c;                 // scale * log2(e), >= 0
        int r0, Nk, off;         // first row of the wave, key length, causal offset
        uint32_t mrow0;          // LDS address of the workgroup-relative row r0 in mask stage 0
                                 // (MASK; wave-uniform: the lane adds 8 * (lane % 32))
    };

    // ------------------------------------------------------------ building blocks

    typedef v8 KFrags[2][DC];  // K fragments of one unit: [32-key half][k-step]

    // K fragments of the unit in ring stage offset koff (read during the softmax
    // phase before the matrix phase that uses them).
    static __device__ __forceinline__ void kload(const State &S, KFrags &kf, uint32_t koff) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int cc = 0; cc < DC; ++cc)
                kf[h][cc] = as_v8(*(const lds_u32x4_t *)(uintptr_t)(S.kaddr[cc] + koff + h * 32 * ROWB));
    }

    // Matrix phase: S^T of unit u (K fragments already in registers) and
    // O^T += V^T P^T of unit u - 1 (V in ring stage offset voff, P from the previous
    // softmax phase).  The V^T reads are issued first; the score MFMAs, which need no
    // LDS data, run while they are in flight.  dma(j) issues load j of this step's
    // load group; the loads go one per quarter of the P V MFMAs, each right after an
    // MFMA, so that a load waiting for the CU's vector-memory pipe (busy with the
    // other waves' loads) delays no MFMA.
    template <typename Dma>
    static __device__ __forceinline__ void gemm(State &S, f32x16_t (&s)[2], const Packed &pk, const KFrags &kf,
                                                uint32_t voff, Dma &&dma) {
        v8 vf[2][2][DB];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint32_t vb = S.vaddr[db] + voff + h * 32 * ROWB + kc * 16 * ROWB;
                    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(vb));
                    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(vb + 4 * ROWB));
                    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
                    vf[h][kc][db] = as_v8((u32x4_t){l2[0], l2[1], h2[0], h2[1]});
                }
        s[0] = (f32x16_t){};
        s[1] = (f32x16_t){};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) s[h] = M::mma(kf[h][cc], S.qf[cc], s[h]);
        // Issue order: kGemmFirstReads V^T reads (none), then each score MFMA followed by
        // its share of the reads (two: a fragment is two transposing reads).
        constexpr int NV = 8 * DB;       // transposing reads per unit
        constexpr int NS = 2 * DC;       // score MFMAs per unit
        constexpr int FIRST = kGemmFirstReads < NV ? kGemmFirstReads : NV;
        constexpr int PER = (NV - FIRST + NS - 1) / NS;
        if constexpr (FIRST > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, FIRST, 0);
        sched_mfma_reads<NS, PER, NV - FIRST>();
        constexpr int NP = 4 * DB;       // P V MFMAs per unit
        constexpr int CHUNK = NP / KVLOADS;
        static_assert(NP % KVLOADS == 0, "P V MFMAs split evenly around the loads");
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int h = j / (2 * DB), kc = (j / DB) % 2, db = j % DB;
            const u32x4_t pp = {pk[h][kc][0], pk[h][kc][1], pk[h][kc][2], pk[h][kc][3]};
            __builtin_amdgcn_sched_barrier(0);
            S.acc[db] = M::mma(vf[h][kc][db], as_v8(pp), S.acc[db]);
            if (j % CHUNK == 0) {
                __builtin_amdgcn_sched_barrier(0);
                dma(j / CHUNK);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Variant used by the persistent kernel, which keeps fewer registers across a phase:
    // the softmax phase reads only the first 32-key half of the next unit's K fragments
    // (kload_half), and the matrix phase reads the second half itself, ahead of the V^T
    // reads, while the score MFMAs of the first half run.  koff: LDS offset of the unit's
    // K ring stage.
    // These two take every fragment address from the k-step 0 and d-block 0 ones: under the
    // swizzles above, the K fragment of k-step cc sits at kaddr[0] ^ (32 cc) and the V^T
    // fragment of d block db at vaddr[0] ^ (64 db), so two registers hold what kaddr[] and
    // vaddr[] hold.
    // A ring stage offset (a multiple of 16 KB) commutes with these XORs (it only touches
    // bits 14 and up), so a stage known only at run time costs one add per phase, not one
    // per read.
    // (a stage known at compile time stays an immediate offset of the reads)
    static __device__ __forceinline__ uint32_t frag_addr(uint32_t base, uint32_t x, uint32_t off) {
        if (__builtin_constant_p(off)) return (base ^ x) + off;
        return (base + off) ^ x;
    }
    static __device__ __forceinline__ void kload_half(const State &S, KFrags &kf, uint32_t koff) {
#pragma unroll
        for (int cc = 0; cc < DC; ++cc)
            kf[0][cc] = as_v8(*(const lds_u32x4_t *)(uintptr_t)(frag_addr(S.kaddr[0], (uint32_t)(cc << 5), koff)));
    }
    template <typename Dma>
    static __device__ __forceinline__ void gemm_half(State &S, f32x16_t (&s)[2], const Packed &pk, KFrags &kf,
                                                     uint32_t koff, uint32_t voff, Dma &&dma) {
        // reads in issue order: while the first half's score MFMAs run, one K fragment of
        // the second half and one V^T fragment half each (a fragment freed, one read in);
        // then the remaining V^T reads, three per score MFMA of the second half
        static_assert(UNIT_B % 16384 == 0 || UNIT_B == 8192, "stage offsets above the XOR'd address bits");
        v8 vf[2][2][DB];
        auto vread = [&](int n) {  // n-th transposing read: fragment n / 2, half n % 2
            const int f = n >> 1, h = f / (2 * DB), kc = (f / DB) % 2, db = f % DB;
            const uint32_t vb = frag_addr(S.vaddr[0], (uint32_t)(db << 6), voff) + h * 32 * ROWB + kc * 16 * ROWB + (n & 1) * 4 * ROWB;
            const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(vb));
            const u32x2_t x2 = __builtin_bit_cast(u32x2_t, x);
            u32x4_t cur = __builtin_bit_cast(u32x4_t, vf[h][kc][db]);
            if (n & 1) {
                cur[2] = x2[0];
                cur[3] = x2[1];
            } else {
                cur[0] = x2[0];
                cur[1] = x2[1];
            }
            vf[h][kc][db] = as_v8(cur);
        };
        constexpr int NVR = 8 * DB;  // transposing reads per unit
#pragma unroll
        for (int cc = 0; cc < DC; ++cc) {
            kf[1][cc] = as_v8(*(const lds_u32x4_t *)(uintptr_t)(frag_addr(S.kaddr[0], (uint32_t)(cc << 5), koff) + 32 * ROWB));
            vread(cc);
        }
#pragma unroll
        for (int n = DC; n < NVR; ++n) vread(n);
        s[0] = (f32x16_t){};
        s[1] = (f32x16_t){};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) s[h] = M::mma(kf[h][cc], S.qf[cc], s[h]);
        constexpr int NS = 2 * DC;  // score MFMAs per unit
        sched_mfma_reads<DC, 2, 2 * DC>();
        sched_mfma_reads<DC, (NVR - DC + DC - 1) / DC, NVR - DC>();
        static_assert(NS == 2 * DC, "two halves of score MFMAs");
        constexpr int NP = 4 * DB;       // P V MFMAs per unit
        constexpr int CHUNK = NP / KVLOADS;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int h = j / (2 * DB), kc = (j / DB) % 2, db = j % DB;
            const u32x4_t pp = {pk[h][kc][0], pk[h][kc][1], pk[h][kc][2], pk[h][kc][3]};
            __builtin_amdgcn_sched_barrier(0);
            S.acc[db] = M::mma(vf[h][kc][db], as_v8(pp), S.acc[db]);
            if (j % CHUNK == 0) {
                __builtin_amdgcn_sched_barrier(0);
                dma(j / CHUNK);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Keys of a unit are visible to this lane's row up to a per-lane limit:
    // accumulator register i of half h holds the key at offset key_off(h, i) from
    // the unit start k0, and that key is visible iff key_off(h, i) <= lim(k0), with
    // lim = min(row + off, Nk - 1) - k0 - 8 g (causal) or Nk - 1 - k0 - 8 g.
    static __device__ __forceinline__ constexpr int key_off(int h, int i) { return 32 * h + (i & 7) + 16 * (i >> 3); }
    static __device__ __forceinline__ int vis_limit(const State &S, int k0) {
        // (lane coordinates from the lane id where used: nothing is kept live for them)
        const uint32_t ln = lane_id_here();
        const int l32 = (int)(ln & 31u), g = (int)(ln >> 5);
        const int last = CAUSAL ? min(S.r0 + l32 + S.off, S.Nk - 1) : S.Nk - 1;
        return last - k0 - 8 * g;
    }

    // MASK: visibility of the lane's 32 scores of a unit as bits, bit 16 h + i for
    // register i of half h: the caller's mask bits (row word of the unit in LDS at
    // moff) and the position limit.  Register i of half h is key 16 r + 8 g + (i & 7)
    // with r = 2 h + (i >> 3), i.e. byte 2 r + g of the row word; key offsets grow
    // with the bit index, so the position limit keeps a prefix of the bits.
    static __device__ __forceinline__ uint32_t visible_bits(const State &S, int k0, uint32_t moff) {
        // the lane's row address and key limit from the lane id (no register is kept
        // for them across the loop)
        const uint32_t ln = lane_id_here();
        const int l32 = (int)(ln & 31u), g = (int)(ln >> 5);
        const uint32_t addr = S.mrow0 + moff + 8u * (uint32_t)l32;
        const u32x2_t wd = *(const __attribute__((address_space(3))) u32x2_t *)(uintptr_t)addr;
        const uint32_t lo = wd[0] >> (8 * g), hi = wd[1] >> (8 * g);
        const uint32_t bits = (lo & 0xffu) | ((lo >> 8) & 0xff00u) | ((hi & 0xffu) << 16) | ((hi & 0xff0000u) << 8);
        const int last = CAUSAL ? min(S.r0 + l32 + S.off, S.Nk - 1) : S.Nk - 1;
        const int lim = last - k0 - 8 * g;
        int n = 0;  // registers whose key offset is <= lim: a prefix of the bit order
#pragma unroll
        for (int r = 0; r < 4; ++r) n += min(max(lim - 16 * r + 1, 0), 8);
        const uint32_t pos = n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
        return bits & pos;
    }
    static __device__ __forceinline__ bool vis_bit(uint32_t vm, int b) { return (vm >> b) & 1u; }

    // p = 2^(s c - m) for the unit starting at key k0 against the current reference
    // m, rounded to T in the B-operand layout; returns this lane's fp32 sum of p.
    template <bool MASKED>
    static __device__ __forceinline__ float exps(const State &S, const f32x16_t (&s)[2], Packed &pk, int k0,
                                                 uint32_t vm) {
        const float nm = S.m_ref == -INFINITY ? 0.f : -S.m_ref;
        const int lim = MASKED && !MASK ? vis_limit(S, k0) : 0;
        float rs = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i0 = 8 * kc + 2 * e;
                    float p0 = fast_exp2(fmaf(s[h][i0], S.c, nm));
                    float p1 = fast_exp2(fmaf(s[h][i0 + 1], S.c, nm));
                    if (MASKED && !MASK) {  // (MASK: hidden scores are already -inf)
                        p0 = key_off(h, i0) <= lim ? p0 : 0.f;
                        p1 = key_off(h, i0 + 1) <= lim ? p1 : 0.f;
                    }
                    pk[h][kc][e] = M::pack(p0, p1);
                    rs += p0 + p1;
                }
        return rs;
    }

    // Softmax phase of the unit starting at key k0.  The exponentials are taken
    // against the current reference m first; the lane's fp32 sum of its 32 values
    // bounds each of them, so when no lane's sum exceeds kSumBound every p is in
    // range and the unit is done.  Otherwise (a row whose max grew well past m) the
    // row max of the unit is taken, m moves to it, O~ and the row sum are rescaled,
    // and the exponentials are taken again.  The first unit of a tile (FIRST: m is
    // still -inf, O~ and the sum are zero) starts from its row max directly.  In the
    // looping variants (a caller's mask, or a row's first unit inside the loop) a
    // unit whose rows still have the reference -inf also takes the row max, which
    // starts the reference (it stays -inf while the row has seen no visible key).
    // moff: LDS offset of the unit's mask stage (MASK only).
    template <bool MASKED, bool FIRST>
    static __device__ __forceinline__ void soft(State &S, f32x16_t (&s)[2], Packed &pk, int k0, uint32_t moff = 0) {
        const uint32_t vm = MASK ? visible_bits(S, k0, moff) : 0u;
        if (MASK && __builtin_amdgcn_ballot_w64(vm != 0xffffffffu)) {
            // some score of the unit is hidden: set it to -inf in place (c > 0 here, so
            // its exponential is 0); wholly visible units skip this
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[h][i] = vis_bit(vm, 16 * h + i) ? s[h][i] : -INFINITY;
        }
        auto move_reference = [&](bool rescale) {
            const int lim = MASKED && !MASK ? vis_limit(S, k0) : 0;
            float mx = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx = fmaxf(mx, MASKED && !MASK ? (key_off(h, i) <= lim ? s[h][i] : -INFINITY) : s[h][i]);
            mx = lane_swap32_max(mx);
            const float mt = mx == -INFINITY ? -INFINITY : mx * S.c;
            const float m_new = fmaxf(S.m_ref, mt);
            if (rescale) {
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(S.m_ref - m_new);
                S.lsum *= alpha;
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) S.acc[b][i] *= alpha;
            }
            S.m_ref = m_new;
        };
        float rs;
        if (FIRST) {
            move_reference(false);
            rs = exps<MASKED>(S, s, pk, k0, vm);
        } else {
            rs = exps<MASKED>(S, s, pk, k0, vm);
            if (__builtin_amdgcn_ballot_w64(!(rs <= kSumBound) || (MODE != kFwdPlain && S.m_ref == -INFINITY))) {
                move_reference(true);
                rs = exps<MASKED>(S, s, pk, k0, vm);
            }
        }
        S.lsum += rs;
    }

    // Epilogue of a wave's 32 rows r0 .. r0 + 31 of one head: O = O~ / l rounded to T,
    // lse = (m + log2 l) ln 2 (fp32); a row that saw no key (l = 0, m = -inf) gets
    // O = 0 and lse = -inf; rows at or past Nq are not stored.  o_head and lse_head
    // point at the head's first row.  Register i of block b is output column
    // 32 b + 8 (i >> 2) + 4 g + (i & 3) of row q: the two lane halves of a row hold
    // alternate groups of 4 columns.  For groups k and k + 1 of a block, one
    // v_permlane32_swap per packed word (group k's word with group k + 1's) leaves lane
    // half 0 with columns 8 k .. 8 k + 7 of its row and lane half 1 with columns
    // 8 k + 8 .. 8 k + 15: one 16-byte store per lane and pair of groups.
    static __device__ __forceinline__ void epilogue(const State &S, uint16_t *o_head, float *lse_head, int r0,
                                                    int Nq, int lane_e) {
        const int l32e = lane_e & 31, ge = lane_e >> 5;
        const int q = r0 + l32e;
        const float ltot = lane_swap32_add(S.lsum);
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        u32x4_t out[DB][2];
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int k = 0; k < 4; k += 2) {  // column groups k and k + 1 of block b
                uint32_t w[2][2];             // [group k, k + 1][packed word]
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int i = 4 * (k + t);
                    w[t][0] = M::pack(S.acc[b][i + 0] * inv, S.acc[b][i + 1] * inv);
                    w[t][1] = M::pack(S.acc[b][i + 2] * inv, S.acc[b][i + 3] * inv);
                }
                const auto x0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
                const auto x1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
                out[b][k >> 1] = (u32x4_t){x0[0], x1[0], x0[1], x1[1]};
            }
        // (a head is below 2^31 bytes: 32-bit offset within it)
        char *dst = reinterpret_cast<char *>(o_head) + ((uint32_t)q * (uint32_t)ROWB + (uint32_t)(16 * ge));
        if (r0 + 32 <= Nq) {  // every row of the wave is stored (wave-uniform)
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int k = 0; k < 2; ++k) *reinterpret_cast<u32x4_t *>(dst + b * 64 + 32 * k) = out[b][k];
        } else if (q < Nq) {
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int k = 0; k < 2; ++k) *reinterpret_cast<u32x4_t *>(dst + b * 64 + 32 * k) = out[b][k];
        }
        if (q < Nq && ge == 0) lse_head[q] = (S.m_ref + fast_log2(ltot)) * kLn2;
    }

    // ------------------------------------------------------------ kernel body

    // Workgroup barrier after this wave's DMA has at most VMCNT loads in flight and
    // its LDS reads have completed; nothing is scheduled across it.
    template <int VMCNT>
    static __device__ __forceinline__ void barrier() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(VMCNT) : "memory");
        __builtin_amdgcn_sched_barrier(0);
    }

    static __device__ void run(const FwdArgs &a) {
        extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

        const int Nq = a.Nq, Nk = a.Nk, off = CAUSAL ? a.off : 0;
        // Work order.  The 8 XCDs take block indices round robin, each with its own L2.
        // Causal: longest tiles first, so that the dispatcher always starts the longest
        // remaining tile.  When B*H is a multiple of 16, XCD x serves the heads congruent
        // to x mod 8, a few at a time: groups of hg heads, each group's tiles from the
        // last (longest) to the first, the heads of a group interleaved.  Tiles of one
        // head then start close together and read its K and V units from the L2 at
        // nearly the same time.  Otherwise the rank is simply longest-first over all
        // heads.  Non-causal tiles are all equal: each XCD takes a contiguous range of
        // (head, tile) pairs, so consecutive tiles of a head share its L2.  With a
        // caller's mask the tiles skip different numbers of units; they take the causal
        // order (later query tiles first), which starts the longest tiles first for the
        // usual lower-triangular and banded masks and costs nothing for uniform ones.
        int bh, qt;
        if (CAUSAL || MASK) {
            const int nq = a.n_qtiles, n_bh = a.total / nq, per = n_bh >> 3;
            if ((n_bh & 15) == 0) {
                const int hg = (per & 3) == 0 ? 4 : 2;
                const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
                const int grp = j / (hg * nq), rem = j - grp * (hg * nq);
                qt = nq - 1 - rem / hg;
                bh = x + 8 * (grp * hg + rem % hg);
            } else {
                bh = blockIdx.x % n_bh;
                qt = nq - 1 - blockIdx.x / n_bh;
            }
        } else {
            const int logical = xcd_contiguous(blockIdx.x, a.total);
            bh = logical / a.n_qtiles;
            qt = logical - bh * a.n_qtiles;
        }
        const size_t head = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
        const uint16_t *Qh = static_cast<const uint16_t *>(a.q) + head;
        const char *Kh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + headk);
        const char *Vh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + headk);

        const int tid = threadIdx.x;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
        const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
        // Waves w and w + 4 share a SIMD and form the two phase groups; they take
        // neighbouring 32-row blocks so that both need the same number of key units.
        const bool lag = w >= NW / 2;

        State S;
        S.r0 = qt * BR + 64 * (w & 3) + 32 * (w >> 2);
        S.Nk = Nk;
        S.off = off;
        // A negative scale is applied as -|c| by negating Q (exact), so c >= 0 below.
        S.c = a.c;
        uint32_t qsign = 0u;
        if (S.c < 0.f) {
            S.c = -S.c;
            qsign = 0x80008000u;
        }
        // MASK writes -inf into hidden scores: keep c > 0 so that -inf * c stays -inf
        // (a scale of 0 becomes 1e-30, which moves no finite score by an ulp of the
        // reference it is added to)
        if (MASK) S.c = fmaxf(S.c, 1e-30f);

        // Q^T as the B operand: lane holds Q[q][16 cc + 8 g .. +7] for its row q
        // (rows past the end read row Nq-1 and are zeroed).
        {
            const int q = S.r0 + l32;
            const uint32_t keep = q < Nq ? 0xffffffffu : 0u;
            const uint16_t *qrow = Qh + (size_t)min(q, Nq - 1) * D + g * 8;
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                u32x4_t x = *reinterpret_cast<const u32x4_t *>(qrow + cc * 16);
                x = (x & keep) ^ qsign;
                S.qf[cc] = as_v8(x);
            }
        }
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) S.acc[b][i] = 0.f;
        S.m_ref = -INFINITY;
        S.lsum = 0.f;

        // Fragment read addresses (stage 0; the stage, the key half and the key chunk
        // are added as immediate offsets).  K: lane reads chunk 2 cc + g of LDS row
        // l32, stored at chunk (2 cc + g) ^ kswz(l32).  V^T: 16-lane group grp reads
        // rows r_lane + 4 t + 16 kc at chunk 4 db + c_lane, stored at chunk
        // (4 db + c_lane) ^ vswz(r_lane).
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
#pragma unroll
        for (int cc = 0; cc < DC; ++cc) S.kaddr[cc] = lds0 + l32 * ROWB + (((2 * cc + g) ^ kswz(l32)) << 4);
        {
            const int j16 = lane & 15, grp = lane >> 4;
            const int r_lane = 8 * (grp >> 1) + (j16 >> 2);
            const int c_lane = 2 * (grp & 1) + ((j16 & 3) >> 1);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                S.vaddr[db] = lds0 + V_BASE + r_lane * ROWB + (((4 * db + c_lane) ^ vswz(r_lane)) << 4) + 8 * (j16 & 1);
        }
        // Unit loads: lane fills LDS slot s with chunk (slot ^ swizzle) of K row
        // sigma(row) and of V row row.  Offsets are unit relative: row * ROWB + chunk * 16.
        uint32_t kld[LOADS], vld[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int s = (w * LOADS + i) * 64 + lane;
            const int r = s / CH, p = s % CH;
            kld[i] = ((r & ~31) | swap_bits23(r & 31)) * ROWB + ((p ^ kswz(r)) << 4);
            vld[i] = r * ROWB + ((p ^ vswz(r)) << 4);
        }
        // Mask loads (MASK): lane fills bytes 4 (lane & 1) .. +3 of the unit word of
        // workgroup row (64 w + lane) / 2, stored densely (8 bytes per row) in LDS.  The
        // lane's source offset is recomputed per load (registers are scarce in the loop).
        const uint64_t *Mh = nullptr;
        size_t mhead = 0;  // mask head of (b, h)
        if (MASK) {
            const int b = bh / a.H, hh = bh - b * a.H;
            mhead = (size_t)b * (size_t)a.mask_sb + (size_t)hh * (size_t)a.mask_sh;
            Mh = a.mask + mhead * (size_t)Nq * (size_t)a.mask_w;
            S.mrow0 = lds0 + M_BASE + (uint32_t)(S.r0 - qt * BR) * 8u;
        }
        auto mask_src = [&]() -> uint32_t {  // from the lane id, recomputed per load
            const int ln = (int)lane_id_here();
            const int q = min(qt * BR + ((w * 64 + ln) >> 1), Nq - 1);
            return (uint32_t)q * (uint32_t)a.mask_w * 8u + 4u * (uint32_t)(ln & 1);
        };

        // Units of BU keys this workgroup and this wave need: causal rows see keys up
        // to row + off (none when that is negative).  A workgroup loads at least one
        // unit so that every load is in bounds; waves without keys only pass barriers.
        auto units_to = [&](int last_key) { return last_key < 0 ? 0 : last_key / BU + 1; };
        const int n_units = (Nk + BU - 1) / BU;
        int nu_wg = CAUSAL ? max(1, min(n_units, units_to(min(qt * BR + BR, Nq) - 1 + off))) : n_units;
        int nu = S.r0 >= Nq ? 0 : (CAUSAL ? min(n_units, units_to(min(S.r0 + 31, Nq - 1) + off)) : n_units);
        // Unit schedule (MASK with a tile summary): the workgroup visits only the units in
        // which some row of its query tile sees a key, in increasing order; position p
        // of the loop below is unit list[p] (LDS).  nu_wg and nu become position counts
        // (this wave: the listed units it needs).  Without a summary position p is unit p.
        // A tile that sees no key at all still loads unit 0 (list[0] = 0) and computes
        // nothing, so that every load is in bounds.
        const bool use_list = MASK && a.tiles != nullptr;
        if (use_list) {
            const uint64_t *tw = a.tiles + (mhead * (size_t)a.tiles_nt + (size_t)qt) * (size_t)a.tiles_w;
            int cnt = 0, cnt_w = 0;
            for (int wi = 0; wi * 64 < nu_wg; ++wi) {
                uint64_t bits = tw[wi];
                const int lim_wg = nu_wg - wi * 64, lim_w = nu - wi * 64;
                if (lim_wg < 64) bits &= (1ull << lim_wg) - 1ull;
                const uint64_t bits_w = lim_w <= 0 ? 0ull : (lim_w >= 64 ? bits : bits & ((1ull << lim_w) - 1ull));
                if (w == 0 && ((bits >> lane) & 1ull)) {
                    const int pos = cnt + __builtin_popcountll(bits & ((1ull << lane) - 1ull));
                    *(__attribute__((address_space(3))) int *)(uintptr_t)(lds0 + LIST_BASE + 4 * pos) = wi * 64 + lane;
                }
                cnt += __builtin_popcountll(bits);
                cnt_w += __builtin_popcountll(bits_w);
            }
            if (w == 0 && lane == 0 && cnt == 0) *(__attribute__((address_space(3))) int *)(uintptr_t)(lds0 + LIST_BASE) = 0;
            nu_wg = max(cnt, 1);
            nu = cnt_w;
            __syncthreads();
        }
        // unit at loop position p (wave-uniform)
        auto unit_at = [&](int p) -> int {
            if (MASK && use_list)
                return __builtin_amdgcn_readfirstlane(
                    *(const __attribute__((address_space(3))) int *)(uintptr_t)(lds0 + LIST_BASE + 4 * p));
            return p;
        };
        // The first nm units are visible to every row of the wave (no caller mask, keys
        // below the first row's diagonal and the sequence end) and take the unmasked
        // softmax; the rest of the wave's units (at least the last one) are masked.
        const int n_full = CAUSAL ? (min(S.r0 + off, Nk - 1) + 1) / BU : Nk / BU;
        const int nm = MASK ? 0 : max(0, min(nu - 1, n_full));
        // kFwdPlain is only launched where nu - nm <= 1 for every wave

        // Load j of a unit (16 bytes per lane) into a ring stage.  Rows past the end of
        // the sequence read row Nk - 1 (their scores are masked); the clamp is a no-op
        // for full units.
        auto load_one = [&](const char *src_head, int lds_off, uint32_t ld, int unit, int j) {
            const int k0 = unit * BU;
            const char *src = src_head + (size_t)k0 * ROWB;
            const uint32_t dst = lds0 + lds_off + (w * LOADS + j) * 1024;
            const uint32_t last = (uint32_t)min(Nk - 1 - k0, BU - 1) * ROWB;
            const uint32_t off = min(ld & ~(uint32_t)(ROWB - 1), last) + (ld & (ROWB - 1));
            dma_to_lds16(src, off, dst);
        };
        auto load_unit = [&](const char *src_head, int lds_off, const uint32_t (&ld)[LOADS], int unit) {
#pragma unroll
            for (int j = 0; j < LOADS; ++j) load_one(src_head, lds_off, ld[j], unit, j);
        };
        // Load group i (i >= 1): K of unit i into stage i mod STAGES, V of unit i - 1
        // into stage (i - 1) mod STAGES and (MASK) the mask bits of unit i - 1 into mask
        // stage (i - 1) mod STAGES.  Groups past the last unit repeat the last unit
        // into stages nobody reads any more, so that every group is GROUP loads and
        // the waits below are constant counts.  issue_part(i, j) issues load j of the
        // group (K loads first, then V loads, then the mask load).
        // The units of group i are looked up once per step (un = units(i)), before the
        // matrix phase that issues the group.
        struct Units {
            int k, v;  // unit of the K load and of the V (and mask) loads
        };
        auto units = [&](int i) { return Units{unit_at(min(i, nu_wg - 1)), unit_at(min(i - 1, nu_wg - 1))}; };
        auto issue_part = [&](const Units &un, int i, int j) {
            if (j < LOADS)
                load_one(Kh, (i % STAGES) * UNIT_B, kld[j], un.k, j);
            else if (j < KVLOADS)
                load_one(Vh, V_BASE + ((i - 1) % STAGES) * UNIT_B, vld[j - LOADS], un.v, j - LOADS);
            else
                dma_to_lds4(Mh + un.v, mask_src(), lds0 + M_BASE + ((i - 1) % STAGES) * MUNIT_B + w * 256);
        };
        // the mask load of a group goes first in its step, the K/V loads are spread
        // over the P V MFMAs by gemm
        auto issue_mask = [&](const Units &un, int i) {
            if (MASK) issue_part(un, i, KVLOADS);
        };
        auto issue = [&](int i) {
            const Units un = units(i);
#pragma unroll
            for (int j = 0; j < GROUP; ++j) issue_part(un, i, j);
        };

        // Barriers wait for this wave's DMA.  Data of load group i is read from the
        // barrier that ends the first group's matrix phase of unit i - 1 on (K fragments
        // of unit i by the first group's softmax phase, V of unit i - 1 by the matrix
        // phases of unit i).  Before a mid-step barrier a wave has issued groups up to
        // u + STAGES - 1 and needs group u + 1; before the barrier that ends a step the
        // lagging group needs group u + 2 (the first group needs less).
        constexpr int MID = GROUP * (STAGES - 2), END = GROUP * (STAGES - 3);
        auto barrier_mid = [&]() { barrier<MID>(); };
        auto barrier_end = [&]() { barrier<END>(); };

        // The matrix phase of unit 0 also runs the P V stream, with P = 0 against the
        // V ring stage that unit -1 would use, zeroed here; the matrix phase of unit
        // nu (P V of the wave's last unit) also computes scores it never uses.
        f32x16_t s[2];
        Packed pk;
        KFrags kf;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[h][kc][e] = 0u;
        {
            u32x4_t *vz = reinterpret_cast<u32x4_t *>(smem + V_BASE + (STAGES - 1) * UNIT_B);
            for (int i = tid; i < UNIT_B / 16; i += THREADS) vz[i] = (u32x4_t){0u, 0u, 0u, 0u};
        }
        // Steps u = 0 .. nu_wg.  A step is the matrix phase of unit u, a barrier, the
        // softmax phase of unit u (which also reads the K fragments of unit u + 1), a
        // barrier.  The lagging group runs one phase behind, so on every SIMD one wave
        // issues MFMAs while the other computes exponentials; both groups pass the
        // same barriers.  This wave computes in steps 0 .. nu (unit nu - 1 masked, step
        // nu only finishes P V) and only loads in the rest.
        auto pin_soft = [&]() {  // softmax results are complete before the barrier that ends their phase
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) asm volatile("" : "+v"(*reinterpret_cast<u32x4_t *>(pk[h][kc])));
            asm volatile("" : "+v"(S.lsum), "+v"(S.m_ref));
        };
        auto plain_step = [&](auto st, int u) {
            constexpr int ST = decltype(st)::value;  // u mod STAGES
            const Units un = units(u + STAGES - 1);
            issue_mask(un, u + STAGES - 1);
            gemm(S, s, pk, kf, ((ST + STAGES - 1) % STAGES) * UNIT_B, [&](int j) { issue_part(un, u + STAGES - 1, j); });
            barrier_mid();
            kload(S, kf, ((ST + 1) % STAGES) * UNIT_B);
            soft<false, false>(S, s, pk, u * BU);
            pin_soft();
            barrier_end();
        };

        // prologue: group 0 is K of unit 0 only (V stage STAGES - 1 holds zeros)
        load_unit(Kh, 0, kld, unit_at(0));
        for (int i = 1; i < STAGES - 1; ++i) issue(i);
        barrier_mid();
        kload(S, kf, 0);
        if (lag) barrier_end();
        int u = 0;
        if (!MASK && nm > 0) {
            // unit 0 (plain, first of the tile), then the plain units up to nm - 1,
            // unrolled by four from unit 1 so that the ring stage is an immediate
            const Units un = units(STAGES - 1);
            issue_mask(un, STAGES - 1);
            gemm(S, s, pk, kf, (STAGES - 1) * UNIT_B, [&](int j) { issue_part(un, STAGES - 1, j); });
            barrier_mid();
            kload(S, kf, 1 * UNIT_B);
            soft<false, true>(S, s, pk, 0);
            pin_soft();
            barrier_end();
            u = 1;
            for (; u + STAGES <= nm; u += STAGES) {
                plain_step(std::integral_constant<int, 1>(), u);
                plain_step(std::integral_constant<int, 2>(), u + 1);
                plain_step(std::integral_constant<int, 3>(), u + 2);
                plain_step(std::integral_constant<int, 0>(), u + 3);
            }
            for (; u < nm; ++u) {  // remaining plain steps, ring stage from u
                const Units un = units(u + STAGES - 1);
                issue_mask(un, u + STAGES - 1);
                gemm(S, s, pk, kf, ((u + STAGES - 1) % STAGES) * UNIT_B, [&](int j) { issue_part(un, u + STAGES - 1, j); });
                barrier_mid();
                kload(S, kf, ((u + 1) % STAGES) * UNIT_B);
                soft<false, false>(S, s, pk, u * BU);
                pin_soft();
                barrier_end();
            }
        }
        // MASK: the units of positions u .. u + 3 ride in a scalar shift register
        // (lst[j] = unit of position min(u + j, nu_wg - 1)); each step reads one new
        // list entry during its softmax phase and takes it after the barrier that ends
        // the step (which has waited for LDS), so no lookup latency lands on a phase.
        int lst[STAGES];
        if (MASK) {
#pragma unroll
            for (int j = 0; j < STAGES; ++j) lst[j] = unit_at(min(j, nu_wg - 1));
        }
        // st: u mod STAGES as a compile-time constant (ring stages as immediates), or -1
        auto masked_step_bits = [&](auto st) {
            constexpr int ST = decltype(st)::value;
            const int sg = ST >= 0 ? ST : u % STAGES;
            const Units un{lst[STAGES - 1], lst[STAGES - 2]};
            issue_mask(un, u + STAGES - 1);
            gemm(S, s, pk, kf, ((sg + STAGES - 1) % STAGES) * UNIT_B, [&](int j) { issue_part(un, u + STAGES - 1, j); });
            barrier_mid();
            const int next = min(u + STAGES, nu_wg - 1);
            int pf = next;
            if (use_list) pf = *(const __attribute__((address_space(3))) int *)(uintptr_t)(lds0 + LIST_BASE + 4 * next);
            kload(S, kf, ((sg + 1) % STAGES) * UNIT_B);
            soft<true, false>(S, s, pk, lst[0] * BU, sg * MUNIT_B);
            pin_soft();
            barrier_end();
#pragma unroll
            for (int j = 0; j + 1 < STAGES; ++j) lst[j] = lst[j + 1];
            lst[STAGES - 1] = __builtin_amdgcn_readfirstlane(pf);
        };
        auto masked_step = [&]() {
            const Units un = units(u + STAGES - 1);
            issue_mask(un, u + STAGES - 1);
            gemm(S, s, pk, kf, ((u + STAGES - 1) % STAGES) * UNIT_B, [&](int j) { issue_part(un, u + STAGES - 1, j); });
            barrier_mid();
            kload(S, kf, ((u + 1) % STAGES) * UNIT_B);
            if (MODE != kFwdPlain)  // a reference still at -inf takes the row max
                soft<true, false>(S, s, pk, unit_at(u) * BU, (u % STAGES) * MUNIT_B);
            else if (u == 0)
                soft<true, true>(S, s, pk, u * BU);
            else
                soft<true, false>(S, s, pk, u * BU);
            pin_soft();
            barrier_end();
        };
        // masked steps nm .. nu - 1: every unit with a caller's mask; one or two where
        // the causal diagonal of the wave's 32 rows may cross a unit boundary; one in
        // kFwdPlain
        if (MASK) {  // from unit 0: unrolled by four so that the ring stage is an immediate
            for (; u + STAGES <= nu; ) {
                masked_step_bits(std::integral_constant<int, 0>());
                ++u;
                masked_step_bits(std::integral_constant<int, 1>());
                ++u;
                masked_step_bits(std::integral_constant<int, 2>());
                ++u;
                masked_step_bits(std::integral_constant<int, 3>());
                ++u;
            }
            for (; u < nu; ++u) masked_step_bits(std::integral_constant<int, -1>());
        } else if (MODE != kFwdPlain) {
            for (; u < nu; ++u) masked_step();
        } else if (u < nu) {
            masked_step();
            ++u;
        }
        if (nu > 0) {  // step nu: P V of the last unit (u = nu)
            const Units un = units(u + STAGES - 1);
            issue_mask(un, u + STAGES - 1);
            gemm(S, s, pk, kf, ((u + STAGES - 1) % STAGES) * UNIT_B, [&](int j) { issue_part(un, u + STAGES - 1, j); });
            barrier_mid();
            barrier_end();
            ++u;
        }
        for (; u <= nu_wg; ++u) {  // steps after this wave's last unit: loads and barriers only
            issue(u + STAGES - 1);
            barrier_mid();
            barrier_end();
        }
        if (!lag) barrier<0>();
        // Every DMA of this wave has landed before it leaves: the LDS it writes belongs
        // to this workgroup only while the workgroup runs.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

        // ---- epilogue (MASK: lane id recomputed, so that it is not live across the loop)
        epilogue(S, static_cast<uint16_t *>(a.o) + head, a.lse + (size_t)bh * Nq, S.r0, Nq,
                 MASK ? (int)lane_id_here() : lane);
    }
};

template <typename T, int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(512, 1)
void attn_fwd_mfma_kernel(FwdArgs a) {
    static_assert(MfmaFwd<T, D, CAUSAL, MODE>::THREADS == 512, "launch bounds");
    MfmaFwd<T, D, CAUSAL, MODE>::run(a);
}

}  // namespace attn
