// Fused attention forward on the gfx950 matrix cores (bf16 / fp16 inputs).
//
// Decomposition ("Understand FlashAttention", section "FlashAttention": outer
// loop over row blocks of Q, inner loop over column blocks of K and V).  One
// workgroup owns one (batch*head, query tile) pair of BR = 256 query rows;
// each of its 8 waves (two per SIMD) owns 32 rows.  The inner loop walks keys
// in tiles of BC = 128, and for every 32 keys of a tile it applies the update
// of that page's section "两块情况的完整推导" (steps 5-7): row max, rescale of
// the running sum and of the unnormalised output, P V; after the last tile it
// divides by the row sum (step 8) and writes the row log-sum-exp (appendix
// "附：数值稳定的logsumexp(L)推导").
//
// Data movement.  K and V tiles go from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging), two stages of K and of V,
// one barrier per tile, the loads of tile j+1 in flight while tile j is
// computed.  Rows keep their row-major layout with each 16-byte chunk placed
// at chunk index XOR a row-dependent swizzle, which makes every fragment read
// below free of LDS bank conflicts.  Fragment addresses are computed once;
// stage, key block and k-step are immediate offsets of the LDS reads.
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
// is a per-lane multiply.  The V^T A operand comes from the row-major V tile
// through ds_read_b64_tr_b16 (each 16-lane group transposes a 4 x 16 block).
//
// Overlap.  Each 64 keys are processed as two 32-key halves so that the
// scores of the second half (MFMA) are computed while the exponentials of the
// first (VALU) run, and each half's P V (MFMA) overlaps the next VALU work; the
// second wave on the SIMD fills the remaining gaps.  Tiles that cross the
// diagonal or the end of the sequence (the last ones of a wave) run a masked
// copy of the same body in a second loop, so the common loop has no masking.
//
// Softmax arithmetic.  t = s * c with c = scale * log2(e); p = 2^(t - m).
// The reference m is only moved when a row max exceeds it by more than
// TAU = 8 (in log2 units), so the O rescale runs a handful of times per row
// instead of once per key block.  This changes no result: softmax is invariant
// to the shift (same page, "数值稳定的 Softmax"), and p <= 2^8 keeps every
// intermediate far inside fp32/bf16/fp16 range.  The row sum adds the fp32
// probabilities before their rounding to the input type, so lse keeps fp32
// accuracy (a sum of bf16-rounded terms would cost ~2^-9 relative in l).
#pragma once

#include "common.hpp"

namespace attn {

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int N;           // sequence length
    int n_qtiles;    // ceil(N / BR)
    int total;       // B * H * n_qtiles
    float c;         // scale * log2(e)
};

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

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

template <typename T, int D, bool CAUSAL, int QG>
struct MfmaFwd {
    static constexpr int NW = 8 / QG;          // waves per workgroup (2 per SIMD for QG = 1, 1 for QG = 2)
    static constexpr int BR = NW * QG * 32;    // query rows per workgroup (256), 32 QG per wave
    static constexpr int BC = 128;             // keys per tile, as four 32-key quarters
    static constexpr int THREADS = NW * 64;
    static constexpr int CH = D / 8;           // 16-byte chunks per row
    static constexpr int ROWB = D * 2;         // bytes per K/V row
    static constexpr int TILE_B = BC * ROWB;   // bytes per K or V tile
    static constexpr int STAGES = 2;           // LDS stages (K tile + V tile each)
    static constexpr int LDS_B = STAGES * 2 * TILE_B;
    static constexpr int V_BASE = STAGES * TILE_B;  // V stages follow the K stages
    static constexpr int LOADS = BC * CH / 64 / NW;  // 16-byte-per-lane loads per wave per tile and tensor
    static constexpr int DB = D / 32;          // 32-row blocks of O^T
    static constexpr int DC = D / 16;          // k-steps of the first product
    static constexpr float TAU = 8.0f;
    typedef Mfma<T> M;
    typedef typename M::v8 v8;

    // chunk swizzles (see the bank analysis in the header comment of this file)
    static __device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

    static __device__ __forceinline__ v8 as_v8(u32x4_t x) { return __builtin_bit_cast(v8, x); }

    typedef uint32_t Packed[2][4];  // one 32-key half as two 16-key B operands

    // State a wave carries across key tiles.
    struct State {
        v8 qf[QG][DC];           // Q^T fragments of the wave's row groups
        f32x16_t acc[QG][DB];    // unnormalised O^T
        float m_ref[QG];         // reference row max (log2 domain)
        float lsum[QG];          // this lane's share of the row sums
        uint32_t kaddr[DC];      // LDS address of this lane's K fragment for k-step cc (stage 0)
        uint32_t vaddr[DB];      // LDS address of this lane's V^T fragment for d block db (stage 0)
        float c;                 // scale * log2(e), >= 0
        int q0, N, l32, g;       // first row of the wave, sequence length, lane coordinates
    };

    // ------------------------------------------------------------ building blocks

    // S^T for the 32 keys of half h of the tile in LDS stage ST, every row group
    // (each K fragment feeds one MFMA per group).  Stage and half are immediate offsets.
    template <int ST>
    static __device__ __forceinline__ void s_half(const State &S, int h, f32x16_t (&s)[QG]) {
        v8 kf[DC];
#pragma unroll
        for (int cc = 0; cc < DC; ++cc)
            kf[cc] = as_v8(*(const lds_u32x4_t *)(uintptr_t)(S.kaddr[cc] + ST * TILE_B + h * 32 * ROWB));
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) s[qg] = (f32x16_t){};
#pragma unroll
        for (int cc = 0; cc < DC; ++cc)
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) s[qg] = M::mma(kf[cc], S.qf[qg][cc], s[qg]);
    }

    // O^T += V^T P^T for the 32 keys of half h of the tile in LDS stage ST, every
    // row group (each V fragment feeds one MFMA per group)
    template <int ST>
    static __device__ __forceinline__ void pv_half(State &S, int h, const Packed (&pk)[QG]) {
        v8 vf[2][DB];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint32_t vb = S.vaddr[db] + ST * TILE_B + h * 32 * ROWB + kc * 16 * ROWB;
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(vb));
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(vb + 4 * ROWB));
                const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
                vf[kc][db] = as_v8((u32x4_t){l2[0], l2[1], h2[0], h2[1]});
            }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int qg = 0; qg < QG; ++qg) {
                    const u32x4_t pp = {pk[qg][kc][0], pk[qg][kc][1], pk[qg][kc][2], pk[qg][kc][3]};
                    S.acc[qg][db] = M::mma(vf[kc][db], as_v8(pp), S.acc[qg][db]);
                }
    }

    // is the key of accumulator register i of half h visible to row group qg of this lane?
    static __device__ __forceinline__ bool visible(const State &S, int k0, int h, int qg, int i) {
        const int key = k0 + 32 * h + (i & 7) + 8 * S.g + 16 * (i >> 3);
        return key < S.N && (!CAUSAL || key <= S.q0 + 32 * qg + S.l32);
    }

    // row max of a half in the log2 domain (-inf when nothing is visible)
    template <bool MASKED>
    static __device__ __forceinline__ float row_max(const State &S, const f32x16_t &s, int k0, int h, int qg) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, MASKED ? (visible(S, k0, h, qg, i) ? s[i] : -INFINITY) : s[i]);
        mx = lane_swap32_max(mx);
        return MASKED ? (mx == -INFINITY ? -INFINITY : mx * S.c) : mx * S.c;
    }

    // p = 2^(s c - m) in place
    template <bool MASKED>
    static __device__ __forceinline__ void exponentials(const State &S, f32x16_t &s, int k0, int h, int qg) {
        const float nm = S.m_ref[qg] == -INFINITY ? 0.f : -S.m_ref[qg];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float p = fast_exp2(fmaf(s[i], S.c, nm));
            if (MASKED) p = visible(S, k0, h, qg, i) ? p : 0.f;
            s[i] = p;
        }
    }

    // round p to T in pairs (two 16-key B operands) and add the fp32 p to the row sum
    static __device__ __forceinline__ void pack_sum(State &S, const f32x16_t &p, int qg, Packed &pk) {
        float rs = 0.f;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = p[8 * kc + 2 * e], p1 = p[8 * kc + 2 * e + 1];
                pk[kc][e] = M::pack(p0, p1);
                rs += p0 + p1;
            }
        S.lsum[qg] += rs;
    }

    // Move the reference max of group qg to mt; returns the factor applied.
    static __device__ __forceinline__ float rescale(State &S, int qg, float mt) {
        const float m_new = fmaxf(S.m_ref[qg], mt);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(S.m_ref[qg] - m_new);
        S.lsum[qg] *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) S.acc[qg][b][i] *= alpha;
        S.m_ref[qg] = m_new;
        return alpha;
    }

    // One key tile for one wave, as two 32-key halves:
    //   S(h0); max; [rescale];  exp(h0) | S(h1);  max; [rescale incl. pending p(h0)];
    //   pack(h0) + exp(h1) | PV(h0);  pack(h1) | PV(h1)
    template <bool MASKED, int ST>
    static __device__ __forceinline__ void tile(State &S, int k0) {
        sub<MASKED, ST, 0>(S, k0);
        sub<MASKED, ST, 2>(S, k0 + 64);
    }
    // 64 keys of the tile: quarters Q0 and Q0 + 1
    template <bool MASKED, int ST, int Q0>
    static __device__ __forceinline__ void sub(State &S, int k0) {
        f32x16_t s0[QG], s1[QG];
        float mt[QG];
        s_half<ST>(S, Q0, s0);
        bool grow = false;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            mt[qg] = row_max<MASKED>(S, s0[qg], k0, 0, qg);
            grow = grow || mt[qg] > S.m_ref[qg] + TAU;
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) rescale(S, qg, mt[qg]);
        }
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) exponentials<MASKED>(S, s0[qg], k0, 0, qg);
        s_half<ST>(S, Q0 + 1, s1);
        grow = false;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            mt[qg] = row_max<MASKED>(S, s1[qg], k0, 1, qg);
            grow = grow || mt[qg] > S.m_ref[qg] + TAU;
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                const float alpha = rescale(S, qg, mt[qg]);
#pragma unroll
                for (int i = 0; i < 16; ++i) s0[qg][i] *= alpha;  // p(h0) joins the new reference
            }
        }
        Packed pk0[QG], pk1[QG];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            pack_sum(S, s0[qg], qg, pk0[qg]);
            exponentials<MASKED>(S, s1[qg], k0, 1, qg);
        }
        pv_half<ST>(S, Q0, pk0);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) pack_sum(S, s1[qg], qg, pk1[qg]);
        pv_half<ST>(S, Q0 + 1, pk1);
    }

    // ------------------------------------------------------------ kernel body

    static __device__ void run(const FwdArgs &a) {
        extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

        const int N = a.N;
        const int logical = xcd_contiguous(blockIdx.x, a.total);
        const int bh = logical / a.n_qtiles;
        const int t_ = logical - bh * a.n_qtiles;
        const int qt = CAUSAL ? a.n_qtiles - 1 - t_ : t_;  // causal: longest rows first
        const size_t head = (size_t)bh * (size_t)N * D;
        const uint16_t *Qh = static_cast<const uint16_t *>(a.q) + head;
        const char *Kh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + head);
        const char *Vh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + head);

        const int tid = threadIdx.x;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
        const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;

        State S;
        S.q0 = qt * BR + w * QG * 32;
        S.N = N;
        S.l32 = l32;
        S.g = g;
        // A negative scale is applied as -|c| by negating Q (exact), so c >= 0 below.
        S.c = a.c;
        uint32_t qsign = 0u;
        if (S.c < 0.f) {
            S.c = -S.c;
            qsign = 0x80008000u;
        }

        // Q^T as the B operand: lane holds Q[q][16 cc + 8 g .. +7] for its rows q
        // (rows past the end read row N-1 and are zeroed).
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            const int q = S.q0 + 32 * qg + l32;
            const uint32_t keep = q < N ? 0xffffffffu : 0u;
            const uint16_t *qrow = Qh + (size_t)min(q, N - 1) * D + g * 8;
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                u32x4_t x = *reinterpret_cast<const u32x4_t *>(qrow + cc * 16);
                x = (x & keep) ^ qsign;
                S.qf[qg][cc] = as_v8(x);
            }
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) S.acc[qg][b][i] = 0.f;
            S.m_ref[qg] = -INFINITY;
            S.lsum[qg] = 0.f;
        }
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
        // Tile loads: lane fills LDS slot s with chunk (slot ^ swizzle) of K row
        // sigma(row) and of V row row.  Offsets are tile relative: row * ROWB + chunk * 16.
        uint32_t kld[LOADS], vld[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int s = (w * LOADS + i) * 64 + lane;
            const int r = s / CH, p = s % CH;
            kld[i] = ((r & ~31) | swap_bits23(r & 31)) * ROWB + ((p ^ kswz(r)) << 4);
            vld[i] = r * ROWB + ((p ^ vswz(r)) << 4);
        }

        const int n_kv_all = (N + BC - 1) / BC;
        const int n_kv = CAUSAL ? min(n_kv_all, (qt * BR + BR - 1) / BC + 1) : n_kv_all;

        auto issue_loads = [&](int j) {
            const int k0 = j * BC;
            unsigned char *ks = smem + (j % STAGES) * TILE_B;
            unsigned char *vs = smem + V_BASE + (j % STAGES) * TILE_B;
            const char *kt = Kh + (size_t)k0 * ROWB;
            const char *vt = Vh + (size_t)k0 * ROWB;
            if (k0 + BC <= N) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_global_load_lds((const void *)(kt + kld[i]),
                                                     (lds_void_t *)(ks + (w * LOADS + i) * 1024), 16, 0, 0);
                    __builtin_amdgcn_global_load_lds((const void *)(vt + vld[i]),
                                                     (lds_void_t *)(vs + (w * LOADS + i) * 1024), 16, 0, 0);
                }
            } else {  // last, partial tile: rows past the end read row N-1 (their scores are masked)
                const uint32_t last = (uint32_t)(N - 1 - k0) * ROWB;
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    const uint32_t kr = kld[i] & ~(uint32_t)(ROWB - 1), vr = vld[i] & ~(uint32_t)(ROWB - 1);
                    const uint32_t ko = min(kr, last) + (kld[i] & (ROWB - 1));
                    const uint32_t vo = min(vr, last) + (vld[i] & (ROWB - 1));
                    __builtin_amdgcn_global_load_lds((const void *)(kt + ko),
                                                     (lds_void_t *)(ks + (w * LOADS + i) * 1024), 16, 0, 0);
                    __builtin_amdgcn_global_load_lds((const void *)(vt + vo),
                                                     (lds_void_t *)(vs + (w * LOADS + i) * 1024), 16, 0, 0);
                }
            }
        };
        auto next = [&](int j) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // tile j is in LDS; every wave is done with tile j-1
            if (j + 1 < n_kv) issue_loads(j + 1);
        };

        // Tiles [0, j_plain) are fully visible to every row of this wave; the rest
        // cross its diagonal, hold the end of the sequence, or (causal) lie wholly
        // after its rows and are skipped.  Two loops keep one tile body per loop.
        const int j_plain = min(n_kv, min(CAUSAL ? (S.q0 + 1) / BC : n_kv, N / BC));
        issue_loads(0);
        int j = 0;
        // (unrolled by two so the LDS stage of each tile is a compile-time offset)
        for (; j + 1 < j_plain; j += 2) {
            next(j);
            tile<false, 0>(S, j * BC);
            next(j + 1);
            tile<false, 1>(S, (j + 1) * BC);
        }
        if (j < j_plain) {
            next(j);
            tile<false, 0>(S, j * BC);  // j is even here
            ++j;
        }
        for (; j < n_kv; ++j) {
            next(j);
            const int k0 = j * BC;
            if (CAUSAL && k0 > S.q0 + QG * 32 - 1) continue;  // every key after every row of this wave
            if (j & 1)
                tile<true, 1>(S, k0);
            else
                tile<true, 0>(S, k0);
        }

        // ---- epilogue: O = O~ / l, lse = (m + log2 l) ln 2.  Register i of block b is
        // output column 32 b + 8 (i >> 2) + 4 g + (i & 3) of row q.
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            const int q = S.q0 + 32 * qg + l32;
            const float ltot = lane_swap32_add(S.lsum[qg]);
            if (q < N) {
                const float inv = 1.f / ltot;
                uint16_t *Oh = static_cast<uint16_t *>(a.o) + head + (size_t)q * D;
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int quad = 0; quad < 4; ++quad) {
                        const uint32_t lo = M::pack(S.acc[qg][b][quad * 4 + 0] * inv, S.acc[qg][b][quad * 4 + 1] * inv);
                        const uint32_t hi = M::pack(S.acc[qg][b][quad * 4 + 2] * inv, S.acc[qg][b][quad * 4 + 3] * inv);
                        const u32x2_t y = {lo, hi};
                        *reinterpret_cast<u32x2_t *>(Oh + b * 32 + quad * 8 + 4 * g) = y;
                    }
                if (g == 0) a.lse[(size_t)bh * N + q] = (S.m_ref[qg] + fast_log2(ltot)) * kLn2;
            }
        }
    }
};

// Rows per wave: 32 (one group, two waves per SIMD).  The kernel also builds
// with two groups (64 rows, one wave per SIMD, half the LDS bytes per MFMA
// flop); on gfx950 that measured slower (820 vs 930 TFLOP/s on the causal
// N=8192 d=128 workload) because the compiler then moves the O accumulators
// between register files.
constexpr int kRowGroups = 1;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512 / kRowGroups, 1)
void attn_fwd_mfma_kernel(FwdArgs a) {
    static_assert(MfmaFwd<T, D, CAUSAL, kRowGroups>::THREADS == 512 / kRowGroups, "launch bounds");
    MfmaFwd<T, D, CAUSAL, kRowGroups>::run(a);
}

}  // namespace attn
