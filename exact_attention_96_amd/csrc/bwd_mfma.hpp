// Attention backward on the gfx950 matrix cores (bf16 / fp16 inputs).
//
// "Understand FlashAttention" (nothiny.github.io), section "反向传播": with
// S = scale Q K^T and P = softmax(S) row by row,
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_j P_ij dP_ij,
//   dQ = scale dS K,  dK = scale dS^T Q.
// P is recomputed from the forward's row log-sum-exp L (same page, section
// "为什么保存 logsumexp": P_ij = e^{S_ij - L_i}), so nothing N x N is stored.
// D_i equals dO_i . O_i (O = P V), computed once per row by a small kernel.
//
// Two kernels share the fragment layouts of the forward (fwd_mfma.hpp):
//   dQ:   each wave keeps 32 query rows (Q^T and dO^T as MFMA B operands in
//         registers) and streams 32-key blocks of K and V through LDS:
//         S^T = K Q^T, dP^T = V dO^T, dS^T = P^T o (dP^T - D), dQ^T += K^T dS^T.
//   dK/dV: each wave keeps 32 key rows (the workgroup's 128 K and V rows stay
//         in LDS) and streams 32-query blocks of Q, dO, L and D through LDS:
//         S = Q K^T, dP = dO V^T, dS = P o (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
// The rows of a streamed block are read as MFMA A operands in the order
// sigma(r) (bits 2 and 3 of r swapped), which makes the accumulator of the
// first products hold, in lane half g, register i, the row 16 (i >> 3) + 8 g +
// (i & 7): exactly the B-operand layout of the last products, so P and dS go
// from the vector ALU to the matrix core without leaving registers.  The
// transposed operands (K^T, dO^T, Q^T) come from the same row-major LDS blocks
// through ds_read_b64_tr_b16.  LDS rows carry their 16-byte chunks at
// chunk ^ swz(row), a swizzle under which both kinds of read are free of bank
// conflicts: sixteen consecutive rows read at one chunk land on sixteen different
// bank groups, and so do the four rows by four chunks of one transposing read.
#pragma once

#include "fwd_mfma.hpp"

namespace attn {

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *delta;    // [B*H*N] D_i = dO_i . O_i (written by the delta kernel)
    int N;           // sequence length
    int n_tiles;     // tiles per head of the kernel being launched
    int total;       // B * H * n_tiles
    float c;         // scale * log2(e)
    float scale;
};

// One dword per lane from a per-lane 64-bit address into LDS at lds + 4 * lane
// (global_load_lds_dword), issued like dma_to_lds16 so that completion is
// tracked only by the explicit vmcnt waits of the kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; see dma_to_lds16
__device__ __forceinline__ void dma_to_lds4(const void *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(addr), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// D_i = sum_c dO[i][c] O[i][c] in fp32, D / 8 lanes per row (16 bytes each).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const void *o, const void *dout, float *delta,
                                                            size_t rows) {
    constexpr int LPR = D / 8;
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t row = t / LPR;
    const int part = (int)(t % LPR);
    float acc = 0.f;
    if (row < rows) {
        const size_t off = (size_t)row * D + part * 8;
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(o) + off);
        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(dout) + off);
        typedef T t8 __attribute__((ext_vector_type(8)));
        const t8 x = __builtin_bit_cast(t8, a), y = __builtin_bit_cast(t8, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (row < rows && part == 0) delta[row] = acc;
}

template <typename T, int D>
struct BwdCommon {
    static constexpr int ROWB = D * 2;           // bytes per row
    static constexpr int CH = D / 8;             // 16-byte chunks per row
    static constexpr int DB = D / 32;            // 32-column blocks of d
    static constexpr int DC = D / 16;            // 16-column k-steps of d
    typedef Mfma<T> M;
    typedef typename M::v8 v8;
    static __device__ __forceinline__ v8 as_v8(u32x4_t x) { return __builtin_bit_cast(v8, x); }
    // chunk swizzle.  d = 128 (a row spans all 64 banks): rows 0..15 get 16 different
    // values, and rows 4m .. 4m + 3 different multiples of 4 (different 64-byte quads).
    // d = 64 (two rows per 256 bytes): the same for the even and for the odd rows.
    // Depends on bits 0-3 of the row only, so rows r and r + 16 share it.
    static __device__ __forceinline__ int swz(int r) {
        return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    }

    // A operand from the rows of a block: lane reads row sigma(l32), k-step cc.
    static __device__ __forceinline__ v8 row_frag(uint32_t base, int l32, int g, int cc) {
        const int pr = swap_bits23(l32);
        return as_v8(*(const lds_u32x4_t *)(uintptr_t)(base + pr * ROWB + (((2 * cc + g) ^ swz(pr)) << 4)));
    }
    // B operand from row n = row0 + l32 of a block (natural order), k-step cc.
    static __device__ __forceinline__ v8 col_frag(uint32_t base, int row, int g, int cc) {
        return as_v8(*(const lds_u32x4_t *)(uintptr_t)(base + row * ROWB + (((2 * cc + g) ^ swz(row)) << 4)));
    }
    // A operand X^T (32 columns of d in block db, 16 rows kc of the block) by transposing reads.
    static __device__ __forceinline__ v8 tr_frag(uint32_t base, int lane, int db, int kc) {
        const int j16 = lane & 15, grp = lane >> 4;
        const int r = 8 * (grp >> 1) + (j16 >> 2);  // and r + 4; both plus 16 kc
        const int cl = 2 * (grp & 1) + ((j16 & 3) >> 1);
        const uint32_t a = base + 16 * kc * ROWB + 8 * (j16 & 1);
        const uint32_t alo = a + r * ROWB + (((4 * db + cl) ^ swz(r)) << 4);
        const uint32_t ahi = a + (r + 4) * ROWB + (((4 * db + cl) ^ swz(r + 4)) << 4);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(alo));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(ahi));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        return as_v8((u32x4_t){l2[0], l2[1], h2[0], h2[1]});
    }
    // Load `rows` rows starting at row0 of a [N, D] head into an LDS block (chunk-swizzled),
    // rows past N - 1 read row N - 1.  The block is split into 1 KiB loads; this wave issues
    // loads first .. first + count - 1.
    static __device__ __forceinline__ void load_rows(const char *head, int row0, int N, uint32_t lds, int first,
                                                     int count, int lane) {
        for (int j = 0; j < count; ++j) {
            const int s = (first + j) * 64 + lane;
            const int r = s / CH, p = s % CH;
            const int src = min(row0 + r, N - 1) - row0;
            dma_to_lds16(head + (size_t)row0 * ROWB, (uint32_t)src * ROWB + ((p ^ swz(r)) << 4),
                         lds + (first + j) * 1024);
        }
    }
    // Epilogue store of a D x 32 accumulator (register i of block b = column
    // 32 b + 8 (i >> 2) + 4 g + (i & 3), lane = row), times mul, as 16-byte stores
    // after one exchange between lane halves (as in the forward).
    static __device__ __forceinline__ void store_rows(const f32x16_t (&acc)[DB], float mul, uint16_t *row_ptr,
                                                      bool valid, int g) {
        auto partner = [&](uint32_t x) -> uint32_t {
            const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
            return g ? r[0] : r[1];
        };
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                u32x2_t mine[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int i = 4 * (k + t);
                    mine[t][0] = M::pack(acc[b][i + 0] * mul, acc[b][i + 1] * mul);
                    mine[t][1] = M::pack(acc[b][i + 2] * mul, acc[b][i + 3] * mul);
                }
                const u32x2_t give = g ? mine[0] : mine[1];
                const u32x2_t got = {partner(give[0]), partner(give[1])};
                const u32x2_t lo = g ? got : mine[0], hi = g ? mine[1] : got;
                if (valid)
                    *reinterpret_cast<u32x4_t *>(row_ptr + b * 32 + 8 * (k + g)) = (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
            }
    }
};

template <int VMCNT>
__device__ __forceinline__ void bwd_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(VMCNT) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------- dQ

template <typename T, int D, bool CAUSAL>
struct BwdDq : BwdCommon<T, D> {
    typedef BwdCommon<T, D> C;
    using C::ROWB;
    using C::DB;
    using C::DC;
    typedef typename C::M M;
    typedef typename C::v8 v8;
    static constexpr int NW = 4, THREADS = NW * 64;
    static constexpr int BR = NW * 32;           // query rows per workgroup
    static constexpr int BK = 32;                // keys per streamed block
    static constexpr int BLK_B = BK * ROWB;      // one K or V block
    static constexpr int STAGE_B = 2 * BLK_B;    // K block then V block
    static constexpr int LDS_B = 2 * STAGE_B;    // two stages
    static constexpr int LOADS = STAGE_B / 1024 / NW;
    static_assert(LOADS * 1024 * NW == STAGE_B, "block loads split evenly over the waves");

    static __device__ void run(const BwdArgs &a) {
        extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
        const int N = a.N;
        int bh, qt;
        if (CAUSAL) {  // longest tiles (last query rows) first
            const int n_bh = a.total / a.n_tiles;
            bh = blockIdx.x % n_bh;
            qt = a.n_tiles - 1 - blockIdx.x / n_bh;
        } else {
            const int logical = xcd_contiguous(blockIdx.x, a.total);
            bh = logical / a.n_tiles;
            qt = logical - bh * a.n_tiles;
        }
        const size_t head = (size_t)bh * (size_t)N * D;
        const char *Kh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + head);
        const char *Vh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + head);
        const int tid = threadIdx.x;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
        const int q0 = qt * BR + 32 * w, q = q0 + l32, qc = min(q, N - 1);

        // Q^T and dO^T of this wave's rows as B operands (rows past the end are zero)
        v8 qT[DC], doT[DC];
        {
            const uint32_t keep = q < N ? 0xffffffffu : 0u;
            const uint16_t *qr = static_cast<const uint16_t *>(a.q) + head + (size_t)qc * D + g * 8;
            const uint16_t *dr = static_cast<const uint16_t *>(a.dout) + head + (size_t)qc * D + g * 8;
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                qT[cc] = C::as_v8(*reinterpret_cast<const u32x4_t *>(qr + cc * 16) & keep);
                doT[cc] = C::as_v8(*reinterpret_cast<const u32x4_t *>(dr + cc * 16) & keep);
            }
        }
        const float nlse = -a.lse[(size_t)bh * N + qc] * kLog2e;
        const float Dq = a.delta[(size_t)bh * N + qc];
        f32x16_t acc[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b) acc[b] = (f32x16_t){};

        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
        const int nkb_all = (N + BK - 1) / BK;
        const int nkb = CAUSAL ? min(nkb_all, (min(qt * BR + BR, N) - 1) / BK + 1) : nkb_all;
        const bool active = q0 < N;
        const int my_last = CAUSAL ? min(q0 + 31, N - 1) / BK : nkb - 1;
        // visible keys of a block: key offset <= lim (causal: key <= q and key < N)
        const int last_key = CAUSAL ? qc : N - 1;

        // this wave's share of a stage: 1 KiB loads w * LOADS .. of the [K | V] block pair
        auto issue = [&](int j) {
            const uint32_t st = lds0 + (j & 1) * STAGE_B;
            constexpr int PER = BLK_B / 1024;  // loads per block
#pragma unroll
            for (int t = 0; t < LOADS; ++t) {
                const int ch = w * LOADS + t;
                const bool isv = ch >= PER;
                C::load_rows(isv ? Vh : Kh, j * BK, N, st + (isv ? BLK_B : 0), ch % PER, 1, lane);
            }
        };

        issue(0);
        for (int j = 0; j < nkb; ++j) {
            if (j + 1 < nkb) {
                issue(j + 1);
                bwd_barrier<LOADS>();
            } else {
                bwd_barrier<0>();
            }
            if (active && j <= my_last) {
                const uint32_t kb = lds0 + (j & 1) * STAGE_B, vb = kb + BLK_B;
                f32x16_t s = (f32x16_t){}, dp = (f32x16_t){};
#pragma unroll
                for (int cc = 0; cc < DC; ++cc) s = M::mma(C::row_frag(kb, l32, g, cc), qT[cc], s);
#pragma unroll
                for (int cc = 0; cc < DC; ++cc) dp = M::mma(C::row_frag(vb, l32, g, cc), doT[cc], dp);
                // fragment reads run three ahead of the products that use them
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 3, 0);
                sched_mfma_reads<2 * DC, 1, 2 * DC - 3>();
                // register i of half g holds key j BK + 16 (i >> 3) + 8 g + (i & 7)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = fast_exp2(fmaf(s[i], a.c, nlse));
                // only blocks not wholly visible to every query of the wave are masked
                if ((CAUSAL && j * BK + BK - 1 > q0) || j * BK + BK > N) {
                    const int lim = last_key - j * BK - 8 * g;
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[i] = 16 * (i >> 3) + (i & 7) <= lim ? s[i] : 0.f;
                }
                uint32_t pk[2][4];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i0 = 8 * h + 2 * e;
                        pk[h][e] = M::pack(s[i0] * (dp[i0] - Dq), s[i0 + 1] * (dp[i0 + 1] - Dq));
                    }
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const v8 ds = C::as_v8((u32x4_t){pk[kc][0], pk[kc][1], pk[kc][2], pk[kc][3]});
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[db] = M::mma(C::tr_frag(kb, lane, db, kc), ds, acc[db]);
                }
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
                sched_mfma_reads<2 * DB, 2, 4 * DB - 4>();
            }
            bwd_barrier<0>();
        }
        uint16_t *dq = static_cast<uint16_t *>(a.dq) + head + (size_t)qc * D;
        C::store_rows(acc, a.scale, dq, q < N, g);
    }
};

// ------------------------------------------------------------------- dK, dV

template <typename T, int D, bool CAUSAL>
struct BwdDkv : BwdCommon<T, D> {
    typedef BwdCommon<T, D> C;
    using C::ROWB;
    using C::DB;
    using C::DC;
    typedef typename C::M M;
    typedef typename C::v8 v8;
    // Two groups of four waves share the workgroup's 128 keys (wave w & 3 of either
    // group owns keys 32 (w & 3) ..) and take alternate query blocks, so that each SIMD
    // runs two waves; their partial dK and dV are added through LDS at the end.
    static constexpr int NW = 8, GW = 4, THREADS = NW * 64;
    static constexpr int BKV = GW * 32;              // key rows per workgroup
    static constexpr int BQ = 32;                    // queries per streamed block
    // The resident K and V tiles are read only row-wise (as B operands), so they use a
    // padded row of CH + 1 chunks instead of the swizzle: sixteen consecutive rows at one
    // chunk still fall on sixteen bank groups, and a lane's fragments for successive
    // k-steps sit at fixed offsets from one address.
    static constexpr int PROW = ROWB + 16;           // padded row bytes
    static constexpr int KV_B = 2 * BKV * PROW;      // resident K then V tile
    static constexpr int BLK_B = BQ * ROWB;          // one Q or dO block
    static constexpr int STAGE_B = 2 * BLK_B + 256;  // Q, dO, then L (32 floats) and D (32 floats)
    static constexpr int RING_B = 2 * STAGE_B;       // two stages per group
    static constexpr int LDS_B = KV_B + 2 * RING_B;
    static constexpr int LOADS = 2 * BLK_B / 1024 / GW;  // Q/dO loads per wave and block
    static constexpr int KV_LOADS = KV_B / 1024;     // 1 KiB loads of both tiles (any wave)
    static constexpr int PART_B = GW * DB * 16 * 64 * 4;  // one group's dK (or dV) partials, fp32
    static_assert(LOADS * 1024 * GW == 2 * BLK_B && KV_LOADS * 1024 == KV_B && KV_LOADS % 2 == 0,
                  "whole loads");
    static_assert(PART_B <= KV_B && PART_B <= 2 * RING_B, "partials fit in the freed LDS");

    static __device__ __forceinline__ void put_part(const f32x16_t (&acc)[DB], uint32_t base, int lane) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                *(lds_u32x4_t *)(uintptr_t)(base + (b * 4 + t) * 1024 + lane * 16) =
                    (u32x4_t){__float_as_uint(acc[b][4 * t]), __float_as_uint(acc[b][4 * t + 1]),
                              __float_as_uint(acc[b][4 * t + 2]), __float_as_uint(acc[b][4 * t + 3])};
    }
    static __device__ __forceinline__ void add_part(f32x16_t (&acc)[DB], uint32_t base, int lane) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4_t x = *(const lds_u32x4_t *)(uintptr_t)(base + (b * 4 + t) * 1024 + lane * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[b][4 * t + e] += __uint_as_float(x[e]);
            }
    }

    static __device__ void run(const BwdArgs &a) {
        extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
        const int N = a.N;
        int bh, kt;
        if (CAUSAL) {  // longest tiles (first key rows) first
            const int n_bh = a.total / a.n_tiles;
            bh = blockIdx.x % n_bh;
            kt = blockIdx.x / n_bh;
        } else {
            const int logical = xcd_contiguous(blockIdx.x, a.total);
            bh = logical / a.n_tiles;
            kt = logical - bh * a.n_tiles;
        }
        const size_t head = (size_t)bh * (size_t)N * D;
        const char *Kh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + head);
        const char *Vh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + head);
        const char *Qh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.q) + head);
        const char *dOh = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.dout) + head);
        const float *lse_h = a.lse + (size_t)bh * N;
        const float *del_h = a.delta + (size_t)bh * N;
        const int tid = threadIdx.x;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int grp = w / GW, wk = w % GW;    // group, wave within the group
        const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
        const int kv0 = kt * BKV;               // first key of the workgroup
        const int k0 = kv0 + 32 * wk, key = k0 + l32;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
        const uint32_t kres = lds0, ring = lds0 + KV_B + grp * RING_B;
        // this lane's B-operand row of the resident tiles: key row 32 wk + l32, chunk g
        const uint32_t kv_lane = kres + (32 * wk + l32) * PROW + 16 * g;

        f32x16_t dk[DB], dv[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            dk[b] = (f32x16_t){};
            dv[b] = (f32x16_t){};
        }

        // resident K and V rows kv0 .. kv0 + BKV - 1: 1 KiB loads w, w + NW, ...; slot s of a
        // tile is row s / (CH + 1), chunk s % (CH + 1); the pad chunk CH loads chunk 0 again
#pragma unroll
        for (int t0 = 0; t0 < KV_LOADS; t0 += NW) {
            const int t = __builtin_amdgcn_readfirstlane(t0 + w);
            if (t >= KV_LOADS) break;
            constexpr int PER = KV_LOADS / 2;  // loads per tile
            const bool isv = t >= PER;
            const int sl = (t % PER) * 64 + lane;
            const int r = sl / (C::CH + 1), p = sl % (C::CH + 1);
            const int src = min(kv0 + r, N - 1) - kv0;
            dma_to_lds16((isv ? Vh : Kh) + (size_t)kv0 * ROWB, (uint32_t)src * ROWB + (p < C::CH ? p << 4 : 0),
                         kres + (isv ? BKV * PROW : 0) + (t % PER) * 1024);
        }
        const int nqb = (N + BQ - 1) / BQ;
        const int qb0 = CAUSAL ? kv0 / BQ : 0;      // queries before kv0 see none of these keys
        const int my_first = CAUSAL ? k0 / BQ : 0;  // first block with a query >= this wave's first key
        const int iters = (nqb - qb0 + 1) / 2;      // group grp takes blocks qb0 + 2 it + grp
        const bool active = k0 < N;
        auto issue = [&](int i, int it) {
            const uint32_t st = ring + (it & 1) * STAGE_B;
            constexpr int PER = BLK_B / 1024;
#pragma unroll
            for (int t = 0; t < LOADS; ++t) {
                const int ch = wk * LOADS + t;
                const bool isd = ch >= PER;
                C::load_rows(isd ? dOh : Qh, i * BQ, N, st + (isd ? BLK_B : 0), ch % PER, 1, lane);
            }
            // L of the block's 32 queries (lanes 0-31) and D (lanes 32-63); every wave of
            // the group issues the same load (identical bytes), so all count the same loads
            const int qi = min(i * BQ + l32, N - 1);
            dma_to_lds4(g ? (const void *)(del_h + qi) : (const void *)(lse_h + qi), st + 2 * BLK_B);
        };

        if (qb0 + grp < nqb) issue(qb0 + grp, 0);
        for (int it = 0; it < iters; ++it) {
            const int i = qb0 + 2 * it + grp;
            if (i + 2 < nqb) {
                issue(i + 2, it + 1);
                bwd_barrier<LOADS + 1>();
            } else {
                bwd_barrier<0>();
            }
            if (active && i < nqb && i >= my_first) {
                const uint32_t qb = ring + (it & 1) * STAGE_B, ob = qb + BLK_B, lb = qb + 2 * BLK_B;
                f32x16_t s = (f32x16_t){}, dp = (f32x16_t){};
#pragma unroll
                for (int cc = 0; cc < DC; ++cc)
                    s = M::mma(C::row_frag(qb, l32, g, cc),
                               C::as_v8(*(const lds_u32x4_t *)(uintptr_t)(kv_lane + 32 * cc)), s);
#pragma unroll
                for (int cc = 0; cc < DC; ++cc)
                    dp = M::mma(C::row_frag(ob, l32, g, cc),
                                C::as_v8(*(const lds_u32x4_t *)(uintptr_t)(kv_lane + BKV * PROW + 32 * cc)), dp);
                // fragment reads run four ahead of the products that use them
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
                sched_mfma_reads<2 * DC, 2, 4 * DC - 4>();
                // register i of half g holds query i BQ + 16 (i >> 3) + 8 g + (i & 7); lane = key
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int qo = 16 * h + 8 * g;  // first query offset of these 8 registers
                    const u32x4_t lv[2] = {*(const lds_u32x4_t *)(uintptr_t)(lb + 4 * qo),
                                           *(const lds_u32x4_t *)(uintptr_t)(lb + 4 * qo + 16)};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        s[8 * h + e] = fast_exp2(fmaf(s[8 * h + e], a.c, -__uint_as_float(lv[e >> 2][e & 3]) * kLog2e));
                }
                // only blocks where some query does not see some key of the wave are masked
                if ((CAUSAL && i * BQ < k0 + 31) || i * BQ + BQ > N) {
#pragma unroll
                    for (int ii = 0; ii < 16; ++ii) {
                        const int qidx = i * BQ + 16 * (ii >> 3) + 8 * g + (ii & 7);
                        s[ii] = qidx < N && (!CAUSAL || qidx >= key) ? s[ii] : 0.f;
                    }
                }
                uint32_t pp[2][4], pd[2][4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int qo = 16 * h + 8 * g;
                    const u32x4_t dv4[2] = {*(const lds_u32x4_t *)(uintptr_t)(lb + 128 + 4 * qo),
                                            *(const lds_u32x4_t *)(uintptr_t)(lb + 128 + 4 * qo + 16)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ii = 8 * h + 2 * e;
                        const float D0 = __uint_as_float(dv4[e >> 1][(2 * e) & 3]);
                        const float D1 = __uint_as_float(dv4[e >> 1][(2 * e + 1) & 3]);
                        pp[h][e] = M::pack(s[ii], s[ii + 1]);
                        pd[h][e] = M::pack(s[ii] * (dp[ii] - D0), s[ii + 1] * (dp[ii + 1] - D1));
                    }
                }
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const v8 P = C::as_v8((u32x4_t){pp[kc][0], pp[kc][1], pp[kc][2], pp[kc][3]});
                    const v8 dS = C::as_v8((u32x4_t){pd[kc][0], pd[kc][1], pd[kc][2], pd[kc][3]});
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        dv[db] = M::mma(C::tr_frag(ob, lane, db, kc), P, dv[db]);
                        dk[db] = M::mma(C::tr_frag(qb, lane, db, kc), dS, dk[db]);
                    }
                }
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
                sched_mfma_reads<4 * DB, 2, 8 * DB - 4>();
            }
            bwd_barrier<0>();
        }
        // a workgroup with no query block still waits for its resident loads
        bwd_barrier<0>();
        // group 1 hands its dK partials to group 0 (in the freed rings), group 0 its dV
        // partials to group 1 (in the freed K/V tile); each then finishes one output
        const uint32_t part_k = lds0 + KV_B + wk * (PART_B / GW), part_v = lds0 + wk * (PART_B / GW);
        if (grp == 1)
            put_part(dk, part_k, lane);
        else
            put_part(dv, part_v, lane);
        bwd_barrier<0>();
        const int kc_ = min(key, N - 1);
        if (grp == 0) {
            add_part(dk, part_k, lane);
            uint16_t *dkp = static_cast<uint16_t *>(a.dk) + head + (size_t)kc_ * D;
            C::store_rows(dk, a.scale, dkp, key < N, g);
        } else {
            add_part(dv, part_v, lane);
            uint16_t *dvp = static_cast<uint16_t *>(a.dv) + head + (size_t)kc_ * D;
            C::store_rows(dv, 1.f, dvp, key < N, g);
        }
    }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdArgs a) {
    BwdDq<T, D, CAUSAL>::run(a);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkv_kernel(BwdArgs a) {
    BwdDkv<T, D, CAUSAL>::run(a);
}

}  // namespace attn
