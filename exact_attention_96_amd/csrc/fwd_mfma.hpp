// Fused attention forward on the gfx950 matrix cores (bf16 / fp16 inputs).
//
// One workgroup owns one (batch*head, query tile) pair: BR = 128 query rows,
// 32 per wave, the outer loop of "Understand FlashAttention", section
// "FlashAttention".  The inner loop walks the key/value sequence in BC = 64
// column blocks staged in LDS.  Per block, each wave applies the update of
// that page's section "两块情况的完整推导" (steps 5-7): new row max, rescale
// factor e^{m_old - m_new}, row sum, rescaled partial output plus P V; after
// the last block it divides by the row sum (step 8) and writes
// lse = m + log l (appendix "附：数值稳定的logsumexp(L)推导").
//
// Layout trick.  The first product is evaluated transposed, S^T = K Q^T, with
// the 32x32x16 MFMA: its accumulator gives every lane one query (lane % 32)
// and 16 keys, so the row max and row sum are in-lane reductions plus one
// exchange with lane ^ 32.  Keys are fed to the A operand in the order
// sigma(r) = r with bits 2 and 3 swapped; then the 8 accumulator registers
// i = 8h .. 8h+7 of lane group g hold the 8 consecutive keys 16h + 8g .. +7,
// which is exactly the B-operand layout the second product O^T = V^T P^T
// needs.  P therefore goes from the softmax straight into the MFMA, and the
// per-query rescale of O^T is a per-lane multiply.  V is stored transposed in
// LDS (d rows of keys) so its A-operand fragments are 16-byte reads.
//
// The exponentials use exp2 with the scale folded into log2(e): t = s * c,
// c = scale * log2(e), p = 2^{t - m}.
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

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
    typedef bf16x8_t v8;
    typedef bf16x4_t v4;
    static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<_Float16> {
    typedef f16x8_t v8;
    typedef f16x4_t v4;
    static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Swap bits 2 and 3 of a row index inside a 32-row block (an involution).
__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <typename T, int D, bool CAUSAL>
struct MfmaFwd {
    static constexpr int NW = 4;           // waves per workgroup
    static constexpr int QW = 32;          // query rows per wave
    static constexpr int BR = NW * QW;     // query rows per workgroup
    static constexpr int BC = 64;          // keys per inner iteration
    static constexpr int THREADS = NW * 64;
    static constexpr int KSTRIDE = D + 8;  // K tile row pitch (elements): 16 B pad, conflict-free
    static constexpr int VSTRIDE = BC + 8; // V^T tile row pitch (elements)
    static constexpr int DB = D / 32;      // 32-wide d blocks of the output
    static constexpr int DC = D / 16;      // 16-deep d chunks of the first product
    typedef typename Mfma<T>::v8 v8;
    typedef typename Mfma<T>::v4 v4;

    static __device__ __forceinline__ v8 as_v8(u32x4_t x) { return __builtin_bit_cast(v8, x); }

    static __device__ void run(const FwdArgs &a) {
        __shared__ __attribute__((aligned(16))) uint16_t k_lds[BC * KSTRIDE];
        __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VSTRIDE];

        const int N = a.N;
        const int logical = xcd_contiguous(blockIdx.x, a.total);
        const int bh = logical / a.n_qtiles;
        const int t = logical - bh * a.n_qtiles;
        // causal: the longest rows first, so the short ones fill the tail of the grid
        const int qt = CAUSAL ? a.n_qtiles - 1 - t : t;
        const size_t head = (size_t)bh * (size_t)N * D;
        const uint16_t *Qh = static_cast<const uint16_t *>(a.q) + head;
        const uint16_t *Kh = static_cast<const uint16_t *>(a.k) + head;
        const uint16_t *Vh = static_cast<const uint16_t *>(a.v) + head;

        const int tid = threadIdx.x;
        const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
        const int q0 = qt * BR + w * QW;      // first query row of this wave
        const int qrow = q0 + l32;            // this lane's query row

        // Q^T as the B operand: lane holds Q[qrow][16c + 8g .. +7] for every chunk c.
        v8 qf[DC];
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (qrow < N) x = *reinterpret_cast<const u32x4_t *>(Qh + (size_t)qrow * D + c * 16 + g * 8);
            qf[c] = as_v8(x);
        }

        f32x16_t acc[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
        float m = -INFINITY;  // running max of t = s * c (log2 domain)
        float lsum = 0.f;     // this lane's share of the running row sum

        const int n_kv_all = (N + BC - 1) / BC;
        const int n_kv = CAUSAL ? min(n_kv_all, (qt * BR + BR - 1) / BC + 1) : n_kv_all;

        for (int j = 0; j < n_kv; ++j) {
            const int k0 = j * BC;
            __syncthreads();  // every wave is done with the previous tile
            // K tile -> LDS, rows permuted by sigma inside each 32-row block.
            for (int idx = tid; idx < BC * D / 8; idx += THREADS) {
                const int r = idx / (D / 8), cc = idx % (D / 8);
                u32x4_t x = {0u, 0u, 0u, 0u};
                if (k0 + r < N) x = *reinterpret_cast<const u32x4_t *>(Kh + (size_t)(k0 + r) * D + cc * 8);
                const int rr = (r & ~31) | swap_bits23(r & 31);
                *reinterpret_cast<u32x4_t *>(k_lds + rr * KSTRIDE + cc * 8) = x;
            }
            // V tile -> LDS transposed: vt[d][key].  Lane pairs up keys 2*l32, 2*l32+1.
            for (int cc = w * 2 + g; cc < D / 8; cc += 2 * NW) {
                const int r0 = 2 * l32;
                u32x4_t x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
                if (k0 + r0 < N) x0 = *reinterpret_cast<const u32x4_t *>(Vh + (size_t)(k0 + r0) * D + cc * 8);
                if (k0 + r0 + 1 < N) x1 = *reinterpret_cast<const u32x4_t *>(Vh + (size_t)(k0 + r0 + 1) * D + cc * 8);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = (x0[e] & 0xffffu) | (x1[e] << 16);
                    const uint32_t hi = (x0[e] >> 16) | (x1[e] & 0xffff0000u);
                    *reinterpret_cast<uint32_t *>(vt_lds + (cc * 8 + 2 * e) * VSTRIDE + r0) = lo;
                    *reinterpret_cast<uint32_t *>(vt_lds + (cc * 8 + 2 * e + 1) * VSTRIDE + r0) = hi;
                }
            }
            __syncthreads();

            if (CAUSAL && k0 > q0 + QW - 1) continue;  // every key of the tile is after every row

            // S^T = K Q^T for the two 32-key blocks of the tile.
            f32x16_t s[2];
            bool on[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                on[kb] = (k0 + kb * 32 < N) && (!CAUSAL || k0 + kb * 32 <= q0 + QW - 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
                if (on[kb]) {
#pragma unroll
                    for (int c = 0; c < DC; ++c) {
                        const v8 kf = as_v8(*reinterpret_cast<const u32x4_t *>(
                            k_lds + (kb * 32 + l32) * KSTRIDE + c * 16 + g * 8));
                        s[kb] = Mfma<T>::mma(kf, qf[c], s[kb]);
                    }
                }
            }

            // Scale to the log2 domain and mask.  Register i of block kb is key
            // k0 + 32 kb + (i & 7) + 8 g + 16 (i >> 3).
            const bool need_mask = (CAUSAL && k0 + BC - 1 > q0) || (k0 + BC > N);
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = s[kb][i] * a.c;
                    if (need_mask) {
                        const int key = k0 + kb * 32 + (i & 7) + 8 * g + 16 * (i >> 3);
                        const bool dead = !on[kb] || key >= N || (CAUSAL && key > qrow);
                        x = dead ? -INFINITY : x;
                    } else if (!on[kb]) {
                        x = -INFINITY;
                    }
                    s[kb][i] = x;
                    mx = fmaxf(mx, x);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // a row with no key yet
            const float alpha = fast_exp2(m - m_use);
            m = m_new;

            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(s[kb][i] - m_use);
                    s[kb][i] = p;
                    rs += p;
                }
            lsum = lsum * alpha + rs;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;

            // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (!on[kb]) continue;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    v8 pf;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pf[e] = static_cast<T>(s[kb][8 * h + e]);
#pragma unroll
                    for (int b = 0; b < DB; ++b) {
                        const v8 vf = as_v8(*reinterpret_cast<const u32x4_t *>(
                            vt_lds + (b * 32 + l32) * VSTRIDE + kb * 32 + 16 * h + 8 * g));
                        acc[b] = Mfma<T>::mma(vf, pf, acc[b]);
                    }
                }
            }
        }

        // Epilogue: O = O~ / l, lse = (m + log2 l) ln 2.  Register i of block b is
        // output column 32 b + 8 (i >> 2) + 4 g + (i & 3) of row qrow.
        const float ltot = lsum + __shfl_xor(lsum, 32);
        if (qrow < N) {
            const float inv = 1.f / ltot;
            uint16_t *Oh = static_cast<uint16_t *>(a.o) + head + (size_t)qrow * D;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int quad = 0; quad < 4; ++quad) {
                    v4 y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = static_cast<T>(acc[b][quad * 4 + e] * inv);
                    *reinterpret_cast<v4 *>(Oh + b * 32 + quad * 8 + 4 * g) = y;
                }
            if (g == 0) a.lse[(size_t)bh * N + qrow] = (m + fast_log2(ltot)) * kLn2;
        }
    }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2)
void attn_fwd_mfma_kernel(FwdArgs a) {
    static_assert(MfmaFwd<T, D, CAUSAL>::THREADS == 256, "launch bounds assume 256 threads");
    MfmaFwd<T, D, CAUSAL>::run(a);
}

}  // namespace attn
