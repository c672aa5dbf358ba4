// Attention forward for fp32 inputs, entirely in fp32 on the vector ALUs.
//
// Same recurrence as the matrix-core kernel ("Understand FlashAttention",
// sections "FlashAttention" and "两块情况的完整推导"): a workgroup of one wave
// owns 32 query rows; keys and values stream through LDS 32 rows at a time;
// each row keeps its running max, running sum and unnormalised output in
// registers and rescales them by e^{m_old - m_new} once per key block.
// Lane l serves query row l % 32 and head-dim half l / 32, so a dot product is
// two half sums joined by one cross-lane exchange.  This path exists for
// accuracy (every product and sum in fp32), not speed.
#pragma once

#include "common.hpp"
#include "fwd_mfma.hpp"  // FwdArgs

namespace attn {

// MASK: keys are also hidden by the caller's bit mask (FwdArgs::mask).
template <int D, bool CAUSAL, bool MASK = false>
struct F32Fwd {
    static constexpr int QW = 32;  // query rows per workgroup
    static constexpr int BK = 32;  // keys per LDS block
    static constexpr int DH = D / 2;
    static constexpr int THREADS = 64;

    static __device__ void run(const FwdArgs &a) {
        __shared__ __attribute__((aligned(16))) float k_lds[BK * D];
        __shared__ __attribute__((aligned(16))) float v_lds[BK * D];

        const int Nq = a.Nq, Nk = a.Nk, off = CAUSAL ? a.off : 0;
        const int logical = xcd_contiguous(blockIdx.x, a.total);
        const int bh = logical / a.n_qtiles;
        const int t = logical - bh * a.n_qtiles;
        const int qt = CAUSAL ? a.n_qtiles - 1 - t : t;
        const size_t head = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
        const float *Qh = static_cast<const float *>(a.q) + head;
        const float *Kh = static_cast<const float *>(a.k) + headk;
        const float *Vh = static_cast<const float *>(a.v) + headk;

        const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
        const int q0 = qt * QW;
        const int qrow = q0 + l32;

        float qv[DH], acc[DH];
#pragma unroll
        for (int e = 0; e < DH; ++e) {
            qv[e] = qrow < Nq ? Qh[(size_t)qrow * D + g * DH + e] : 0.f;
            acc[e] = 0.f;
        }
        float m = -INFINITY, l = 0.f;

        // the row's mask words (MASK); rows past the end read row Nq - 1
        const uint64_t *mrow = nullptr;
        if (MASK) {
            const int b = bh / a.H, hh = bh - b * a.H;
            const size_t mhead = (size_t)b * (size_t)a.mask_sb + (size_t)hh * (size_t)a.mask_sh;
            mrow = a.mask + (mhead * (size_t)Nq + (size_t)min(qrow, Nq - 1)) * (size_t)a.mask_w;
        }
        // causal: the workgroup's last row sees keys up to its index + off
        const int n_kv_all = (Nk + BK - 1) / BK;
        const int last_key = min(q0 + QW, Nq) - 1 + off;
        const int n_kv = CAUSAL ? (last_key < 0 ? 0 : min(n_kv_all, last_key / BK + 1)) : n_kv_all;
        for (int j = 0; j < n_kv; ++j) {
            const int k0 = j * BK;
            __syncthreads();
            for (int idx = lane; idx < BK * D / 4; idx += THREADS) {
                const int r = idx / (D / 4), cc = idx % (D / 4);
                f32x4_t kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
                if (k0 + r < Nk) {
                    kx = *reinterpret_cast<const f32x4_t *>(Kh + (size_t)(k0 + r) * D + cc * 4);
                    vx = *reinterpret_cast<const f32x4_t *>(Vh + (size_t)(k0 + r) * D + cc * 4);
                }
                *reinterpret_cast<f32x4_t *>(k_lds + r * D + cc * 4) = kx;
                *reinterpret_cast<f32x4_t *>(v_lds + r * D + cc * 4) = vx;
            }
            __syncthreads();

            // BK = 32 keys from k0 (a multiple of 32) lie in one mask word
            const uint32_t mbits = MASK ? (uint32_t)(mrow[k0 / 64] >> (k0 % 64)) : 0xffffffffu;
            float s[BK];
            float mx = -INFINITY;
#pragma unroll
            for (int jj = 0; jj < BK; ++jj) {
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < DH; ++e) part = fmaf(qv[e], k_lds[jj * D + g * DH + e], part);
                float x = (part + __shfl_xor(part, 32)) * a.c;
                const int key = k0 + jj;
                if (key >= Nk || (CAUSAL && key > qrow + off) || !((mbits >> jj) & 1u)) x = -INFINITY;
                s[jj] = x;
                mx = fmaxf(mx, x);
            }
            const float m_new = fmaxf(m, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            m = m_new;
            float rs = 0.f;
#pragma unroll
            for (int jj = 0; jj < BK; ++jj) {
                s[jj] = fast_exp2(s[jj] - m_use);
                rs += s[jj];
            }
            l = l * alpha + rs;
#pragma unroll
            for (int e = 0; e < DH; ++e) {
                float o = acc[e] * alpha;
#pragma unroll
                for (int jj = 0; jj < BK; ++jj) o = fmaf(s[jj], v_lds[jj * D + g * DH + e], o);
                acc[e] = o;
            }
        }

        if (qrow < Nq) {  // a row that saw no key (l = 0, m = -inf): O = 0, lse = -inf
            const float inv = l > 0.f ? 1.f / l : 0.f;
            float *Oh = static_cast<float *>(a.o) + head + (size_t)qrow * D + g * DH;
#pragma unroll
            for (int e = 0; e < DH; ++e) Oh[e] = acc[e] * inv;
            if (g == 0) a.lse[(size_t)bh * Nq + qrow] = (m + fast_log2(l)) * kLn2;
        }
    }
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(64)
void attn_fwd_f32_kernel(FwdArgs a) {
    F32Fwd<D, CAUSAL, MASK>::run(a);
}

}  // namespace attn
