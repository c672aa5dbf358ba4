// Causal linear attention forward (fp32), a second workload beside softmax attention.
//
// "hqwc.cn" notes on the fast-transformers linear attention CUDA kernels: the
// similarity is phi(q) . phi(k) with phi(x) = elu(x) + 1 (section 0x0); the causal
// module returns causal_dot_product(phi(Q), phi(K), V) scaled by
// 1 / (phi(q_j) . sum_{t<=j} phi(k_t) + eps) (section 0x1); the causal dot product
// is V'_j = sum_{t<=j} (q_j . k_t) v_t, computed by carrying the state
// S_j = sum_{t<=j} k_t v_t^T and taking q_j S_j (section 0x2).
//
// Decomposition for gfx950.  One workgroup of 256 threads per (batch * head, slice
// of 16 value columns); thread (e-group g, column m) keeps E / 16 entries of the
// state S[e][m] (e = g * E/16 + i) and of the key sum z[e] in registers for the
// whole sequence.  Tokens go through LDS in chunks of T: phi is applied on the way
// in, every thread advances its state token by token and writes its partial
// readouts q_t . S (and q_t . z) to LDS, and after the chunk each output is the sum
// of its 16 partials.  The scan is sequential per workgroup; the grid holds
// B * H * M / 16 of them.  HBM traffic is one read of q, k (per column slice; the
// slices of a head share them through L2), v and one write of o.
#pragma once

#include "common.hpp"

namespace attn {

struct LinArgs {
    const float *q, *k, *v;
    float *o;
    int N, M;            // sequence length, value width
    int n_mslices;       // M / 16
    float eps;           // added to the normaliser (feature_map only)
    int feature_map;     // 0: causal dot product of q, k as given; 1: phi = elu + 1 and the normaliser
};

template <int E>
struct LinFwd {
    static constexpr int T = 32;          // tokens per chunk
    static constexpr int MS = 16;         // value columns per workgroup
    static constexpr int EG = 16;         // e-groups
    static constexpr int EPT = E / EG;    // state rows per thread
    static constexpr int THREADS = EG * MS;
    // LDS: q and k chunks [T][E], v chunk [T][MS], partial numerators [T][EG][MS],
    // partial denominators [T][EG]
    static constexpr int QS = 0, KS = QS + T * E, VS = KS + T * E, RN = VS + T * MS, RD = RN + T * EG * MS;
    static constexpr int LDS_FLOATS = RD + T * EG;
    static constexpr int LDS_B = LDS_FLOATS * 4;
    static_assert(E % EG == 0 && E % 4 == 0 && T % (THREADS / MS) == 0, "tile shape");
    static_assert(LDS_B <= 160 * 1024, "LDS budget");

    static __device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }

    static __device__ void run(const LinArgs &a) {
        extern __shared__ __attribute__((aligned(16))) float lds[];
        const int N = a.N, M = a.M;
        const int bh = blockIdx.x / a.n_mslices, ms = blockIdx.x - bh * a.n_mslices;
        const float *Qh = a.q + (size_t)bh * N * E;
        const float *Kh = a.k + (size_t)bh * N * E;
        const float *Vh = a.v + (size_t)bh * N * M + ms * MS;
        float *Oh = a.o + (size_t)bh * N * M + ms * MS;
        const int tid = threadIdx.x, m = tid % MS, g = tid / MS;
        const bool fm = a.feature_map != 0;

        float S[EPT], z[EPT];
#pragma unroll
        for (int i = 0; i < EPT; ++i) S[i] = z[i] = 0.f;

        for (int c0 = 0; c0 < N; c0 += T) {
            __syncthreads();  // the previous chunk's LDS is no longer read
            // q, k chunk: rows past the end are zero after the feature map (a zero key
            // adds nothing to the state or to the key sum)
            for (int x = tid; x < T * E / 4; x += THREADS) {
                const int t = x / (E / 4), c4 = x - t * (E / 4);
                f32x4_t qv = {0.f, 0.f, 0.f, 0.f}, kv = {0.f, 0.f, 0.f, 0.f};
                if (c0 + t < N) {
                    qv = *reinterpret_cast<const f32x4_t *>(Qh + (size_t)(c0 + t) * E + 4 * c4);
                    kv = *reinterpret_cast<const f32x4_t *>(Kh + (size_t)(c0 + t) * E + 4 * c4);
                    if (fm) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            qv[j] = phi(qv[j]);
                            kv[j] = phi(kv[j]);
                        }
                    }
                }
                *reinterpret_cast<f32x4_t *>(lds + QS + t * E + 4 * c4) = qv;
                *reinterpret_cast<f32x4_t *>(lds + KS + t * E + 4 * c4) = kv;
            }
            for (int x = tid; x < T * MS / 4; x += THREADS) {
                const int t = x / (MS / 4), c4 = x - t * (MS / 4);
                f32x4_t vv = {0.f, 0.f, 0.f, 0.f};
                if (c0 + t < N) vv = *reinterpret_cast<const f32x4_t *>(Vh + (size_t)(c0 + t) * M + 4 * c4);
                *reinterpret_cast<f32x4_t *>(lds + VS + t * MS + 4 * c4) = vv;
            }
            __syncthreads();
            // scan the chunk: state and key sum include token t before its readout
#pragma unroll 4
            for (int t = 0; t < T; ++t) {
                const float vt = lds[VS + t * MS + m];
                float pn = 0.f, pd = 0.f;
#pragma unroll
                for (int i = 0; i < EPT; ++i) {
                    const float kk = lds[KS + t * E + g * EPT + i];
                    const float qq = lds[QS + t * E + g * EPT + i];
                    S[i] = fmaf(kk, vt, S[i]);
                    z[i] += kk;
                    pn = fmaf(qq, S[i], pn);
                    pd = fmaf(qq, z[i], pd);
                }
                lds[RN + (t * EG + g) * MS + m] = pn;
                if (m == 0) lds[RD + t * EG + g] = pd;
            }
            __syncthreads();
            // outputs: thread (row r, column m) sums the 16 partials of its rows
#pragma unroll
            for (int t = tid / MS; t < T; t += THREADS / MS) {
                if (c0 + t >= N) break;
                float num = 0.f, den = 0.f;
#pragma unroll
                for (int e = 0; e < EG; ++e) {
                    num += lds[RN + (t * EG + e) * MS + m];
                    den += lds[RD + t * EG + e];
                }
                Oh[(size_t)(c0 + t) * M + m] = fm ? num / (den + a.eps) : num;
            }
        }
    }
};

template <int E>
__global__ __launch_bounds__(256) void attn_linear_fwd_kernel(LinArgs a) {
    LinFwd<E>::run(a);
}

}  // namespace attn
