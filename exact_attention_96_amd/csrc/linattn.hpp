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
// whole sequence.  Tokens go through LDS in chunks of T (the next chunk is loaded
// into registers while the current one is scanned): phi is applied on the way in,
// every thread advances its state token by token and writes its partial readouts
// q_t . S (and q_t . z) to LDS, and after the chunk each output is the sum of its 16
// partials.  The scan is sequential per workgroup; the grid holds
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
    static constexpr int T = 64;          // tokens per chunk
    static constexpr int MS = 16;         // value columns per workgroup
    static constexpr int EG = 16;         // e-groups
    static constexpr int EPT = E / EG;    // state rows per thread
    static constexpr int THREADS = EG * MS;
    static constexpr int G = E >= 128 ? 4 : 8;  // tokens per register group of the scan
    static constexpr int RP = EG + 4;     // padded stride of a (token, column) row of partials:
                                          // the 64 lanes of a write hit 64 different banks
    // LDS (floats): q and k chunks [T][E], v chunk [T][MS], partial numerators
    // [T][MS][RP], partial denominators [T][EG]
    static constexpr int QS = 0, KS = QS + T * E, VS = KS + T * E, RN = VS + T * MS, RD = RN + T * MS * RP;
    static constexpr int LDS_FLOATS = RD + T * EG;
    static constexpr int LDS_B = LDS_FLOATS * 4;
    // 16-byte pieces of a chunk per thread (q or k; v)
    static constexpr int QK4 = T * E / 4 / THREADS, V4 = T * MS / 4 / THREADS;
    static_assert(E % EG == 0 && QK4 * THREADS * 4 == T * E && V4 * THREADS * 4 == T * MS && T % G == 0,
                  "tile shape");
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

        // The next chunk is loaded into registers while the current one is scanned, so
        // no load latency lands between chunks.  Piece x of a tensor's chunk is row
        // x / (width / 4), 16-byte column x % (width / 4); rows past the end load zeros.
        f32x4_t rq[QK4], rk[QK4], rv[V4];
        auto fetch = [&](int c0) {
#pragma unroll
            for (int j = 0; j < QK4; ++j) {
                const int x = tid + j * THREADS, t = x / (E / 4), c4 = x - t * (E / 4);
                const bool ok = c0 + t < N;
                rq[j] = ok ? *reinterpret_cast<const f32x4_t *>(Qh + (size_t)(c0 + t) * E + 4 * c4)
                           : (f32x4_t){0.f, 0.f, 0.f, 0.f};
                rk[j] = ok ? *reinterpret_cast<const f32x4_t *>(Kh + (size_t)(c0 + t) * E + 4 * c4)
                           : (f32x4_t){0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < V4; ++j) {
                const int x = tid + j * THREADS, t = x / (MS / 4), c4 = x - t * (MS / 4);
                rv[j] = c0 + t < N ? *reinterpret_cast<const f32x4_t *>(Vh + (size_t)(c0 + t) * M + 4 * c4)
                                   : (f32x4_t){0.f, 0.f, 0.f, 0.f};
            }
        };
        // registers -> LDS, with the feature map; rows past the end stay zero (a zero key
        // adds nothing to the state or the key sum)
        auto stage = [&](int c0) {
#pragma unroll
            for (int j = 0; j < QK4; ++j) {
                const int x = tid + j * THREADS, t = x / (E / 4), c4 = x - t * (E / 4);
                f32x4_t qv = rq[j], kv = rk[j];
                if (fm && c0 + t < N) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qv[i] = phi(qv[i]);
                        kv[i] = phi(kv[i]);
                    }
                }
                *reinterpret_cast<f32x4_t *>(lds + QS + t * E + 4 * c4) = qv;
                *reinterpret_cast<f32x4_t *>(lds + KS + t * E + 4 * c4) = kv;
            }
#pragma unroll
            for (int j = 0; j < V4; ++j) {
                const int x = tid + j * THREADS, t = x / (MS / 4), c4 = x - t * (MS / 4);
                *reinterpret_cast<f32x4_t *>(lds + VS + t * MS + 4 * c4) = rv[j];
            }
        };

        fetch(0);
        for (int c0 = 0; c0 < N; c0 += T) {
            __syncthreads();  // the previous chunk's LDS is no longer read
            stage(c0);
            __syncthreads();
            if (c0 + T < N) fetch(c0 + T);
            // scan the chunk: state and key sum include token t before its readout.  Tokens
            // go in groups of G: all LDS reads of a group first, then the arithmetic, then
            // the partial stores (a store between reads would order every token's reads
            // after the previous token's store, one LDS round trip per token).
            for (int t0 = 0; t0 < T; t0 += G) {
                float kk[G][EPT], qq[G][EPT], vv[G], pn[G], pd[G];
#pragma unroll
                for (int tt = 0; tt < G; ++tt) {
                    vv[tt] = lds[VS + (t0 + tt) * MS + m];
#pragma unroll
                    for (int i = 0; i < EPT; ++i) {
                        kk[tt][i] = lds[KS + (t0 + tt) * E + g * EPT + i];
                        qq[tt][i] = lds[QS + (t0 + tt) * E + g * EPT + i];
                    }
                }
#pragma unroll
                for (int tt = 0; tt < G; ++tt) {
                    pn[tt] = 0.f;
                    pd[tt] = 0.f;
#pragma unroll
                    for (int i = 0; i < EPT; ++i) {
                        S[i] = fmaf(kk[tt][i], vv[tt], S[i]);
                        z[i] += kk[tt][i];
                        pn[tt] = fmaf(qq[tt][i], S[i], pn[tt]);
                        pd[tt] = fmaf(qq[tt][i], z[i], pd[tt]);
                    }
                }
#pragma unroll
                for (int tt = 0; tt < G; ++tt) {
                    lds[RN + ((t0 + tt) * MS + m) * RP + g] = pn[tt];
                    if (m == 0) lds[RD + (t0 + tt) * EG + g] = pd[tt];
                }
            }
            __syncthreads();
            // outputs: thread (row, column m) sums the 16 partials of its rows (16-byte reads)
#pragma unroll
            for (int t = tid / MS; t < T; t += THREADS / MS) {
                if (c0 + t >= N) break;
                float num = 0.f, den = 0.f;
#pragma unroll
                for (int e4 = 0; e4 < EG / 4; ++e4) {
                    const f32x4_t pn = *reinterpret_cast<const f32x4_t *>(lds + RN + (t * MS + m) * RP + 4 * e4);
                    const f32x4_t pd = *reinterpret_cast<const f32x4_t *>(lds + RD + t * EG + 4 * e4);
                    num += (pn[0] + pn[1]) + (pn[2] + pn[3]);
                    den += (pd[0] + pd[1]) + (pd[2] + pd[3]);
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
