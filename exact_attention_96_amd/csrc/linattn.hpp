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

namespace attn {

// ---------------------------------------------------------------------------
// Chunked form of the same computation, for a caller's workspace.  The page's
// sum over t <= j splits at chunk boundaries (chunks of TC tokens):
//   o_j = phi(q_j) S_c + sum_{t in chunk c, t <= j} (phi(q_j) . phi(k_t)) v_t,
//   S_c = sum over earlier chunks of phi(K)^T V,
// and likewise the normaliser with z_c = sum over earlier chunks of phi(k_t).
// Three launches: (1) per chunk, its own phi(K_c)^T V_c and key sum into the
// workspace; (2) per head, an exclusive prefix of those over the chunks, in place;
// (3) per chunk, the outputs.  Every launch has B * H * (chunks) or more
// workgroups, instead of one sequential scan per (head, column slice).
// Workspace: [B * H][n_chunks][E * M + E] fp32 (state, then key sum).

struct LinChunkArgs {
    const float *q, *k, *v;
    float *o;
    float *ws;
    int N, M, n_chunks;
    float eps;
    int feature_map;
};

template <int E>
struct LinChunk {
    static constexpr int TC = 64;          // tokens per chunk
    static constexpr int TP = TC + 4;      // row stride of the transposed LDS tiles: a wave's
                                           // transposing writes spread over 16 banks instead of
                                           // one, and rows stay 16-byte aligned for the reads
    static constexpr int THREADS = 256;
    static __device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }

    // chunk rows [c0, c0 + TC) of a [N, W] tensor into LDS transposed, dst[w * TP + t]
    // (zeros past the end; the feature map if fm).  Each thread issues all its 16-byte
    // loads before the first use, so the chunk costs one memory latency, not one per load.
    template <int W>
    static __device__ __forceinline__ void load_t(float *dst, const float *src, int c0, int N, bool fm) {
        constexpr int PER = TC * W / 4 / THREADS;
        static_assert(PER >= 1 && PER * THREADS * 4 == TC * W, "whole 16-byte pieces per thread");
        f32x4_t val[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int x = threadIdx.x + j * THREADS, t = x / (W / 4), c4 = x - t * (W / 4);
            val[j] = c0 + t < N ? *reinterpret_cast<const f32x4_t *>(src + (size_t)(c0 + t) * W + 4 * c4)
                                : (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int x = threadIdx.x + j * THREADS, t = x / (W / 4), c4 = x - t * (W / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(4 * c4 + i) * TP + t] = fm && c0 + t < N ? phi(val[j][i]) : val[j][i];
        }
    }
    // the same for a width known only at run time (v in the state kernel), four loads at a time
    static __device__ __forceinline__ void load_t_rt(float *dst, const float *src, int c0, int N, int W) {
        const int n4 = TC * W / 4;
        for (int x0 = threadIdx.x; x0 < n4; x0 += 4 * THREADS) {
            f32x4_t val[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int x = x0 + j * THREADS, t = x / (W / 4), c4 = x - t * (W / 4);
                val[j] = x < n4 && c0 + t < N ? *reinterpret_cast<const f32x4_t *>(src + (size_t)(c0 + t) * W + 4 * c4)
                                              : (f32x4_t){0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int x = x0 + j * THREADS, t = x / (W / 4), c4 = x - t * (W / 4);
                if (x < n4)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[(4 * c4 + i) * TP + t] = val[j][i];
            }
        }
    }

    // (1) per (head, chunk): dS = phi(K_c)^T V_c [E][M] and dz = sum_t phi(k_t) [E]
    static __device__ void states(const LinChunkArgs &a) {
        extern __shared__ __attribute__((aligned(16))) float lds[];
        const int N = a.N, M = a.M;
        const int bh = blockIdx.x / a.n_chunks, c = blockIdx.x - bh * a.n_chunks, c0 = c * TC;
        float *Kt = lds;            // [E][TP]
        float *Vt = lds + E * TP;   // [M][TP]
        load_t<E>(Kt, a.k + (size_t)bh * N * E, c0, N, a.feature_map != 0);
        load_t_rt(Vt, a.v + (size_t)bh * N * M, c0, N, M);
        __syncthreads();
        float *W = a.ws + ((size_t)bh * a.n_chunks + c) * (size_t)(E * M + E);
        // 4 x 4 blocks of (e, m)
        const int nb = (E / 4) * (M / 4);
        for (int blk = threadIdx.x; blk < nb; blk += THREADS) {
            const int e0 = 4 * (blk / (M / 4)), m0 = 4 * (blk % (M / 4));
            float acc[4][4] = {};
#pragma unroll 2
            for (int t = 0; t < TC; t += 4) {
                f32x4_t kk[4], vv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kk[i] = *reinterpret_cast<const f32x4_t *>(Kt + (e0 + i) * TP + t);
                    vv[i] = *reinterpret_cast<const f32x4_t *>(Vt + (m0 + i) * TP + t);
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(kk[i][tt], vv[j][tt], acc[i][j]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4_t *>(W + (size_t)(e0 + i) * M + m0) =
                    (f32x4_t){acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        }
        for (int e = threadIdx.x; e < E; e += THREADS) {
            float zz = 0.f;
            for (int t = 0; t < TC; ++t) zz += Kt[e * TP + t];
            W[(size_t)E * M + e] = zz;
        }
    }

    // (3) per (head, chunk): outputs of the chunk's rows from the prefix S_c, z_c (workspace)
    static __device__ void outputs(const LinChunkArgs &a) {
        extern __shared__ __attribute__((aligned(16))) float lds[];
        const int N = a.N, M = a.M;
        const bool fm = a.feature_map != 0;
        const int bh = blockIdx.x / a.n_chunks, c = blockIdx.x - bh * a.n_chunks, c0 = c * TC;
        constexpr int KA = E * TP > TC * TC ? E * TP : TC * TC;  // K^T, later A^T
        float *Qt = lds;               // [E][TP]
        float *Kt = Qt + E * TP;       // [E][TP]
        float *Vr = Kt + KA;           // [TC][M] (row-major)
        float *Sc = Vr + TC * M;       // [E][M] + z [E]
        float *At = Kt;                // [TC (key t')][TC (query t)]: A^T, causal; written over
                                       // K^T (region of KA floats) once every block of A is in registers
        float *Dn = Sc + E * M + E;    // [TC] denominators
        load_t<E>(Qt, a.q + (size_t)bh * N * E, c0, N, fm);
        load_t<E>(Kt, a.k + (size_t)bh * N * E, c0, N, fm);
        {
            const float *src = a.v + (size_t)bh * N * M;
#pragma unroll 4
            for (int x = threadIdx.x; x < TC * M / 4; x += THREADS) {
                const int t = x / (M / 4), c4 = x - t * (M / 4);
                f32x4_t val = {0.f, 0.f, 0.f, 0.f};
                if (c0 + t < N) val = *reinterpret_cast<const f32x4_t *>(src + (size_t)(c0 + t) * M + 4 * c4);
                *reinterpret_cast<f32x4_t *>(Vr + t * M + 4 * c4) = val;
            }
            const float *W = a.ws + ((size_t)bh * a.n_chunks + c) * (size_t)(E * M + E);
#pragma unroll 4
            for (int x = threadIdx.x; x < (E * M + E) / 4; x += THREADS)
                *reinterpret_cast<f32x4_t *>(Sc + 4 * x) = *reinterpret_cast<const f32x4_t *>(W + 4 * x);
        }
        __syncthreads();
        // A^T[t'][t] = phi(q_t) . phi(k_t') for t' <= t, else 0: 4 x 4 blocks (t', t), each
        // thread's blocks in registers until every thread is done with K^T
        constexpr int NB = (TC / 4) * (TC / 4), BPT = (NB + THREADS - 1) / THREADS;
        float ablk[BPT][4][4];
#pragma unroll
        for (int r = 0; r < BPT; ++r) {
            const int blk = threadIdx.x + r * THREADS;
            const int p0 = 4 * (blk / (TC / 4)), t0 = 4 * (blk % (TC / 4));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) ablk[r][i][j] = 0.f;
            if (blk < NB && p0 <= t0 + 3) {
#pragma unroll 8
                for (int e = 0; e < E; ++e) {
                    const f32x4_t kk = *reinterpret_cast<const f32x4_t *>(Kt + e * TP + p0);
                    const f32x4_t qq = *reinterpret_cast<const f32x4_t *>(Qt + e * TP + t0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) ablk[r][i][j] = fmaf(kk[i], qq[j], ablk[r][i][j]);
                }
            }
        }
        __syncthreads();  // K^T is read by every thread above; A^T takes its place
#pragma unroll
        for (int r = 0; r < BPT; ++r) {
            const int blk = threadIdx.x + r * THREADS;
            if (blk >= NB) break;
            const int p0 = 4 * (blk / (TC / 4)), t0 = 4 * (blk % (TC / 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4_t row;
#pragma unroll
                for (int j = 0; j < 4; ++j) row[j] = p0 + i <= t0 + j ? ablk[r][i][j] : 0.f;
                *reinterpret_cast<f32x4_t *>(At + (p0 + i) * TC + t0) = row;
            }
        }
        __syncthreads();
        // denominators: phi(q_t) . z_c + sum_{t' <= t} A[t][t'], four rows per thread
        if (fm && threadIdx.x < TC / 4) {
            const int t0 = 4 * threadIdx.x;
            f32x4_t d = {0.f, 0.f, 0.f, 0.f};
            for (int e = 0; e < E; ++e) {
                const f32x4_t qq = *reinterpret_cast<const f32x4_t *>(Qt + e * TP + t0);
                const float zz = Sc[E * M + e];
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] = fmaf(qq[j], zz, d[j]);
            }
            for (int p = 0; p <= t0 + 3; ++p) {  // A^T is zero above each row's diagonal
                const f32x4_t aa = *reinterpret_cast<const f32x4_t *>(At + p * TC + t0);
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] += aa[j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) Dn[t0 + j] = d[j] + a.eps;
        }
        __syncthreads();
        // outputs: 4 x 4 blocks (t, m): phi(Q) S_c + A V
        float *Oh = a.o + (size_t)bh * N * M;
        for (int blk = threadIdx.x; blk < (TC / 4) * (M / 4); blk += THREADS) {
            const int t0 = 4 * (blk / (M / 4)), m0 = 4 * (blk % (M / 4));
            float acc[4][4] = {};
#pragma unroll 8
            for (int e = 0; e < E; ++e) {
                const f32x4_t qq = *reinterpret_cast<const f32x4_t *>(Qt + e * TP + t0);
                const f32x4_t ss = *reinterpret_cast<const f32x4_t *>(Sc + e * M + m0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(qq[i], ss[j], acc[i][j]);
            }
            // (several iterations' reads in flight: with one workgroup per CU nothing
            // else hides the LDS latency)
#pragma unroll 8
            for (int p = 0; p <= t0 + 3; ++p) {  // keys of the chunk up to the block's last row
                const f32x4_t aa = *reinterpret_cast<const f32x4_t *>(At + p * TC + t0);
                const f32x4_t vv = *reinterpret_cast<const f32x4_t *>(Vr + p * M + m0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(aa[i], vv[j], acc[i][j]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (c0 + t0 + i >= N) break;
                const float inv = fm ? 1.f / Dn[t0 + i] : 1.f;
                *reinterpret_cast<f32x4_t *>(Oh + (size_t)(c0 + t0 + i) * M + m0) =
                    (f32x4_t){acc[i][0] * inv, acc[i][1] * inv, acc[i][2] * inv, acc[i][3] * inv};
            }
        }
    }

    static constexpr int states_lds(int M) { return (E * TP + M * TP) * 4; }
    static constexpr int outputs_lds(int M) {
        return (E * TP + (E * TP > TC * TC ? E * TP : TC * TC) + TC * M + E * M + E + TC) * 4;
    }
};

template <int E>
__global__ __launch_bounds__(256) void attn_linear_states_kernel(LinChunkArgs a) {
    LinChunk<E>::states(a);
}

template <int E>
__global__ __launch_bounds__(256, 2) void attn_linear_outputs_kernel(LinChunkArgs a) {
    LinChunk<E>::outputs(a);
}

// The same chunk kernels on the fp32 matrix cores (E in {32, 64, 128}).
// v_mfma_f32_32x32x2_f32 adds a 32 x 32 product over 2 terms: lane l gives row l % 32 of
// the left operand and column l % 32 of the right one, each at term l / 32, and keeps 16
// entries of the result: column l % 32, rows 8 (r / 4) + 4 (l / 32) + r % 4 of register r.
// A sum over e (or over tokens) may visit its terms in any order, so each lane takes
// the half h = l / 32 of the terms in one contiguous run: its operands are 16-byte loads
// of one row, straight from global memory into registers.
//   states:  one wave per (head, chunk, 32 x 32 tile (e, m)) of dS = phi(K)^T V over the
//            chunk's 64 tokens, and z = sum of phi(k); operand columns staged in 4 KB of
//            the wave's own LDS.
//   outputs: wave w of a chunk owns query rows 32 (w & 1) ... + 31 and the value-column
//            blocks w >> 1, (w >> 1) + 2, ...  The chunk's three nonzero blocks of
//            A^T = phi(K) phi(Q)^T (the causal zero block is skipped, the diagonal one
//            masked) are formed once and shared through LDS.  In that layout a lane holds
//            one query row and 16 keys, which are exactly the left operand of A V for
//            those 16 keys, so A never returns to memory; the normaliser's row sums are
//            in-lane plus one exchange.
template <int E>
struct LinChunkMfma {
    static constexpr int TC = 64, THREADS = 256, HE = E / 2;
    static_assert(E % 32 == 0 && HE % 4 == 0, "E in {32, 64, 128}");
    static __device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }
    static __device__ __forceinline__ f32x16_t mma(float a, float b, const f32x16_t &c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // x[s] = (phi of) row[s], s < HE; zeros for a row past the sequence end
    static __device__ __forceinline__ void load_half(float (&x)[HE], const float *row, bool ok, bool fm) {
#pragma unroll
        for (int j = 0; j < HE / 4; ++j) {
            const f32x4_t v = ok ? *reinterpret_cast<const f32x4_t *>(row + 4 * j) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * j + i] = v[i];
        }
        if (fm && ok)
#pragma unroll
            for (int s = 0; s < HE; ++s) x[s] = phi(x[s]);
    }

    // One wave per (head, chunk, tile (e block, m block)) of dS over the chunk's tokens.
    // The wave loads rows [c0, c0 + 64) x 32 columns of phi(K) and of V with 16-byte
    // loads (eight rows per load; zeros past the sequence end or the row), 16 tokens at
    // a time, and stages each part in LDS (4 KB per wave, so LDS does not limit occupancy)
    // and reads the operand columns from there.  Token of term (h, s) within a part is
    // 2 s + h, so the two half-waves read adjacent LDS rows (distinct banks).
    static constexpr int STATE_TILES_PER_E = E / 32;
    // rows t0 + 8 j (j = 0, 1) of phi(K) and V (one 16-token part of the chunk per lane group)
    static __device__ __forceinline__ void load_part(f32x4_t (&kx)[2], f32x4_t (&vx)[2], const float *kh,
                                                     const float *vh, int t0, int N, int M, int e0, int m0,
                                                     bool fm, int q) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = t0 + 8 * j;
            const bool ok = t < N, okv = ok && m0 + 4 * q < M;
            kx[j] = ok ? *reinterpret_cast<const f32x4_t *>(kh + (size_t)t * E + e0 + 4 * q)
                       : (f32x4_t){0.f, 0.f, 0.f, 0.f};
            if (fm && ok)
#pragma unroll
                for (int i = 0; i < 4; ++i) kx[j][i] = phi(kx[j][i]);
            vx[j] = okv ? *reinterpret_cast<const f32x4_t *>(vh + (size_t)t * M + m0 + 4 * q)
                        : (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
    }
    static __device__ void states(const LinChunkArgs &a) {
        __shared__ __attribute__((aligned(16))) float lds[2 * 16 * 32];
        const int N = a.N, M = a.M;
        const bool fm = a.feature_map != 0;
        const int lane = threadIdx.x, col = lane & 31, h = lane >> 5, q = lane & 7, r0 = lane >> 3;
        const int nm = (M + 31) / 32, tiles = STATE_TILES_PER_E * nm;
        // each XCD takes a contiguous range of tiles, so the tiles of a chunk (which read
        // the same rows of phi(K) and V) share one L2
        const int lin = xcd_contiguous(blockIdx.x, gridDim.x);
        const int chunk = lin / tiles, tile = lin - chunk * tiles;
        const int bh = chunk / a.n_chunks, c = chunk - bh * a.n_chunks, c0 = c * TC;
        const int eb = tile / nm, mb = tile - eb * nm, e = 32 * eb + col, m = 32 * mb + col;
        float *W = a.ws + ((size_t)bh * a.n_chunks + c) * (size_t)(E * M + E);
        float *Ks = lds, *Vs = lds + 16 * 32;
        const float *kh = a.k + (size_t)bh * N * E, *vh = a.v + (size_t)bh * N * M;
        // two parts of 16 tokens in flight: part p + 2 is loaded once part p is in LDS
        f32x4_t kb[2][2], vb[2][2];
        load_part(kb[0], vb[0], kh, vh, c0 + r0, N, M, 32 * eb, 32 * mb, fm, q);
        load_part(kb[1], vb[1], kh, vh, c0 + 16 + r0, N, M, 32 * eb, 32 * mb, fm, q);
        f32x16_t acc = {};
        float zs = 0.f;
#pragma unroll
        for (int part = 0; part < 4; ++part) {
            const int b = part & 1;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                *reinterpret_cast<f32x4_t *>(Ks + (r0 + 8 * j) * 32 + 4 * q) = kb[b][j];
                *reinterpret_cast<f32x4_t *>(Vs + (r0 + 8 * j) * 32 + 4 * q) = vb[b][j];
            }
            if (part + 2 < 4)
                load_part(kb[b], vb[b], kh, vh, c0 + 16 * (part + 2) + r0, N, M, 32 * eb, 32 * mb, fm, q);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float kv = Ks[(2 * s + h) * 32 + col];
                acc = mma(kv, Vs[(2 * s + h) * 32 + col], acc);
                zs += kv;
            }
        }
        if (m < M)
#pragma unroll
            for (int r = 0; r < 16; ++r) W[(size_t)(32 * eb + 8 * (r >> 2) + 4 * h + (r & 3)) * M + m] = acc[r];
        if (mb == 0) {
            zs += __shfl_xor(zs, 32);
            if (h == 0) W[(size_t)E * M + e] = zs;
        }
    }

    // Raw buffer accesses (stride 0): the resource holds the base and the byte count, a
    // lane gives a 32-bit byte offset, and an offset at or past the count reads 0 and
    // drops a store.  Rows past the sequence end and value columns past M need no branch.
    typedef __amdgpu_buffer_rsrc_t rsrc_t;
    static constexpr uint32_t kOff = 0x80000000u;  // an offset past every resource used here
    static __device__ __forceinline__ rsrc_t rsrc(const float *p, uint32_t bytes) {
        // word 3: 32-bit data format, the setting for untyped (raw) buffer accesses on gfx9
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, (int)bytes, 0x00020000);
    }
    static __device__ __forceinline__ float bload(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, float x) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, (int)off, 0, 0);
    }

    static __device__ void outputs(const LinChunkArgs &a) {
        const int N = a.N, M = a.M;
        const bool fm = a.feature_map != 0;
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 31, h = lane >> 5;
        const int bh = blockIdx.x / a.n_chunks, c = blockIdx.x - bh * a.n_chunks, c0 = c * TC;
        const int tb = w & 1, t0 = c0 + 32 * tb;
        const float *qh = a.q + (size_t)bh * N * E, *kh = a.k + (size_t)bh * N * E;
        const float *W = a.ws + ((size_t)bh * a.n_chunks + c) * (size_t)(E * M + E);
        // the head's v and o, and the chunk's state (the host keeps each under 2^31 bytes)
        const rsrc_t vr = rsrc(a.v + (size_t)bh * N * M, (uint32_t)N * M * 4);
        const rsrc_t orr = rsrc(a.o + (size_t)bh * N * M, (uint32_t)N * M * 4);
        const rsrc_t sr = rsrc(W, (uint32_t)E * M * 4);
        float qf[HE];
        load_half(qf, qh + (size_t)(t0 + col) * E + h * HE, t0 + col < N, fm);
        // The chunk's three nonzero blocks of A^T (key block, query block) = (0, 0), (0, 1),
        // (1, 1) are formed once, by waves 0, 1 and 3, and exchanged through LDS; lane:
        // query col of the block, keys 8 (r / 4) + 4 h + r % 4.
        __shared__ f32x4_t ash[3][4][64];
        const int role = w == 0 ? 0 : w == 1 ? 1 : w == 3 ? 2 : -1;
        if (role >= 0) {
            const int kb = role == 2 ? 32 : 0;
            float kf[HE];
            load_half(kf, kh + (size_t)(c0 + kb + col) * E + h * HE, c0 + kb + col < N, fm);
            f32x16_t ab = {};
#pragma unroll
            for (int s = 0; s < HE; ++s) ab = mma(kf[s], qf[s], ab);
            if (role != 1)  // diagonal block: key p is visible to query col when p <= col
#pragma unroll
                for (int r = 0; r < 16; ++r) ab[r] = 8 * (r >> 2) + 4 * h + (r & 3) > col ? 0.f : ab[r];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                ash[role][g][lane] = (f32x4_t){ab[4 * g], ab[4 * g + 1], ab[4 * g + 2], ab[4 * g + 3]};
        }
        __syncthreads();
        f32x16_t a0 = {}, a1 = {};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4_t x = ash[tb][g][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) a0[4 * g + i] = x[i];
        }
        if (tb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4_t x = ash[2][g][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) a1[4 * g + i] = x[i];
            }
        // normaliser of query t0 + col: phi(q) . z + sum of its row of A, plus eps
        float inv = 1.f;
        if (fm) {
            float d = 0.f;
            const float *z = W + (size_t)E * M + h * HE;
#pragma unroll
            for (int j = 0; j < HE / 4; ++j) {
                const f32x4_t zz = *reinterpret_cast<const f32x4_t *>(z + 4 * j);
#pragma unroll
                for (int i = 0; i < 4; ++i) d = fmaf(qf[4 * j + i], zz[i], d);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) d += a0[r] + a1[r];
            d += __shfl_xor(d, 32);
            inv = 1.f / (d + a.eps);
        }
        const uint32_t M4 = (uint32_t)M * 4;
        for (int mb = w >> 1; 32 * mb < M; mb += 2) {
            const int m = 32 * mb + col;
            const bool okm = m < M;
            f32x16_t acc = {};
            // phi(Q) S_c: term e = h E/2 + s
            const uint32_t so = okm ? (uint32_t)(h * HE) * M4 + 4u * m : kOff;
#pragma unroll
            for (int s = 0; s < HE; ++s) acc = mma(qf[s], bload(sr, so + s * M4), acc);
            // A V over the chunk's keys up to this row block: term s is key 8 (s / 4) + 4 h + s % 4
            const uint32_t vo = okm ? (uint32_t)(c0 + 4 * h) * M4 + 4u * m : kOff;
#pragma unroll
            for (int s = 0; s < 16; ++s) acc = mma(a0[s], bload(vr, vo + (8 * (s >> 2) + (s & 3)) * M4), acc);
            if (tb)
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    acc = mma(a1[s], bload(vr, vo + (32 + 8 * (s >> 2) + (s & 3)) * M4), acc);
            const uint32_t oo = okm ? (uint32_t)(t0 + 4 * h) * M4 + 4u * m : kOff;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + (r & 3);  // row t0 + 4 h + i
                bstore(orr, oo + i * M4, acc[r] * __shfl(inv, i + 4 * h));
            }
        }
    }
};

// seven waves per SIMD (4 KB of LDS per wave)
template <int E>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(7)))
void attn_linear_states_mfma_kernel(LinChunkArgs a) {
    LinChunkMfma<E>::states(a);
}

// up to E = 64 the output kernel fits four waves per SIMD without spilling
template <int E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(E <= 64 ? 4 : 1)))
void attn_linear_outputs_mfma_kernel(LinChunkArgs a) {
    LinChunkMfma<E>::outputs(a);
}

// (2) exclusive prefix over the chunks of each head, in place: thread x of the head
// owns workspace entry x of every chunk (state and key sum alike).
__global__ __launch_bounds__(256) void attn_linear_prefix_kernel(float *ws, int n_chunks, int per_chunk,
                                                                 int blocks_per_head) {
    const int bh = blockIdx.x / blocks_per_head;
    const int x = (blockIdx.x - bh * blocks_per_head) * 256 + threadIdx.x;
    if (x >= per_chunk) return;
    float *p = ws + (size_t)bh * n_chunks * per_chunk + x;
    float run = 0.f;
    int c = 0;
    for (; c + 4 <= n_chunks; c += 4) {  // four loads in flight
        float d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = p[(size_t)(c + i) * per_chunk];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[(size_t)(c + i) * per_chunk] = run;
            run += d[i];
        }
    }
    for (; c < n_chunks; ++c) {
        const float d = p[(size_t)c * per_chunk];
        p[(size_t)c * per_chunk] = run;
        run += d;
    }
}

}  // namespace attn
