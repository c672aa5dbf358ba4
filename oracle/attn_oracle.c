/*
 * Reference attention forward and backward in fp64 — TEST INFRASTRUCTURE ONLY.
 *
 * This file is the oracle that the GPU path is checked against.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no source, header, helper or constant with the HIP
 * library, and nothing in the product path may call it.
 *
 * What it computes is the plain definition of scaled-dot-product attention,
 * written out literally, with no tiling, no online softmax and no reordering:
 *
 *   "Understand FlashAttention" (nothiny.github.io), section "Attention 前向和
 *   反向传播公式 / 前向传播": S = Q K^T, P = softmax(S), O = P V, with
 *   Q, K, V in R^{N x d}.
 *
 *   "PyTorch profiling part 3: attention" (Hugging Face blog, Chinese
 *   translation), section "朴素注意力" (naive attention), its five steps:
 *   scores = q k^T; scores *= scale; masked entries set to -inf;
 *   softmax over the key axis; out = attn v.  The causal mask is the
 *   lower triangle (section "构建因果掩码": ones -> tril), so key j is
 *   allowed for query i iff j <= i.
 *
 *   "Understand FlashAttention", section "数值稳定的 Softmax": softmax is
 *   evaluated as e^{x_i - m} / sum_j e^{x_j - m} with m the row max, and the
 *   section "附：数值稳定的logsumexp(L)推导" defines the per-row
 *   log-sum-exp L_i = m_i + log(sum_j e^{S_ij - m_i}) (natural log).
 *
 * Readings taken where the pages are silent:
 *   - the scale multiplies the raw dot product before masking (naive
 *     attention, steps 1-3);
 *   - a row with every key masked (plain softmax would give 0/0) yields
 *     o = 0 and lse = -inf, the "safe softmax" reading of that page's section
 *     "安全 softmax".  The plain forward (equal query and key lengths,
 *     diagonal kept) never produces such a row; the masked one below can.
 *
 * The backward (oracle_attn_bwd_f64, below) follows the same page's section
 * "反向传播" and recomputes each softmax row from the definition.
 *
 * Every row materialises its whole score row s[0..N) in fp64; inputs are the
 * exact values the GPU sees, widened to double by the caller.  Summation is a
 * plain left-to-right loop, so results are deterministic.  Rows are
 * independent and are spread over OpenMP threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One query row of one head.
 *   q_i  : [d]      the query row
 *   k, v : [N, d]   keys and values of the head, row-major
 *   s    : [N]      scratch for the score row (written)
 *   o_i  : [d]      output row (written)
 *   lse_i: scalar   log-sum-exp of the scaled, masked score row (written)
 */
static void attention_row(const double *q_i, const double *k, const double *v,
                          int64_t N, int64_t d, double scale, int causal,
                          int64_t i, double *s, double *o_i, double *lse_i)
{
    /* naive attention steps 1-2: scores = (q . k_j) * scale */
    for (int64_t j = 0; j < N; ++j) {
        const double *k_j = k + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += q_i[c] * k_j[c];
        s[j] = dot * scale;
    }
    /* step 3: causal mask (lower triangle, diagonal kept) */
    if (causal)
        for (int64_t j = i + 1; j < N; ++j)
            s[j] = -INFINITY;

    /* step 4: numerically stable softmax, m = row max, l = sum e^{s-m} */
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j)
        if (s[j] > m)
            m = s[j];

    for (int64_t c = 0; c < d; ++c)
        o_i[c] = 0.0;
    if (m == -INFINITY) { /* every key masked: safe-softmax reading */
        *lse_i = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        s[j] = exp(s[j] - m); /* s now holds the unnormalised weights */
        l += s[j];
    }
    /* step 5: out = P v with P_ij = e^{s_ij - m} / l */
    for (int64_t j = 0; j < N; ++j) {
        const double p = s[j] / l;
        const double *v_j = v + j * d;
        for (int64_t c = 0; c < d; ++c)
            o_i[c] += p * v_j[c];
    }
    *lse_i = m + log(l);
}

/* Returns 0 on success, 1 on an invalid argument, 2 when scratch memory
 * cannot be allocated. */
static int check_args(const void *q, const void *k, const void *v,
                      const void *o, const void *lse, int64_t N, int64_t d,
                      int causal)
{
    if (!q || !k || !v || !o || !lse) return 1;
    if (N < 1 || d < 1) return 1;
    if (causal != 0 && causal != 1) return 1;
    return 0;
}

/* Full forward for all heads.
 *   q, k, v : [B, H, N, d] row-major fp64
 *   o       : [B, H, N, d] (written)
 *   lse     : [B, H, N]    (written)
 */
int oracle_attn_fwd_f64(const double *q, const double *k, const double *v,
                        double *o, double *lse, int64_t B, int64_t H,
                        int64_t N, int64_t d, double scale, int causal)
{
    int rc = check_args(q, k, v, o, lse, N, d, causal);
    if (rc) return rc;
    if (B < 1 || H < 1) return 1;
    const int64_t rows = B * H * N;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            if (!s) continue;
            const int64_t head = r / N, i = r % N;
            const int64_t base = head * N * d;
            attention_row(q + base + i * d, k + base, v + base, N, d, scale,
                          causal, i, s, o + r * d, lse + r);
        }
        free(s);
    }
    return failed ? 2 : 0;
}

/* Selected query rows of ONE head (used to check large problems row by row).
 *   q, k, v : [N, d] of the head
 *   rows    : [nrows] query indices in [0, N)
 *   o       : [nrows, d] (written);  lse : [nrows] (written)
 */
int oracle_attn_rows_f64(const double *q, const double *k, const double *v,
                         int64_t N, int64_t d, double scale, int causal,
                         const int64_t *rows, int64_t nrows, double *o,
                         double *lse)
{
    int rc = check_args(q, k, v, o, lse, N, d, causal);
    if (rc) return rc;
    if (!rows || nrows < 0) return 1;
    for (int64_t t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= N) return 1;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!s) continue;
            const int64_t i = rows[t];
            attention_row(q + i * d, k, v, N, d, scale, causal, i, s,
                          o + t * d, lse + t);
        }
        free(s);
    }
    return failed ? 2 : 0;
}

/* Dense intermediates of ONE head, for small N:
 *   S : [N, N] scaled scores with masked entries set to -inf (written)
 *   P : [N, N] softmax rows (written)
 */
int oracle_attn_dense_f64(const double *q, const double *k, int64_t N,
                          int64_t d, double scale, int causal, double *S,
                          double *P)
{
    if (!q || !k || !S || !P || N < 1 || d < 1) return 1;
    if (causal != 0 && causal != 1) return 1;
    for (int64_t i = 0; i < N; ++i) {
        double *s = S + i * N, *p = P + i * N;
        for (int64_t j = 0; j < N; ++j) {
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c)
                dot += q[i * d + c] * k[j * d + c];
            s[j] = dot * scale;
            if (causal && j > i) s[j] = -INFINITY;
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j)
            if (s[j] > m) m = s[j];
        if (m == -INFINITY) {
            for (int64_t j = 0; j < N; ++j) p[j] = 0.0;
            continue;
        }
        double l = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            p[j] = exp(s[j] - m);
            l += p[j];
        }
        for (int64_t j = 0; j < N; ++j) p[j] /= l;
    }
    return 0;
}

/* Backward of the same attention, all heads (gradients of a scalar loss L
 * whose gradient with respect to O is dout):
 *
 *   "Understand FlashAttention", section "Attention 前向和反向传播公式 /
 *   反向传播": dV = P^T dO, dP = dO V^T, dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
 *   dQ = dS K, dK = dS^T Q.  Here S = scale * Q K^T, so the chain rule puts
 *   the scale on dQ and dK: dQ = scale * dS K, dK = scale * dS^T Q.  Masked
 *   entries have P_ij = 0 and so contribute nothing.
 *
 * Each query row i is taken in turn: its softmax row P_i (recomputed from the
 * definition, as in the forward), dP_i, the row term D_i = sum_j P_ij dP_ij,
 * dS_i, then dQ_i, and its contributions to every dK_j and dV_j.  Heads are
 * independent and are spread over OpenMP threads; inside a head the rows
 * accumulate into dK and dV in order, so results are deterministic.
 *   q, k, v, dout : [B, H, N, d] row-major fp64
 *   dq, dk, dv    : [B, H, N, d] (written)
 */
int oracle_attn_bwd_f64(const double *q, const double *k, const double *v,
                        const double *dout, double *dq, double *dk, double *dv,
                        int64_t B, int64_t H, int64_t N, int64_t d,
                        double scale, int causal)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
    if (B < 1 || H < 1 || N < 1 || d < 1) return 1;
    if (causal != 0 && causal != 1) return 1;
    const int64_t heads = B * H;
    int failed = 0;
#pragma omp parallel
    {
        double *P = (double *)malloc((size_t)N * sizeof(double));
        double *dP = (double *)malloc((size_t)N * sizeof(double));
        if (!P || !dP) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t hd = 0; hd < heads; ++hd) {
            if (!P || !dP) continue;
            const int64_t base = hd * N * d;
            const double *qh = q + base, *kh = k + base, *vh = v + base, *doh = dout + base;
            double *dqh = dq + base, *dkh = dk + base, *dvh = dv + base;
            for (int64_t t = 0; t < N * d; ++t) {
                dkh[t] = 0.0;
                dvh[t] = 0.0;
            }
            for (int64_t i = 0; i < N; ++i) {
                const double *q_i = qh + i * d, *do_i = doh + i * d;
                const int64_t nvis = causal ? i + 1 : N;  /* keys 0 .. nvis-1 are visible */
                /* the softmax row, as in the forward */
                double m = -INFINITY;
                for (int64_t j = 0; j < nvis; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c) dot += q_i[c] * kh[j * d + c];
                    P[j] = dot * scale;
                    if (P[j] > m) m = P[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < nvis; ++j) {
                    P[j] = exp(P[j] - m);
                    l += P[j];
                }
                for (int64_t j = 0; j < nvis; ++j) P[j] /= l;
                /* dP_ij = dO_i . v_j and D_i = sum_j P_ij dP_ij */
                double D = 0.0;
                for (int64_t j = 0; j < nvis; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c) dot += do_i[c] * vh[j * d + c];
                    dP[j] = dot;
                    D += P[j] * dot;
                }
                /* dS_ij = P_ij (dP_ij - D_i); dQ_i = scale sum_j dS_ij k_j;
                 * dK_j += scale dS_ij q_i; dV_j += P_ij dO_i */
                double *dq_i = dqh + i * d;
                for (int64_t c = 0; c < d; ++c) dq_i[c] = 0.0;
                for (int64_t j = 0; j < nvis; ++j) {
                    const double ds = P[j] * (dP[j] - D);
                    for (int64_t c = 0; c < d; ++c) {
                        dq_i[c] += scale * ds * kh[j * d + c];
                        dkh[j * d + c] += scale * ds * q_i[c];
                        dvh[j * d + c] += P[j] * do_i[c];
                    }
                }
            }
        }
        free(P);
        free(dP);
    }
    return failed ? 2 : 0;
}

/* Attention with a general mask and unequal query and key lengths, all heads.
 *
 *   q       : [B, H, Nq, d];  k, v : [B, H, Nk, d]   row-major fp64
 *   o       : [B, H, Nq, d] (written);  lse : [B, H, Nq] (written)
 *   bias    : NULL (no mask) or an additive mask; element (b, h, i, j) sits at
 *             bias[b * sb + h * sh + i * Nk + j] (sb = 0 or sh = 0 broadcasts
 *             one mask over batches or heads).  -inf hides key j from query i;
 *             finite values are added to the scaled score.
 *   causal  : key j is visible to query i iff j <= i + (Nk - Nq): the lower
 *             triangle anchored at the bottom-right corner, so the Nq queries
 *             are the last Nq positions of the key sequence.
 *
 * "PyTorch profiling part 3: attention", section "朴素注意力": scores = q k^T,
 * times the scale, masked entries -inf, softmax over keys, times v; section
 * "构建因果掩码": a mask is applied as an additive bias of 0 or -inf after the
 * scaling; section "安全 softmax": a row whose every entry is -inf would give
 * 0/0, and the safe softmax returns zeros there, so such a row gets o = 0 and
 * lse = -inf.  The log-sum-exp is that of the scaled, biased, masked row
 * ("Understand FlashAttention", appendix "附：数值稳定的logsumexp(L)推导").
 */
int oracle_attn_masked_f64(const double *q, const double *k, const double *v,
                           const double *bias, int64_t sb, int64_t sh,
                           double *o, double *lse, int64_t B, int64_t H,
                           int64_t Nq, int64_t Nk, int64_t d, double scale,
                           int causal)
{
    if (!q || !k || !v || !o || !lse) return 1;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return 1;
    if (causal != 0 && causal != 1) return 1;
    const int64_t rows = B * H * Nq;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Nk * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            if (!s) continue;
            const int64_t head = r / Nq, i = r % Nq;
            const int64_t b = head / H, h = head % H;
            const double *q_i = q + r * d;
            const double *kh = k + head * Nk * d, *vh = v + head * Nk * d;
            const double *bias_i = bias ? bias + b * sb + h * sh + i * Nk : NULL;
            double *o_i = o + r * d;
            /* steps 1-3: scaled scores, plus the additive mask, causal entries -inf */
            for (int64_t j = 0; j < Nk; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += q_i[c] * kh[j * d + c];
                s[j] = dot * scale;
                if (bias_i)
                    s[j] += bias_i[j];
                if (causal && j > i + (Nk - Nq))
                    s[j] = -INFINITY;
            }
            /* step 4: stable softmax; a row with no visible key is all zeros */
            double m = -INFINITY;
            for (int64_t j = 0; j < Nk; ++j)
                if (s[j] > m)
                    m = s[j];
            for (int64_t c = 0; c < d; ++c)
                o_i[c] = 0.0;
            if (m == -INFINITY) {
                lse[r] = -INFINITY;
                continue;
            }
            double l = 0.0;
            for (int64_t j = 0; j < Nk; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            /* step 5: out = P v */
            for (int64_t j = 0; j < Nk; ++j) {
                const double w = s[j] / l;
                for (int64_t c = 0; c < d; ++c)
                    o_i[c] += w * vh[j * d + c];
            }
            lse[r] = m + log(l);
        }
        free(s);
    }
    return failed ? 2 : 0;
}

/* Number of OpenMP threads a parallel region of this library will use. */
/*
 * Causal linear attention (another method, from the hqwc.cn notes on the
 * fast-transformers linear attention CUDA kernels, "Transformers are RNNs"):
 *
 *   section 0x0: the softmax similarity exp(q.k / sqrt(D)) is replaced by a
 *   kernel sim(q, k) = phi(q) . phi(k) with phi(x) = elu(x) + 1;
 *   section 0x1: the CausalLinearAttention module applies phi to the queries
 *   and keys, computes the normaliser Z_j = 1 / (phi(q_j) . sum_{t<=j}
 *   phi(k_t) + eps) and returns causal_dot_product(phi(Q), phi(K), V) * Z;
 *   section 0x2: causal_dot_product computes V'_j = sum_{t<=j} (q_j . k_t) v_t.
 *
 * feature_map = 0 computes the causal dot product alone (q, k used as given,
 * no normaliser); feature_map = 1 the whole module.  Written as the definition:
 * for each query row j a plain sum over the keys t <= j (O(N^2) per head), not
 * the running-state recurrence of the page's CPU and CUDA code.
 *   q, k : [BH, N, E]; v : [BH, N, M]; out : [BH, N, M] (written).
 */
static double elu_plus_one(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

int oracle_linattn_f64(const double *q, const double *k, const double *v,
                       double *out, int64_t BH, int64_t N, int64_t E, int64_t M,
                       int feature_map, double eps)
{
    if (!q || !k || !v || !out || BH < 1 || N < 1 || E < 1 || M < 1) return 1;
    if (feature_map != 0 && feature_map != 1) return 1;
    const int64_t nq = BH * N * E;
    double *fq = malloc(sizeof(double) * (size_t)nq);
    double *fk = malloc(sizeof(double) * (size_t)nq);
    if (!fq || !fk) { free(fq); free(fk); return 2; }
    for (int64_t x = 0; x < nq; ++x) {   /* the feature map, elementwise */
        fq[x] = feature_map ? elu_plus_one(q[x]) : q[x];
        fk[x] = feature_map ? elu_plus_one(k[x]) : k[x];
    }
    int failed = 0;
#pragma omp parallel
    {
        double *num = malloc(sizeof(double) * (size_t)M);
        double *ksum = malloc(sizeof(double) * (size_t)E);
        if (!num || !ksum) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < BH * N; ++r) {
            if (!num || !ksum) continue;
            const int64_t h = r / N, j = r % N;
            const double *qj = fq + r * E;
            for (int64_t m = 0; m < M; ++m) num[m] = 0.0;
            for (int64_t e = 0; e < E; ++e) ksum[e] = 0.0;
            for (int64_t t = 0; t <= j; ++t) {   /* causal: keys t <= j */
                const double *kt = fk + (h * N + t) * E;
                const double *vt = v + (h * N + t) * M;
                double sim = 0.0;
                for (int64_t e = 0; e < E; ++e) sim += qj[e] * kt[e];
                for (int64_t m = 0; m < M; ++m) num[m] += sim * vt[m];
                for (int64_t e = 0; e < E; ++e) ksum[e] += kt[e];
            }
            double *oj = out + r * M;
            if (feature_map) {
                double den = 0.0;   /* phi(q_j) . sum_{t<=j} phi(k_t) */
                for (int64_t e = 0; e < E; ++e) den += qj[e] * ksum[e];
                const double z = 1.0 / (den + eps);
                for (int64_t m = 0; m < M; ++m) oj[m] = num[m] * z;
            } else {
                for (int64_t m = 0; m < M; ++m) oj[m] = num[m];
            }
        }
        free(num);
        free(ksum);
    }
    free(fq);
    free(fk);
    return failed ? 2 : 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
