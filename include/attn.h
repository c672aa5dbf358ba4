/*
 * attn.h — C ABI of the exact attention library for MI355X (gfx950):
 * forward (attn_fwd), backward (attn_bwd, and attn_bwd_noalloc for callers that
 * cannot allocate), forward with unequal query/key lengths and boolean masks
 * (attn_fwd_masked, attn_mask_pack), and causal linear attention
 * (attn_linear_fwd, attn_linear_workspace_bytes).
 *
 * The operation is exact scaled-dot-product attention, one (batch, head) at a
 * time:
 *
 *   S = scale * Q K^T,   S_ij = -inf where causal and key j > query i,
 *   P = softmax(S) over the key axis,   O = P V,
 *   lse_i = log sum_j e^{S_ij} = m_i + log l_i   (natural log)
 *
 * as defined in "Understand FlashAttention" (nothiny.github.io), section
 * "Attention 前向和反向传播公式 / 前向传播" (S = Q K^T, P = softmax(S), O = P V)
 * and its appendix "附：数值稳定的logsumexp(L)推导" (L = m + log l), with the
 * scale and the lower-triangle causal mask of "PyTorch profiling part 3:
 * attention" (Hugging Face blog), sections "朴素注意力" and "构建因果掩码".
 * It is computed FlashAttention-style ("Understand FlashAttention", section
 * "FlashAttention": Q split into row blocks in the outer loop, K/V into column
 * blocks in the inner loop; section "两块情况的完整推导": running row max m and
 * normaliser l, the partial output rescaled by e^{m_old - m_new}), so the
 * N x N score matrix never reaches device memory.
 *
 * All entry points are extern "C" and take plain pointers and sizes.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of this header are the library's only exported names. */
#define ATTN_API __attribute__((visibility("default")))

/* Element type of q, k, v and o.  lse is always fp32. */
typedef enum {
    ATTN_F32 = 0,  /* IEEE binary32 */
    ATTN_F16 = 1,  /* IEEE binary16 */
    ATTN_BF16 = 2  /* bfloat16 */
} attn_dtype_t;

/* Return codes. */
typedef enum {
    ATTN_OK = 0,
    ATTN_EINVAL = 1,       /* invalid argument; nothing was launched */
    ATTN_EUNSUPPORTED = 2, /* valid but unsupported (head dim, size); nothing launched */
    ATTN_EHIP = 3,         /* the HIP runtime reported an error at launch */
    ATTN_ESCRATCH = 4      /* attn_bwd_noalloc: B*H*N above its fixed scratch; nothing launched */
} attn_status_t;

/* Version of this ABI; bumped when entry points change or are added. */
#define ATTN_ABI_VERSION 5

/*
 * attn_fwd — attention forward for B*H independent heads.
 *
 * Arguments
 *   q, k, v  device pointers, each [B, H, N, d] contiguous, d innermost, of
 *            element type `dtype`; read only.
 *   o        device pointer, [B, H, N, d] contiguous of `dtype`; written.
 *            o[b,h,i,:] = sum_j P_ij v[b,h,j,:], rounded to `dtype` (nearest even).
 *   lse      device pointer, [B, H, N] contiguous fp32; written.
 *            lse[b,h,i] = m_i + ln l_i of the scaled, masked score row.
 *   B, H, N  batch, heads, sequence length (queries and keys alike), each >= 1.
 *   d        head dimension; 64 or 128.
 *   scale    finite multiplier of q.k (the usual value is 1/sqrt(d)).
 *   causal   0: every key is visible; 1: key j is visible to query i iff j <= i.
 *   dtype    an attn_dtype_t.
 *   stream   HIP stream the work is enqueued on (0 = the null stream).
 *
 * Arithmetic: bf16/fp16 inputs are multiplied on the matrix cores with fp32
 * accumulation; the softmax statistics and the output accumulator are fp32;
 * the probabilities fed to the second product are rounded to the input type.
 * fp32 inputs are processed entirely in fp32.  Results of one build on one
 * input are bitwise reproducible from call to call.
 *
 * Ownership and concurrency: all buffers belong to the caller.  The library
 * allocates no memory; its only mutable state is a per-device flag recording
 * that the matrix-core kernels were opted in to their LDS size (set once,
 * atomically), so calls on different streams or host threads may run
 * concurrently.  o and lse must not overlap q, k, v or each other.
 *
 * Errors are returned synchronously and nothing is launched on error:
 *   ATTN_EINVAL       a NULL pointer; B, H or N < 1; d < 1; unknown dtype;
 *                     causal not 0/1; non-finite scale; q, k, v or o not 16-byte
 *                     aligned or lse not 4-byte aligned; o or lse overlapping
 *                     q, k, v or each other.
 *   ATTN_EUNSUPPORTED d not 64 or 128; a problem whose tile count exceeds the
 *                     launch grid.
 *   ATTN_EHIP         the launch itself failed (status of hipLaunchKernel or of
 *                     the LDS opt-in, not an error left by an earlier call).
 * The call is asynchronous: results are valid once `stream` has completed.
 */
ATTN_API int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int H, int N, int d, float scale, int causal, int dtype,
                      hipStream_t stream);

/*
 * attn_fwd_masked — attention forward with unequal query and key lengths and
 * an optional boolean mask, for B*H independent heads.
 *
 * The mask follows "PyTorch profiling part 3: attention" (Hugging Face blog),
 * section "构建因果掩码": a boolean matrix whose false entries become -inf
 * scores after scaling (equivalently an additive 0 / -inf bias), combined with
 * the causal triangle; a query row whose every key is hidden gets o = 0 and
 * lse = -inf (the "safe softmax" reading of that page's section "安全 softmax",
 * where the plain softmax of such a row would be 0/0).  With Nq != Nk the
 * causal triangle is anchored at the bottom-right corner: the queries are the
 * last Nq of the Nk positions, so key j is visible to query i iff
 * j <= i + Nk - Nq (for Nq = Nk this is attn_fwd's mask).
 *
 * Arguments
 *   q        device pointer, [B, H, Nq, d] contiguous of `dtype`; read only.
 *   k, v     device pointers, [B, H, Nk, d] contiguous of `dtype`; read only.
 *   mask_bits  NULL (no mask) or a device pointer to 64-bit words, 8-byte
 *            aligned, as written by attn_mask_pack: mask head m is Nq rows of
 *            W = ceil(Nk / 64) words starting at word m * Nq * W; bit j % 64 of
 *            word j / 64 of row i is 1 iff key j is visible to query i.  Head
 *            (b, h) uses mask head m = b * mask_stride_b + h * mask_stride_h.
 *            Read only.
 *   mask_tiles NULL, or (with mask_bits) the tile summary attn_mask_pack wrote for
 *            the same mask heads: the bf16/fp16 kernels then skip, per 256-row
 *            query tile, the 64-key units no row of the tile can see (W <= 4096
 *            keeps the unit list on chip).  It must describe mask_bits exactly:
 *            a unit marked empty is never read.  fp32 ignores it.  Read only.
 *   mask_stride_b, mask_stride_h  mask-head strides, 0 .. 2^31 (0 shares one
 *            mask across that axis; [B, H] masks use H and 1); ignored without
 *            a mask.
 *   o        device pointer, [B, H, Nq, d] contiguous of `dtype`; written.
 *   lse      device pointer, [B, H, Nq] contiguous fp32; written.
 *   B, H, Nq, Nk  batch, heads, query and key lengths, each >= 1.
 *   d, scale, dtype, stream  as in attn_fwd.
 *   causal   0: only the mask hides keys; 1: also keys j > i + Nk - Nq.
 *
 * Arithmetic, reproducibility, ownership and concurrency: as attn_fwd.  o and
 * lse must not overlap q, k, v, the mask words read or each other.
 *
 * Errors are returned synchronously and nothing is launched on error:
 *   ATTN_EINVAL       as attn_fwd (with Nq, Nk in place of N); mask_tiles
 *                     without mask_bits; mask words not 8-byte aligned; a
 *                     negative stride; o or lse overlapping the mask words.
 *   ATTN_EUNSUPPORTED as attn_fwd; a mask head larger than 4 GiB; a stride
 *                     above 2^31; mask_tiles with W > 4096.
 *   ATTN_EHIP         as attn_fwd.
 */
ATTN_API int attn_fwd_masked(const void *q, const void *k, const void *v, const void *mask_bits,
                             const void *mask_tiles, long long mask_stride_b,
                             long long mask_stride_h, void *o, float *lse, int B, int H, int Nq,
                             int Nk, int d, float scale, int causal, int dtype,
                             hipStream_t stream);

/*
 * attn_mask_pack — packs a boolean mask into the bit format of attn_fwd_masked.
 *
 * Arguments
 *   mask     device pointer, [heads, Nq, Nk] contiguous bytes; nonzero = visible
 *            ("PyTorch profiling part 3: attention", section "构建因果掩码":
 *            true entries keep their score).  Read only.
 *   bits     device pointer, [heads, Nq, W] 64-bit words (W = ceil(Nk / 64)),
 *            8-byte aligned; written: bit j % 64 of word j / 64 of row r =
 *            (mask[.., r, j] != 0); bits past Nk are 0.
 *   tiles    NULL, or a device pointer to [heads, ceil(Nq / 256), ceil(W / 64)]
 *            64-bit words, 8-byte aligned; written: bit u % 64 of word u / 64 of
 *            (head, t) = 1 iff some row of rows 256 t .. 256 t + 255 has a
 *            visible key in keys 64 u .. 64 u + 63 (the tile summary of
 *            attn_fwd_masked).
 *   heads, Nq, Nk  >= 1.
 *   stream   HIP stream the work is enqueued on.
 *
 * The packed mask can be reused by any number of attn_fwd_masked calls.
 * Errors: ATTN_EINVAL (NULL mask or bits, a size < 1, bits or tiles misaligned,
 * outputs overlapping the mask or each other), ATTN_EUNSUPPORTED (more than
 * 2^40 words), ATTN_EHIP (launch failure).  Asynchronous like attn_fwd.
 */
ATTN_API int attn_mask_pack(const void *mask, void *bits, void *tiles, long long heads, int Nq,
                            int Nk, hipStream_t stream);

/*
 * attn_bwd — gradients of attention for B*H independent heads.
 *
 * Given dO = dLoss/dO for the forward above, computes dQ, dK, dV following
 * "Understand FlashAttention" (nothiny.github.io), section "反向传播":
 *
 *   dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij = dO_i . O_i,
 *   dS = P o (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,
 *
 * with P recomputed tile by tile from the forward's lse (same page, section
 * "为什么保存 logsumexp": P_ij = e^{S_ij - lse_i}), so nothing N x N reaches
 * device memory.
 *
 * Arguments
 *   q, k, v  as in attn_fwd; read only.
 *   o, lse   the forward's outputs for these q, k, v, scale and causal; read only.
 *   dout     device pointer, [B, H, N, d] contiguous of `dtype`; read only.
 *   dq, dk, dv  device pointers, [B, H, N, d] contiguous of `dtype`; written,
 *            rounded to `dtype` (nearest even).
 *   delta    device pointer, [B, H, N] contiguous fp32 workspace owned by the
 *            caller; written with D_i = dO_i . O_i (fp32).
 *   B, H, N, d, scale, causal, stream  as in attn_fwd.
 *   dtype    ATTN_BF16 or ATTN_F16 (ATTN_F32 is ATTN_EUNSUPPORTED).
 *
 * Arithmetic: products on the matrix cores with fp32 accumulation; P and dS
 * are rounded to the input type before the products that consume them.
 * Results of one build on one input are bitwise reproducible (no atomics).
 *
 * Ownership and concurrency: as attn_fwd.  dq, dk, dv and delta must not
 * overlap any input or each other.
 *
 * Errors are returned synchronously and nothing is launched on error:
 *   ATTN_EINVAL       a NULL pointer; B, H or N < 1; d < 1; unknown dtype;
 *                     causal not 0/1; non-finite scale; a [B, H, N, d] buffer
 *                     not 16-byte aligned or lse/delta not 4-byte aligned; an
 *                     output overlapping an input or another output.
 *   ATTN_EUNSUPPORTED dtype ATTN_F32; d not 64 or 128; a problem whose tile
 *                     count exceeds the launch grid.
 *   ATTN_EHIP         a launch failed (its own status).  Launches before the
 *                     failing one stay enqueued.
 * The call is asynchronous: results are valid once `stream` has completed.
 */
ATTN_API int attn_bwd(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dout, void *dq, void *dk, void *dv,
                      float *delta, int B, int H, int N, int d, float scale, int causal,
                      int dtype, hipStream_t stream);

/*
 * attn_bwd_noalloc — attn_bwd without the workspace argument, for callers that
 * cannot allocate device memory (code being captured into a HIP graph, serving
 * loops that must not call hipMalloc, harnesses that forbid it).
 *
 * Same operation, arguments (minus delta), arithmetic, results (bitwise those
 * of attn_bwd on the same inputs) and errors as attn_bwd.  The per-row term
 * D_i = dO_i . O_i lives in a scratch array that the library keeps in device
 * memory for the life of the process, one copy per GPU, of 2^22 fp32 rows
 * (16 MiB): B*H*N above 2^22 returns ATTN_ESCRATCH and launches nothing.  The
 * call allocates nothing; its first call on a device looks up that device's
 * copy (hipGetSymbolAddress) once.  Every row the call reads is written by the
 * same call first, so nothing needs clearing between calls.
 *
 * Concurrency: all calls on one GPU share its scratch, so calls that may overlap
 * in time on one GPU (different streams, or threads without ordering) race and
 * give wrong gradients; serialise them (one stream, or events).
 */
ATTN_API int attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                              const float *lse, const void *dout, void *dq, void *dk, void *dv,
                              int B, int H, int N, int d, float scale, int causal, int dtype,
                              hipStream_t stream);

/*
 * attn_linear_fwd — causal linear attention forward (fp32) for B*H independent
 * heads, a second attention method next to the softmax one above.
 *
 * From the hqwc.cn notes on the fast-transformers linear attention kernels
 * ("Transformers are RNNs"): the similarity exp(q.k / sqrt(D)) is replaced by
 * phi(q) . phi(k) with phi(x) = elu(x) + 1 (section 0x0); the causal module
 * returns causal_dot_product(phi(Q), phi(K), V) times
 * 1 / (phi(q_j) . sum_{t<=j} phi(k_t) + eps) (section 0x1); the causal dot
 * product is V'_j = sum_{t<=j} (q_j . k_t) v_t (section 0x2).
 *
 * Arguments
 *   q, k     device pointers, [B, H, N, E] contiguous fp32; read only.
 *   v        device pointer, [B, H, N, M] contiguous fp32; read only.
 *   o        device pointer, [B, H, N, M] contiguous fp32; written:
 *            feature_map = 0: o_j = sum_{t<=j} (q_j . k_t) v_t (the causal dot
 *            product of q and k as given); feature_map = 1: the same product of
 *            phi(q), phi(k) and v, divided by phi(q_j) . sum_{t<=j} phi(k_t) + eps.
 *   B, H, N  batch, heads, sequence length, each >= 1.
 *   E        query/key width: 16, 32, 64 or 128.
 *   M        value width: a multiple of 16.
 *   eps      finite, >= 0 (used with feature_map = 1; the page's default 1e-6).
 *   workspace  NULL, or device memory of at least attn_linear_workspace_bytes(B,
 *            H, N, E, M) bytes, 16-byte aligned, owned by the caller, overwritten
 *            (it must not overlap q, k, v or o).  It needs no initialisation, and
 *            calls that share one workspace must not overlap in time.  With it the
 *            sum over t <= j is split at blocks of tokens, in one of two forms:
 *            - E and M in {32, 64}: one launch; per span of 128 tokens, the
 *              in-span products and the span's state (phi(K)^T V, key sum), then
 *              the prefix of the earlier spans taken from the workspace in a fixed
 *              order (spans publish their states there with flags), then
 *              phi(Q) times the prefix (products on the bf16 matrix cores from
 *              three-part bf16 splits of the fp32 operands: fp32-level accuracy);
 *            - otherwise: chunks of 64 tokens in three launches: per chunk
 *              phi(K)^T V and the key sum into the workspace, an exclusive prefix
 *              over the chunks, then each chunk's outputs (for E >= 32 on the fp32
 *              matrix cores).
 *            Without a workspace one sequential scan per (head, 16 value columns)
 *            runs instead; so it does where a block form's limits are exceeded:
 *            for E >= 32, (N + 256) * max(E, M) * 4 and (E * M + E) * 4 below
 *            2^31 bytes; for E = 16, tiles within LDS.
 *   workspace_bytes  size of workspace in bytes (ignored when it is NULL).
 *   stream   HIP stream the work is enqueued on.
 *
 * Arithmetic: fp32 throughout; the scan carries the state in token order, the
 * block forms sum per block then over blocks (results of the forms differ by
 * rounding).  Results of one form are bitwise reproducible from call to call.
 * Ownership: as attn_fwd; o must not overlap q, k or v.
 * Errors (synchronous, nothing launched): ATTN_EINVAL (NULL pointer, a size < 1,
 * feature_map not 0/1, eps negative or not finite, a pointer not 16-byte aligned,
 * o overlapping an input, a workspace too small or overlapping a tensor),
 * ATTN_EUNSUPPORTED (E not 16/32/64/128, M not a multiple of 16, a grid or row
 * offset beyond 32 bits), ATTN_EHIP (launch).
 */
ATTN_API int attn_linear_fwd(const float *q, const float *k, const float *v, float *o, int B,
                             int H, int N, int E, int M, int feature_map, float eps,
                             void *workspace, long long workspace_bytes, hipStream_t stream);

/* Bytes of workspace attn_linear_fwd's block forms need for these sizes, or -1
 * for a size < 1: the larger of the chunked form's B * H * ceil(N / 64) *
 * (E * M + E) * 4 and, for E and M in {32, 64}, the one-pass form's layout (per
 * head, an 8-byte flag and an (E * M + E)-float state per span of 128 tokens,
 * and the same per group of 4 spans; four parts, each rounded up to 256 bytes). */
ATTN_API long long attn_linear_workspace_bytes(int B, int H, int N, int E, int M);

/* Static, NUL-terminated description of a status code (never NULL). */
ATTN_API const char *attn_strerror(int status);

/* Returns ATTN_ABI_VERSION of the built library. */
ATTN_API int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
