// Causal linear attention in one pass over the sequence (fp32 data; products on the
// bf16 matrix cores from three-part splits, to fp32 accuracy).
//
// "hqwc.cn" notes on the fast-transformers linear attention kernels, sections
// 0x1-0x2: o_j = phi(q_j) S_j / (phi(q_j) . z_j + eps), S_j = sum_{t<=j} phi(k_t)
// v_t^T, z_j = sum_{t<=j} phi(k_t), with phi = elu + 1.  The page carries S along
// the sequence one token at a time; here the sum over t <= j is split at blocks of
// tokens, as in the chunked kernels of linattn.hpp, but all three steps of those
// kernels (block states, their prefix, the outputs) run in one launch.
//
// One workgroup (4 waves) per (head, span of L = 128 tokens); wave w owns the
// 32 tokens T0 = 128 j + 32 w ... of span j.
//   1. Each wave forms, from its own rows of phi(Q), phi(K), V, its block state
//      phi(K)^T V and key sum, written to its LDS region, and A^T = phi(K) phi(Q)^T on
//      its 32 x 32 diagonal block (masked to key <= query) with the row sums of A.
//   2. The span's aggregate (the four block states added in wave order) goes to the
//      workspace; while those stores complete, each wave forms the in-span part of its
//      outputs, A V.  Then a flag, and the workgroup takes the prefix of every earlier
//      span of the head, P_j, in a fixed order (below).
//   3. In LDS, each wave's region is replaced by its exclusive prefix P_j + the
//      states of the waves before it; each wave then adds phi(Q) (that prefix) to
//      its outputs, divides by the normaliser and stores o.
// Spans are grouped by G = 4.  The last span of each group also publishes its
// inclusive prefix.  Span j of group g0 = j - j % G sums, always in this order,
//   P_j = INCL_{g0 - 1} + AGG_{g0} + AGG_{g0 + 1} + ... + AGG_{j - 1},
// so the result does not depend on timing (the run is bitwise repeatable), a span
// reads at most G - 1 aggregates and one prefix, and the chain of inclusive prefixes
// has one link per group instead of one per span (G = 4 measured 7 % faster than 8 and
// 16 on the 2 x 32 x 8192 heads, and steadier than 2).
//
// Workgroup b runs (head b % BHp, span b / BHp) with BHp a multiple of 8: every
// span of a head is on the same XCD (workgroups go to the XCDs round robin), and
// a span only waits for spans with a smaller index, which were dispatched before it.
// A wait that has not ended after 2^18 polls (well under a second) gives up and marks
// the outputs NaN rather than hang.
//
// The exchange goes through device-coherent accesses, 16 bytes (4 consecutive
// entries) per thread and access: the aggregates and prefixes
// are stored with device-scope stores (write-through), the storing threads wait for
// their completion (vmcnt) before the workgroup barrier after which one thread
// writes the flag, and readers load the flag and then the data with device-scope
// loads.  A flag holds the call's epoch (a 64-bit value the host takes fresh for
// each call), so the workspace needs no clearing between calls.
//
// Products.  Each 16-term piece of a product runs as six v_mfma_f32_32x32x16_bf16 on
// three-part bf16 splits of its operands (x = h + m + l to within 2^-24 |x|; see
// split8): each product is then within a few units of 2^-24 of its value and the sums
// are fp32, so the results keep fp32-level accuracy at 2.7x the rate of
// v_mfma_f32_32x32x2_f32 (6 x 32 cycles against 8 x 64 for 16 terms).
//
// MFMA layouts (32 x 32 x 16: lane l gives row l % 32 of the left operand and column
// l % 32 of the right one, at terms 8 (l / 32) .. 8 (l / 32) + 7; it keeps column
// l % 32, rows 8 (r / 4) + 4 (l / 32) + r % 4 of register r).  Any sum may take its
// terms in any order, so term (i, h) of the 16-term piece kb may be index
// tok(8 kb + i) = 8 ((8 kb + i) / 4) + 4 h + i % 4: exactly the row that half h holds
// in register 8 kb + i of an accumulator.  Hence an accumulator is already an operand
// of the next product (A^T for A V), with no data movement; the pieces over the state
// width take, for half h, the e that the lane's rows of phi(Q) and phi(K) hold
// (32 eb + 16 kk + 8 (j / 4) + 4 h + j % 4 for element j of piece (eb, kk)).
#pragma once

#include "common.hpp"

namespace attn {

struct LinScanArgs {
    const float *q, *k, *v;
    float *o;
    unsigned long long *flag_agg, *flag_incl;  // [BH][S], [BH][SG]
    float *agg, *incl;                          // [BH][S][ENT], [BH][SG][ENT]
    unsigned long long epoch;                   // this call's flag value (nonzero)
    int N, BH, BHp, S, SG;                      // S spans per head, SG groups of G spans
    float eps;
    int feature_map;
};

template <int E, int M, int NW = 4>
struct LinScan {
    static constexpr int TS = 32, L = NW * TS, THREADS = NW * 64, G = 4;
    static constexpr int EB = E / 32, MB = M / 32;
    // A state sits in LDS by value column: row m holds the E entries (e, m), EP floats
    // apart, then the key sum.  A lane reads or writes 4 consecutive e of its column m
    // at once, and the 16 lanes of one 16-byte LDS access (columns c .. c + 15) start 4
    // banks apart.  The region also holds, before the state is written, the wave's phi(K)
    // block (TS rows of E + 8 floats).
    static constexpr int EP = E + 4;
    static constexpr int REG = M * EP + E > TS * (E + 8) ? M * EP + E : TS * (E + 8);
    static constexpr int ENT = E * M + E;   // entries of a state and key sum
    // a thread handles groups of 4 consecutive entries x4 = tid, tid + THREADS, ...
    static constexpr int CH = ENT / 4, PER = (CH + THREADS - 1) / THREADS;
    static constexpr int LDS_B = NW * REG * 4;
    static constexpr int NB = 17 / PER < 1 ? 1 : 17 / PER;  // aggregates loaded together (~68 registers)
    static constexpr uint32_t kOut = 0x80000000u;  // a buffer offset past every resource here
    static constexpr int kSpins = 1 << 18;
    static constexpr int kSc1 = 16;  // cache-policy bit of a buffer access: device scope
    static_assert((E == 32 || E == 64) && (M == 32 || M == 64), "E, M in {32, 64}");
    static_assert(8 / NW * LDS_B <= 160 * 1024, "LDS of the workgroups that fill a CU at two waves per SIMD");

    typedef __amdgpu_buffer_rsrc_t rsrc_t;
    static __device__ __forceinline__ rsrc_t rsrc(const float *p, uint32_t bytes) {
        // word 3: 32-bit data format, the setting for untyped (raw) buffer accesses on gfx9
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, (int)bytes, 0x00020000);
    }
    // raw buffer accesses: an offset at or past the resource's size reads 0 / drops the store
    static __device__ __forceinline__ float ld(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ f32x4_t ld4(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void st4(rsrc_t r, uint32_t off, f32x4_t x) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, (int)off, 0, 0);
    }
    // device-scope (sc1) 16-byte accesses: the stores write through, the loads are coherent
    static __device__ __forceinline__ f32x4_t ld4_dev(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSc1));
    }
    static __device__ __forceinline__ void st4_dev(rsrc_t r, uint32_t off, f32x4_t x) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, (int)off, 0, kSc1);
    }
    // phi(x) = elu(x) + 1: x + 1 for x > 0, else e^x as x log2(e) = th + tl (a two-part
    // constant; tl holds the rounding of x c_hi and the constant's tail), 2^th from
    // v_exp_f32, times (1 + tl ln 2): a few operations instead of the library expf's
    // range reduction.  Measured on gfx950 against fp64 exp over x in [-87, 0]: at most
    // 1.26 ulp (the library expf: 0.85 ulp); results below the normal range flush to 0.
    // Written as e^xn (1 + tl ln 2) + (x - xn) with xn = min(x, 0), with no branch (a
    // conditional exponential compiles to a branch per element): for x > 0 the
    // exponential of 0 is exactly 1 and x - xn = x, one rounding of x + 1; otherwise
    // x - xn is exactly 0.  A NaN x gives NaN.
    static __device__ __forceinline__ float phi(float x) {
        const float c_hi = 1.44269502162933349609375f;  // log2(e) rounded to float
        const float c_lo = 1.92596298909109e-8f;        // log2(e) - c_hi
        const bool pos = x > 0.f;
        const float xn = pos ? 0.f : x;
        const float th = xn * c_hi;
        const float tl = fmaf(xn, c_hi, -th) + xn * c_lo;
        const float e = __builtin_amdgcn_exp2f(th);
        return fmaf(e, tl * 0.69314718055994530942f, e + (x - xn));
    }
    // lane id (0..63) computed where it is used (volatile: not hoisted, not shared with
    // earlier uses)
    static __device__ __forceinline__ uint32_t lane_now() {
        uint32_t x;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
        return x;
    }
    // Three-part bf16 split of 8 floats, for products on the bf16 matrix cores that keep
    // fp32 accuracy: x = h + m + l + d with h = bf16(x), m = bf16(x - h), l = bf16(x - h - m)
    // (nearest even; each difference exact in fp32), so |m| <= 2^-8 |x|, |l| <= 2^-16 |x|
    // and |d| <= 2^-24 |x|.  The product x y then takes the six terms h h' + h m' + m h'
    // + m m' + h l' + l h'; the terms left out, m l', l m' and l l', are at most 2^-24,
    // 2^-24 and 2^-32 of |x y|.  Packed pairs: element 2 i in the low half of word i.
    struct Split8 {
        bf16x8_t h, m, l;
    };
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
        const f32x2_t v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    }
    static __device__ __forceinline__ float lo_f(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
    static __device__ __forceinline__ float hi_f(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
    static __device__ __forceinline__ Split8 split8(const float *x) {
        u32x4_t h, m, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = x[2 * i], b = x[2 * i + 1];
            h[i] = pk_bf16(a, b);
            const float ra = a - lo_f(h[i]), rb = b - hi_f(h[i]);
            m[i] = pk_bf16(ra, rb);
            l[i] = pk_bf16(ra - lo_f(m[i]), rb - hi_f(m[i]));
        }
        return {__builtin_bit_cast(bf16x8_t, h), __builtin_bit_cast(bf16x8_t, m), __builtin_bit_cast(bf16x8_t, l)};
    }
    static __device__ __forceinline__ f32x16_t mma16(bf16x8_t a, bf16x8_t b, const f32x16_t &c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // 16 terms of a product in fp32 accuracy from split operands (small terms first)
    static __device__ __forceinline__ f32x16_t mma_x3(const Split8 &a, const Split8 &b, f32x16_t c) {
        c = mma16(a.l, b.h, c);
        c = mma16(a.h, b.l, c);
        c = mma16(a.m, b.m, c);
        c = mma16(a.m, b.h, c);
        c = mma16(a.h, b.m, c);
        return mma16(a.h, b.h, c);
    }
    // LDS offset (floats, within a region) of piece x4 of a state and key sum, the order of
    // the exchange (a thread's 16-byte accesses) and of the workspace slots: piece
    // x4 = M p + m < E M / 4 holds entries e = 4 p .. 4 p + 3 of value column m, so that the
    // consecutive pieces of a wave's lanes sit in consecutive rows, four banks apart; then
    // the key sum
    static __device__ __forceinline__ int lds_of4(int x4) {
        return x4 < CH - E / 4 ? (x4 % M) * EP + 4 * (x4 / M) : M * EP + 4 * (x4 - (CH - E / 4));
    }
    static __device__ __forceinline__ f32x4_t &lds4(float *base, int o) { return *(f32x4_t *)(base + o); }
    static __device__ __forceinline__ rsrc_t rsrc_u64(const unsigned long long *p, int n) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned long long *>(p), (short)0, n * 8, 0x00020000);
    }
    // flag i of a resource, loaded device-coherently (sc1)
    static __device__ __forceinline__ unsigned long long ld_flag(rsrc_t r, int i) {
        return __builtin_bit_cast(unsigned long long, __builtin_amdgcn_raw_buffer_load_b64(r, i * 8, 0, kSc1));
    }
    // every thread's device-scope stores are complete, then one thread raises the flag
    static __device__ __forceinline__ void publish(unsigned long long *f, unsigned long long ep) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(f, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    static __device__ void run(const LinScanArgs &a) {
        extern __shared__ __attribute__((aligned(16))) float lds[];
        const int b = blockIdx.x, hh = b % a.BHp, j = b / a.BHp;
        if (hh >= a.BH) return;  // padding of BH up to a multiple of 8
        const int N = a.N;
        const bool fm = a.feature_map != 0;
        const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
        const int T0 = j * L + TS * w;
        // the head's tensors (the host keeps each below 2^31 bytes, one span past the end included)
        const rsrc_t rq = rsrc(a.q + (size_t)hh * N * E, (uint32_t)N * E * 4);
        const rsrc_t rk = rsrc(a.k + (size_t)hh * N * E, (uint32_t)N * E * 4);
        const rsrc_t rv = rsrc(a.v + (size_t)hh * N * M, (uint32_t)N * M * 4);
        const rsrc_t ro = rsrc(a.o + (size_t)hh * N * M, (uint32_t)N * M * 4);

        // ---- 1. this wave's block: loads (rows past N read 0)
        // qf, kf: row T0 + c, terms e = 32 eb + 8 i + 4 h + u  ->  [16 eb + 4 i + u]
        // vf: V[T0 + tok(r)][32 mb + c], kt: phi(K)[T0 + tok(r)][32 eb + c], tok(r) = 8 (r / 4) + 4 h + r % 4
        float qf[EB * 16], kf[EB * 16], kt[EB * 16], vf[MB * 16];
        {
            // in the order of use: K (for kt), V, then Q
            const uint32_t row = (uint32_t)(T0 + c) * (E * 4);
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4_t y = ld4(rk, row + (uint32_t)(32 * eb + 8 * i + 4 * h) * 4);
#pragma unroll
                    for (int u = 0; u < 4; ++u) kf[16 * eb + 4 * i + u] = y[u];
                }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t tok = (uint32_t)(T0 + 8 * (r >> 2) + 4 * h + (r & 3));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) vf[16 * mb + r] = ld(rv, (tok * M + 32 * mb + c) * 4);
            }
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4_t x = ld4(rq, row + (uint32_t)(32 * eb + 8 * i + 4 * h) * 4);
#pragma unroll
                    for (int u = 0; u < 4; ++u) qf[16 * eb + 4 * i + u] = x[u];
                }
        }
        // phi of K now (its loads were issued first); phi of Q just before A^T, so that the
        // K transposition and the state product need not wait for Q
        if (fm)
#pragma unroll
            for (int i = 0; i < EB * 16; ++i) kf[i] = phi(kf[i]);
        float *reg = lds + w * REG;
        {
            // kt is kf transposed, through this wave's LDS region (free until its state is
            // written): rows of KP floats, so that the two lane halves (rows 4 apart) read
            // the two halves of the banks
            constexpr int KP = E + 8;
            static_assert(TS * KP <= REG, "the phi(K) block fits in a wave's region");
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds4(reg, c * KP + 32 * eb + 8 * i + 4 * h) =
                        (f32x4_t){kf[16 * eb + 4 * i], kf[16 * eb + 4 * i + 1], kf[16 * eb + 4 * i + 2], kf[16 * eb + 4 * i + 3]};
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int eb = 0; eb < EB; ++eb) kt[16 * eb + r] = reg[(8 * (r >> 2) + 4 * h + (r & 3)) * KP + 32 * eb + c];
            if (T0 + TS > N)  // phi(0) = 1: keys past N are zeroed (a wave at the sequence end)
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int eb = 0; eb < EB; ++eb)
                        kt[16 * eb + r] = T0 + 8 * (r >> 2) + 4 * h + (r & 3) < N ? kt[16 * eb + r] : 0.f;
        }

        // block state phi(K)^T V and key sum into this wave's region
        // (16 terms per bf16 product: lane half h gives tokens tok(8 kb + i), i = 0 .. 7)
        Split8 vs[MB][2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) vs[mb][kb] = split8(&vf[16 * mb + 8 * kb]);
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
            const Split8 ks0 = split8(&kt[16 * eb]), ks1 = split8(&kt[16 * eb + 8]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                f32x16_t d = {};
                d = mma_x3(ks0, vs[mb][0], d);
                d = mma_x3(ks1, vs[mb][1], d);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    lds4(reg, (32 * mb + c) * EP + 32 * eb + 8 * g + 4 * h) =
                        (f32x4_t){d[4 * g], d[4 * g + 1], d[4 * g + 2], d[4 * g + 3]};
            }
            float zs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) zs += kt[16 * eb + r];
            zs += __shfl_xor(zs, 32);
            if (h == 0) reg[M * EP + 32 * eb + c] = zs;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (fm)
#pragma unroll
            for (int i = 0; i < EB * 16; ++i) qf[i] = phi(qf[i]);
        // A^T (keys x queries) of the diagonal block: lane = query T0 + c, register r = key tok(r)
        f32x16_t at = {};
#pragma unroll
        for (int i = 0; i < EB * 2; ++i) at = mma_x3(split8(&kf[8 * i]), split8(&qf[8 * i]), at);
        float rs = 0.f;  // row sum of A for query T0 + c (keys up to the query)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            at[r] = 8 * (r >> 2) + 4 * h + (r & 3) > c ? 0.f : at[r];
            rs += at[r];
        }
        rs += __shfl_xor(rs, 32);
        __builtin_amdgcn_sched_barrier(0);  // (the products above, before the wait for the other waves)
        __syncthreads();

        // ---- 2. the span's aggregate, then the prefix of the earlier spans
        const int jg = j % G, g0 = j - jg;
        const bool last = j == a.S - 1;
        // the head's aggregates and inclusive prefixes; an offset of kOut reads 0 and
        // drops a store (entry groups past ENT, slots that are not there)
        const rsrc_t rag = rsrc(a.agg + (size_t)hh * a.S * ENT, (uint32_t)a.S * ENT * 4);
        const rsrc_t rin = rsrc(a.incl + (size_t)hh * a.SG * ENT, (uint32_t)a.SG * ENT * 4);
        f32x4_t ag[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int x4 = tid + i * THREADS;
            ag[i] = (f32x4_t){};
            if (x4 < CH) {
                const int o = lds_of4(x4);
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) ag[i] += lds4(lds, ww * REG + o);
            }
        }
        // stored when the later spans of the group read it (else dropped: issuing the stores
        // on every path keeps the compiler's count of memory operations in flight the same
        // on all paths, so that later waits for loads do not also wait for these stores)
        const bool pub_agg = jg != G - 1 && !last;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int x4 = tid + i * THREADS;
            st4_dev(rag, pub_agg && x4 < CH ? (uint32_t)(j * ENT + 4 * x4) * 4 : kOut, ag[i]);
        }
        // the in-span products below run while the stores complete
        __builtin_amdgcn_sched_barrier(0);
        // in-span outputs A V: lane = column 32 mb + c, register r = query T0 + tok(r)
        f32x16_t ov[MB];
        {
            const float af[16] = {at[0], at[1], at[2],  at[3],  at[4],  at[5],  at[6],  at[7],
                                  at[8], at[9], at[10], at[11], at[12], at[13], at[14], at[15]};
            const Split8 as0 = split8(&af[0]), as1 = split8(&af[8]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                ov[mb] = (f32x16_t){};
                ov[mb] = mma_x3(as0, vs[mb][0], ov[mb]);
                ov[mb] = mma_x3(as1, vs[mb][1], ov[mb]);
            }
        }
        if (pub_agg) publish(a.flag_agg + (size_t)hh * a.S + j, a.epoch);
        // every flag this span needs (the previous group's inclusive prefix, the earlier
        // spans of its own group) is polled together, then all their data is loaded at
        // once and added in the fixed order
        bool ok = true;
        if (j > 0) {
            // device-scope (sc1) loads through buffer resources, so that the polls of one
            // round are all in flight together; the compiler barrier makes every round load
            // again
            const rsrc_t fa = rsrc_u64(a.flag_agg + (size_t)hh * a.S, a.S);
            const rsrc_t fi = rsrc_u64(a.flag_incl + (size_t)hh * a.SG, a.SG);
            ok = false;
            for (int it = 0; it < kSpins && !ok; ++it) {
                asm volatile("" ::: "memory");
                // (unconditional loads; an index past a resource, the previous group's for
                // g0 = 0 included, reads 0 and is not used)
                unsigned long long f[G];
#pragma unroll
                for (int u = 0; u < G; ++u) f[u] = ld_flag(fa, g0 + u);
                const unsigned long long fg = ld_flag(fi, g0 / G - 1);
                bool all = g0 == 0 || fg == a.epoch;
#pragma unroll
                for (int u = 0; u < G; ++u) all &= g0 + u >= j || f[u] == a.epoch;
                ok = all;
                if (!ok) __builtin_amdgcn_s_sleep(4);
            }
            asm volatile("" ::: "memory");  // the data loads stay after the flags
        }
        f32x4_t pr[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int x4 = tid + i * THREADS;
            pr[i] = ld4_dev(rin, g0 > 0 && x4 < CH ? (uint32_t)((g0 / G - 1) * ENT + 4 * x4) * 4 : kOut);
        }
        for (int k0 = g0; k0 < j; k0 += NB) {  // NB aggregates in flight
            f32x4_t t[NB][PER];
#pragma unroll
            for (int u = 0; u < NB; ++u)
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int x4 = tid + i * THREADS;
                    t[u][i] = ld4_dev(rag, k0 + u < j && x4 < CH ? (uint32_t)((k0 + u) * ENT + 4 * x4) * 4 : kOut);
                }
            // (slots past j - 1 were read at kOut: zeros)
#pragma unroll
            for (int u = 0; u < NB; ++u)
#pragma unroll
                for (int i = 0; i < PER; ++i) pr[i] += t[u][i];
        }
        if (!ok)
#pragma unroll
            for (int i = 0; i < PER; ++i) pr[i] = (f32x4_t)__builtin_nanf("");
        // ---- 3. exclusive prefix of each wave's block, in place; the group's last span
        // publishes its inclusive prefix
        const bool pub_incl = jg == G - 1 && !last;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int x4 = tid + i * THREADS;
            if (x4 < CH) {
                const int o = lds_of4(x4);
                f32x4_t run = pr[i];
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    const f32x4_t t = lds4(lds, ww * REG + o);
                    lds4(lds, ww * REG + o) = run;
                    run += t;
                }
                if (pub_incl) st4_dev(rin, (uint32_t)((j / G) * ENT + 4 * x4) * 4, run);
            }
        }
        if (pub_incl) publish(a.flag_incl + (size_t)hh * a.SG + j / G, a.epoch);
        __syncthreads();

        // outputs: + phi(Q) (exclusive prefix), over e in the order of qf
        // (16 terms per bf16 product: lane half h gives e = 32 eb + 16 kk + 8 (j / 4) + 4 h
        // + j % 4, j = 0 .. 7, which are qf[16 eb + 8 kk + j])
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const Split8 qs = split8(&qf[16 * eb + 8 * kk]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int o = (32 * mb + c) * EP + 32 * eb + 16 * kk + 4 * h;
                    const f32x4_t b0 = lds4(reg, o), b1 = lds4(reg, o + 8);
                    const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                    ov[mb] = mma_x3(qs, split8(bv), ov[mb]);
                }
            }
        float inv = 1.f;
        if (fm) {
            float d = 0.f;
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4_t zv = lds4(reg, M * EP + 32 * eb + 8 * g + 4 * h);
#pragma unroll
                    for (int t = 0; t < 4; ++t) d = fmaf(qf[16 * eb + 4 * g + t], zv[t], d);
                }
            d += __shfl_xor(d, 32);
            inv = 1.f / (d + rs + a.eps);
        }
        // Outputs through this wave's LDS region (its prefix state and key sum have been
        // read): the accumulators (lane = column, registers = rows) become rows of OP
        // floats, then each lane scales and stores 16-byte pieces of whole rows.  (Row pitch
        // M + 8: the lane halves write rows 4 apart, on the two halves of the banks.)
        constexpr int OP = M + 8, PIECES = TS * M / 4 / 64;
        static_assert(TS * OP <= REG, "the output rows fit in a wave's region");
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) reg[(8 * (r >> 2) + 4 * h + (r & 3)) * OP + 32 * mb + c] = ov[mb][r];
        // (store offsets from a lane id taken here, so that the compiler does not keep the
        // load offsets of the start alive until now)
        const uint32_t ln = lane_now();
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const uint32_t q = ln + 64 * p, row = q / (M / 4), col = 4 * (q % (M / 4));
            const f32x4_t x = lds4(reg, row * OP + col) * __shfl(inv, (int)row);  // (inv = 1 without the feature map)
            st4(ro, ((uint32_t)(T0 + row) * M + col) * 4, x);
        }
    }

    // workspace layout (bytes from the start; every part 256-byte aligned)
    struct Layout {
        size_t flag_agg, flag_incl, agg, incl, bytes;
    };
    static Layout layout(long long BH, long long S, long long SG) {
        auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
        Layout l;
        l.flag_agg = 0;
        l.flag_incl = up(l.flag_agg + (size_t)BH * S * 8);
        l.agg = up(l.flag_incl + (size_t)BH * SG * 8);
        l.incl = up(l.agg + (size_t)BH * S * ENT * 4);
        l.bytes = up(l.incl + (size_t)BH * SG * ENT * 4);
        return l;
    }
};

template <int E, int M, int NW = 4>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_linear_scan_kernel(LinScanArgs a) {
    LinScan<E, M, NW>::run(a);
}

}  // namespace attn
