// Persistent form of the matrix-core forward: equal query and key lengths, no
// caller mask, scale >= 0 (the problem attn_fwd states).
//
// The work is the same as MfmaFwd<T, D, CAUSAL, kFwdPlain> (same tiles of 256
// query rows, same 64-key units, same matrix and softmax phases, same ping-pong of
// two wave groups, same K/V rings in LDS), but one workgroup per compute unit walks
// a list of query tiles ("Understand FlashAttention", section "FlashAttention":
// the outer loop over row blocks of Q) and carries its pipeline from one tile into
// the next, so that the costs a tile pays once are paid while other work runs:
//
//   * K/V.  The load groups run three units ahead of the compute through one
//     continuous sequence of positions: the groups issued in a tile's last steps
//     carry the next tile's first units (no cold prologue per tile).
//   * Q.  A wave loads the next tile's 32 Q rows into its operand registers in the
//     softmax phase of the tile's last step, after the last score product that reads
//     the old ones; they are needed one phase later.  Three steps earlier the same
//     rows are fetched into the L2 (1 KB loads into an LDS landing zone that nothing
//     reads), so that this load does not wait for HBM.
//   * P V of the last unit.  The matrix phase of a tile's first step, which computes
//     the scores of the new tile's first unit, also finishes P V of the previous
//     tile's last unit; that wave then writes the previous tile's rows (O = O~ / l,
//     lse) in the softmax phase, before the softmax of the new unit.  A wave whose
//     rows end earlier in the tile writes them in the step after its last unit.
//
// Each tile takes a whole number of ring turns (its unit count rounded up to a
// multiple of 4; the extra steps only load and pass barriers), so a unit's ring
// stage is its index in the tile mod 4 and the main loop keeps its stages as
// immediates.
//
// Registers.  The tile loop has to fit the 256 registers a wave has at two waves per
// SIMD with nothing spilled: a spill's reload waits for every load in flight, the
// K/V DMA included.  So, compared with the one-tile kernel: the softmax phase reads
// only the first 32-key half of the next unit's K fragments and the matrix phase the
// second (MfmaFwd::kload_half / gemm_half); all fragment addresses come from two
// registers by XOR (MfmaFwd::frag_addr); the lanes' DMA offsets sit in LDS and are
// read where a load group is issued; lane coordinates are rebuilt from the lane id
// where used; zeros are written with a v_mov each where needed.
//
// Work lists.  Causal tiles pair up: query tile j with tile nq - 1 - j of the same
// head (the long one first), so every pair has the same number of units, nq + 1
// tiles' worth; non-causal tiles are equal and go singly.  Such a pair or tile is a
// job.  When the head count and the grid are multiples of 8, the workgroups on XCD
// x (block index = x mod 8) take the jobs of the heads congruent to x mod 8, in head
// order, so the workgroups of one XCD work on one or two heads at a time and read
// their K/V units through that XCD's L2; otherwise the jobs are dealt round robin.
// Workgroup g takes jobs g, g + G, g + 2G, ... of its list.
#pragma once

#include "fwd_mfma.hpp"

namespace attn {

template <typename T, int D, bool CAUSAL>
struct MfmaFwdPersist {
    typedef MfmaFwd<T, D, CAUSAL, kFwdPlain> F;
    static constexpr int NW = F::NW, BR = F::BR, BU = F::BU, STAGES = F::STAGES, THREADS = F::THREADS;
    static constexpr int ROWB = F::ROWB, UNIT_B = F::UNIT_B, V_BASE = F::V_BASE;
    static constexpr int LOADS = F::LOADS, KVLOADS = F::KVLOADS, DB = F::DB, DC = F::DC;
    static constexpr int OFFS_BASE = F::LDS_B;  // per-thread load offsets follow the rings
    static constexpr int QPF_BASE = OFFS_BASE + THREADS * 8;  // 1 KB per wave: landing zone of the Q prefetch
    static constexpr int LDS_B = QPF_BASE + NW * 1024;
    static_assert(LDS_B <= 160 * 1024, "LDS budget");
    static constexpr int MID = F::GROUP * (STAGES - 2), END = F::GROUP * (STAGES - 3);
    static constexpr int QLOADS = DC;  // 16-byte loads per lane for a wave's 32 Q rows
    static_assert(STAGES == 4 && F::GROUP == KVLOADS, "positions padded to whole ring turns; no mask loads");
    typedef typename F::State State;
    typedef typename F::Packed Packed;
    typedef typename F::KFrags KFrags;

    // One tile of a workgroup's list: job jl of the workgroup, part 0 or 1 of it.
    struct Tile {
        int jl, part, parts, bh, qt;
        bool valid;
    };

    // Fills bh, qt, parts and valid of t from t.jl and t.part.
    static __device__ __forceinline__ void tile_set(const FwdArgs &a, int g, int n_jobs, Tile &t) {
        t.valid = t.jl < n_jobs;
        if (!t.valid) return;
        int head, jj;
        if (a.p_xcd) {
            const int jx = (g >> 3) + t.jl * (a.p_grid >> 3);
            const int hi = jx / a.p_jph;
            head = (g & 7) + 8 * hi;
            jj = jx - hi * a.p_jph;
        } else {
            const int J = g + t.jl * a.p_grid;
            head = J / a.p_jph;
            jj = J - head * a.p_jph;
        }
        t.bh = head;
        if (CAUSAL) {
            const int longer = a.n_qtiles - 1 - jj;
            t.parts = longer != jj ? 2 : 1;
            t.qt = t.part == 0 ? longer : jj;
        } else {
            t.parts = 1;
            t.qt = jj;
        }
    }
    static __device__ __forceinline__ void tile_next(const FwdArgs &a, int g, int n_jobs, Tile &t) {
        if (t.part + 1 < t.parts) {
            ++t.part;
        } else {
            ++t.jl;
            t.part = 0;
        }
        tile_set(a, g, n_jobs, t);
    }
    // Key units the workgroup walks for query tile qt (causal: up to its last row).
    static __device__ __forceinline__ int tile_units(int qt, int N) {
        const int n_units = (N + BU - 1) / BU;
        if (!CAUSAL) return n_units;
        return max(1, min(n_units, (min(qt * BR + BR, N) - 1) / BU + 1));
    }

    static __device__ void run(const FwdArgs &a) {
        extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
        const int N = a.Nq;
        const int g = blockIdx.x;
        int n_jobs;
        if (a.p_xcd) {
            const int per_x = (a.p_nbh >> 3) * a.p_jph, s = g >> 3, gx = a.p_grid >> 3;
            n_jobs = s < per_x ? (per_x - s + gx - 1) / gx : 0;
        } else {
            const int tot = a.p_nbh * a.p_jph;
            n_jobs = g < tot ? (tot - g + a.p_grid - 1) / a.p_grid : 0;
        }
        Tile ct;
        ct.jl = 0;
        ct.part = 0;
        tile_set(a, g, n_jobs, ct);
        if (!ct.valid) return;  // (the host launches no more workgroups than jobs)

        const size_t head_elems = (size_t)N * D;
        const uint16_t *Qb = static_cast<const uint16_t *>(a.q);
        const char *Kb = static_cast<const char *>(a.k);
        const char *Vb = static_cast<const char *>(a.v);
        uint16_t *Ob = static_cast<uint16_t *>(a.o);

        const int tid = threadIdx.x;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63, l32 = lane & 31, gh = lane >> 5;
        const bool lag = w >= NW / 2;
        const int wrow = 64 * (w & 3) + 32 * (w >> 2);  // the wave's first row within a tile

        State S;
        S.Nk = N;
        S.off = 0;
        S.c = a.c;  // >= 0 (the host sends negative scales to the other kernel)

        // the wave's 32 Q rows of tile (bh, qt) as the B operand (rows past the end
        // read row N - 1: finite, and never stored)
        // (lane coordinates from lane_id_here() and a 32-bit offset within the head: no
        // per-lane address is kept live across the loop for this)
        auto load_q = [&](int bh, int qt) {
            const uint32_t ln = lane_id_here();
            const uint32_t q = (uint32_t)min(qt * BR + wrow + (int)(ln & 31u), N - 1);
            const char *qh = reinterpret_cast<const char *>(Qb + (size_t)bh * head_elems);
            const char *qrow = qh + (q * (uint32_t)ROWB + (ln >> 5) * 16u);
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) S.qf[cc] = F::as_v8(*reinterpret_cast<const u32x4_t *>(qrow + cc * 32));
        };
        // Zeros written where they are needed (a v_mov each): as constants the compiler
        // keeps a whole zero tuple live across the tile loop to copy from.
        auto zero = []() {
            float z;
            asm volatile("v_mov_b32 %0, 0" : "=v"(z));
            return z;
        };
        // L2 prefetch of the wave's 32 Q rows of tile (bh, qt): 1 KB loads straight into a
        // landing zone in LDS that nothing reads (the data only has to reach the L2), three
        // steps before load_q reads the rows; the barriers in between allow for them.
        auto prefetch_q = [&](int bh, int qt) {
            constexpr int RPL = 64 / F::CH;  // rows per 1 KB load
            const uint32_t ln = lane_id_here();
            const char *qh = reinterpret_cast<const char *>(Qb + (size_t)bh * head_elems);
            uint32_t zone = (uint32_t)(uintptr_t)(lds_void_t *)smem + QPF_BASE + (uint32_t)w * 1024u;
            asm volatile("" : "+s"(zone));
#pragma unroll
            for (int j = 0; j < QLOADS; ++j) {
                const uint32_t row = (uint32_t)min(qt * BR + wrow + j * RPL + (int)(ln / F::CH), N - 1);
                dma_to_lds16(qh, row * (uint32_t)ROWB + (ln % F::CH) * 16u, zone);
            }
        };
        static_assert(QLOADS * (64 / F::CH) == 32, "the prefetch covers the wave's 32 rows");
        auto reset = [&]() {
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) S.acc[b][i] = zero();
            S.m_ref = -INFINITY;
            S.lsum = 0.f;
        };

        // fragment read addresses (stage 0) and unit load offsets, as in MfmaFwd::run
        // (the dynamic LDS starts at an address whose low 8 bits are 0, so the fragment
        // addresses of k-step 0 and d block 0 determine the others by an XOR; see
        // MfmaFwd::kaddr_x)
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
        S.kaddr[0] = lds0 + l32 * ROWB + ((gh ^ F::kswz(l32)) << 4);
        {
            const int j16 = lane & 15, grp = lane >> 4;
            const int r_lane = 8 * (grp >> 1) + (j16 >> 2);
            const int c_lane = 2 * (grp & 1) + ((j16 & 3) >> 1);
            S.vaddr[0] = lds0 + V_BASE + r_lane * ROWB + ((c_lane ^ F::vswz(r_lane)) << 4) + 8 * (j16 & 1);
        }
        // unit load offsets: load 0 of each tensor; at d = 128 load 1 of K is load 0's
        // offset ^ 0x840 (8 rows on, chunk ^ 4 under the swizzle) and of V load 0's + 1024
        static_assert(LOADS == 1 || (LOADS == 2 && D == 128), "load offsets derived from load 0");
        uint32_t kld0, vld0;
        {
            const int s0 = (w * LOADS) * 64 + lane;
            const int r = s0 / F::CH, p = s0 % F::CH;
            kld0 = ((r & ~31) | swap_bits23(r & 31)) * ROWB + ((p ^ F::kswz(r)) << 4);
            vld0 = r * ROWB + ((p ^ F::vswz(r)) << 4);
        }
        // The two offsets live in LDS (8 bytes per thread past the rings) and are read where
        // a load group is issued, at an address made from the lane id: no register holds
        // them, or their address, across the loop.
        *reinterpret_cast<u32x2_t *>(smem + OFFS_BASE + 8 * tid) = (u32x2_t){kld0, vld0};
        const uint32_t offs_w = lds0 + OFFS_BASE + (uint32_t)w * 512u;  // wave-uniform
        auto offsets = [&]() {
            return *(const __attribute__((address_space(3))) u32x2_t *)(uintptr_t)(offs_w + 8u * lane_id_here());
        };

        // load j of a unit (16 bytes per lane) into a ring stage; rows past the end of
        // the sequence read row N - 1
        // (the lane's offset is made opaque where it is used, so that the compiler keeps one
        // register for it rather than hoisting parts of the clamp out of the loop)
        // The LDS destinations of a wave's loads are its base plus an immediate; the base is
        // made opaque at each use, so the compiler does not keep every sum in a register.
        const uint32_t wlds = lds0 + w * LOADS * 1024;
        auto dst_of = [&](int off) {
            uint32_t b = wlds;
            asm volatile("" : "+s"(b));
            return b + (uint32_t)off;
        };
        auto load_one = [&](const char *src_head, int k0, int lds_off, uint32_t ld, int j) {
            const char *src = src_head + (size_t)k0 * ROWB;
            const uint32_t dst = dst_of(lds_off + j * 1024);
            asm volatile("" : "+v"(ld));
            if (k0 + BU > N) {  // the sequence's last, partial unit
                const uint32_t last = (uint32_t)(N - 1 - k0) * ROWB;
                ld = min(ld & ~(uint32_t)(ROWB - 1), last) + (ld & (ROWB - 1));
            }
            dma_to_lds16(src, ld, dst);
        };
        // A load group: the K unit of one position and the V unit of the position before.
        struct Group {
            const char *kh, *vh;
            int k0, vk0;
        };
        // Tile geometry the load groups need: byte offset of the current tile's head and
        // its unit count U (positions 0 .. Upad - 1), and the same for the next tile of
        // the list (nvalid = 0 after the last one).  A position past U (padding) repeats
        // unit U - 1; positions Upad.. are the next tile's; after the last tile the last
        // unit is repeated.
        size_t c_off = 0, n_off = 0;
        int c_U = 1, c_Upad = 4, n_U = 1;
        bool n_valid = false;
        auto unit_of = [&](int p, size_t &off) -> int {  // key offset of position p's unit
            if (p < c_Upad) {
                off = c_off;
                return min(p, c_U - 1) * BU;
            }
            if (n_valid) {
                off = n_off;
                return min(p - c_Upad, n_U - 1) * BU;
            }
            off = c_off;
            return (c_U - 1) * BU;
        };
        // the group issued in step u: K of position u + 3, V of position u + 2
        auto group_at = [&](int u) {
            size_t ko, vo;
            const int k0 = unit_of(u + 3, ko), vk0 = unit_of(u + 2, vo);
            return Group{Kb + ko, Vb + vo, k0, vk0};
        };
        // load j of a group whose K stage is ks (V goes into stage ks - 1)
        auto issue_part = [&](const Group &gr, int ks, int j, u32x2_t ofs) {
            if (j < LOADS)
                load_one(gr.kh, gr.k0, ks * UNIT_B, j == 0 ? ofs[0] : (ofs[0] ^ 0x840u), j);
            else
                load_one(gr.vh, gr.vk0, V_BASE + ((ks + STAGES - 1) % STAGES) * UNIT_B, ofs[1] + (uint32_t)((j - LOADS) * 1024),
                         j - LOADS);
        };

        f32x16_t s[2];
        Packed pk;
        KFrags kf;
        auto zero_pk = [&]() {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                    for (int e = 0; e < 4; ++e) pk[h][kc][e] = __float_as_uint(zero());
        };
        auto pin_soft = [&]() {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) asm volatile("" : "+v"(*reinterpret_cast<u32x4_t *>(pk[h][kc])));
            asm volatile("" : "+v"(S.lsum), "+v"(S.m_ref));
        };
        auto barrier_mid = [&]() { F::template barrier<MID>(); };
        auto barrier_end = [&]() { F::template barrier<END>(); };
        // the barrier that ends a step in whose softmax phase the next tile's Q was loaded
        auto barrier_end_q = [&]() { F::template barrier<END + QLOADS>(); };

        // matrix phase of the step at ring stage st: scores of this position (K
        // fragments in kf), P V of the previous one (V in stage st - 1), and the load
        // group of position + 3 (K into stage st + 3, V into st + 2)
        auto mat = [&](auto stc, int u) {
            constexpr int ST = decltype(stc)::value;
            const Group gr = group_at(u);
            const u32x2_t ofs = offsets();
            F::gemm_half(S, s, pk, kf, ST * UNIT_B, ((ST + STAGES - 1) % STAGES) * UNIT_B,
                    [&](int j) { issue_part(gr, (ST + 3) % STAGES, j, ofs); });
        };
        auto mat_dyn = [&](int u) {
            const int st = u % STAGES;
            const Group gr = group_at(u);
            const u32x2_t ofs = offsets();
            F::gemm_half(S, s, pk, kf, st * UNIT_B, ((st + STAGES - 1) % STAGES) * UNIT_B,
                    [&](int j) { issue_part(gr, (st + 3) % STAGES, j, ofs); });
        };
        auto idle_loads = [&](int u) {
            const Group gr = group_at(u);
            const u32x2_t ofs = offsets();
#pragma unroll
            for (int j = 0; j < KVLOADS; ++j) issue_part(gr, (u + 3) % STAGES, j, ofs);
        };
        // A plain step whose loads are full units of the current tile (K of unit u + 3,
        // V of unit u + 2, both below the tile's last unit): no clamp, no lookup.
        auto mat_fast = [&](auto stc, int u) {
            constexpr int ST = decltype(stc)::value;
            {
                const char *kh = Kb + c_off + (size_t)(u + 3) * UNIT_B, *vh = Vb + c_off + (size_t)(u + 2) * UNIT_B;
                const u32x2_t ofs = offsets();
                F::gemm_half(S, s, pk, kf, ST * UNIT_B, ((ST + STAGES - 1) % STAGES) * UNIT_B, [&](int j) {
                    constexpr int KS = (ST + 3) % STAGES, VS = (ST + 2) % STAGES;
                    if (j < LOADS)
                        dma_to_lds16(kh, j == 0 ? ofs[0] : (ofs[0] ^ 0x840u), dst_of(KS * UNIT_B + j * 1024));
                    else
                        dma_to_lds16(vh + (j - LOADS) * 1024, ofs[1], dst_of(V_BASE + VS * UNIT_B + (j - LOADS) * 1024));
                });
            }
        };
        auto plain_step = [&](auto stc, int u) {
            constexpr int ST = decltype(stc)::value;
            mat_fast(stc, u);
            barrier_mid();
            F::kload_half(S, kf, ((ST + 1) % STAGES) * UNIT_B);
            F::template soft<false, false>(S, s, pk, u * BU);
            pin_soft();
            barrier_end();
        };

        // ---- prologue: Q of the first tile, load groups 0 (K of position 0 only; the V
        // stage that position -1 would use holds zeros and P is 0), 1 and 2
        load_q(ct.bh, ct.qt);
        reset();
        zero_pk();
        {
            u32x4_t *vz = reinterpret_cast<u32x4_t *>(smem + V_BASE + (STAGES - 1) * UNIT_B);
            for (int i = tid; i < UNIT_B / 16; i += THREADS) vz[i] = (u32x4_t){0u, 0u, 0u, 0u};
        }
        Tile nt = ct;
        tile_next(a, g, n_jobs, nt);
        c_off = (size_t)ct.bh * head_elems * 2;
        c_U = tile_units(ct.qt, N);
        c_Upad = (c_U + 3) & ~3;
        n_valid = nt.valid;
        if (n_valid) {
            n_off = (size_t)nt.bh * head_elems * 2;
            n_U = tile_units(nt.qt, N);
        }
        {
            const Group gr = group_at(-3);  // K of position 0
#pragma unroll
            for (int j = 0; j < LOADS; ++j) issue_part(gr, 0, j, (u32x2_t){kld0, vld0});
        }
#pragma unroll
        for (int i = 1; i < STAGES - 1; ++i) {
            const Group gr = group_at(i - 3);
#pragma unroll
            for (int j = 0; j < KVLOADS; ++j) issue_part(gr, i, j, (u32x2_t){kld0, vld0});
        }
        barrier_mid();
        if (lag) barrier_end();

        bool pending = false;  // P V of the previous tile's last unit and its rows still to do
        int p_bh = 0, p_r0 = 0;
        const int n_units = (N + BU - 1) / BU;
        for (;;) {
            const int Upad = c_Upad;
            const int r0 = ct.qt * BR + wrow;
            S.r0 = r0;
            // this wave's units; the last one takes the masked softmax
            const int nu = r0 >= N ? 0 : (CAUSAL ? min(n_units, min(r0 + 31, N - 1) / BU + 1) : n_units);
            const int n_full = CAUSAL ? (min(r0, N - 1) + 1) / BU : N / BU;
            const int nm = max(0, min(nu - 1, n_full));
            // step 0: scores of unit 0; P V of the previous tile's last unit (pending) or
            // of P = 0; then that tile's rows, and the first softmax of this one
            // (the first half of unit 0's K fragments is read here rather than in the previous
            // step: fewer registers live across the tile loop)
            F::kload_half(S, kf, 0);
            __builtin_amdgcn_sched_barrier(0);
            mat(std::integral_constant<int, 0>(), 0);
            barrier_mid();
            if (pending) {
                // (nothing is scheduled across the rows' stores: the next unit's K fragments
                // are read only after them)
                __builtin_amdgcn_sched_barrier(0);
                F::epilogue(S, Ob + (size_t)p_bh * head_elems, a.lse + (size_t)p_bh * N, p_r0, N, (int)lane_id_here());
                reset();
                __builtin_amdgcn_sched_barrier(0);
            }
            if (nu >= 1) {
                F::kload_half(S, kf, 1 * UNIT_B);
                if (nm == 0)
                    F::template soft<true, true>(S, s, pk, 0);
                else
                    F::template soft<false, true>(S, s, pk, 0);
            } else {
                zero_pk();
            }
            pin_soft();
            barrier_end();

            // plain steps 1 .. nm - 1, unrolled by four (ring stages 1, 2, 3, 0)
            int u = 1;
            for (; u + STAGES <= nm && u + 6 < c_U; u += STAGES) {
                plain_step(std::integral_constant<int, 1>(), u);
                plain_step(std::integral_constant<int, 2>(), u + 1);
                plain_step(std::integral_constant<int, 3>(), u + 2);
                plain_step(std::integral_constant<int, 0>(), u + 3);
            }
            // Steps from pf_u = Upad - 3 on are never in the loop above.  In the softmax phase
            // of step pf_u every wave prefetches its next-tile Q rows; the barriers of the
            // next three phases allow those loads to be in flight (they are older than the
            // load group that the barrier ending step pf_u + 1 waits for).
            const int pf_u = Upad - 3;
            const bool qpf = nt.valid;
            auto bmid = [&](int uu) {
                if (qpf && (uu == pf_u + 1 || uu == pf_u + 2))
                    F::template barrier<MID + QLOADS>();
                else
                    F::template barrier<MID>();
            };
            auto bend = [&](int uu) {
                if (qpf && (uu == pf_u || uu == pf_u + 1))
                    F::template barrier<END + QLOADS>();
                else
                    F::template barrier<END>();
            };
            auto maybe_prefetch = [&](int uu) {
                if (qpf && uu == pf_u) prefetch_q(nt.bh, nt.qt);
            };
            for (; u < nm; ++u) {
                mat_dyn(u);
                bmid(u);
                F::kload_half(S, kf, ((u + 1) % STAGES) * UNIT_B);
                F::template soft<false, false>(S, s, pk, u * BU);
                pin_soft();
                maybe_prefetch(u);
                bend(u);
            }
            // The rest of the tile.  The last step (u = Upad - 1) ends in one shared tail,
            // whatever its kind: the K fragments of the next tile's first unit (stage 0),
            // the next tile's Q, and the barrier that ends the step.
            // the masked unit (u = nu - 1 >= 1)
            if (u < nu) {
                mat_dyn(u);
                bmid(u);
                F::template soft<true, false>(S, s, pk, u * BU);
                pin_soft();
                maybe_prefetch(u);
                if (u + 1 < Upad) {
                    F::kload_half(S, kf, ((u + 1) % STAGES) * UNIT_B);
                    bend(u);
                }
                ++u;
            }
            // P V of this wave's last unit and its rows (unless that is the next tile's
            // step 0: nu = Upad)
            if (nu >= 1 && u < Upad) {
                mat_dyn(u);
                bmid(u);
                __builtin_amdgcn_sched_barrier(0);
                F::epilogue(S, Ob + (size_t)ct.bh * head_elems, a.lse + (size_t)ct.bh * N, r0, N, (int)lane_id_here());
                reset();
                zero_pk();
                __builtin_amdgcn_sched_barrier(0);
                pin_soft();
                maybe_prefetch(u);
                if (u + 1 < Upad) bend(u);
                ++u;
            }
            // steps after this wave's rows are done: loads and barriers only
            for (; u < Upad; ++u) {
                idle_loads(u);
                bmid(u);
                maybe_prefetch(u);
                if (u + 1 < Upad) bend(u);
            }
            if (nt.valid) {
                load_q(nt.bh, nt.qt);
                barrier_end_q();
            } else {
                barrier_end();
            }
            pending = nu == Upad;
            p_bh = ct.bh;
            p_r0 = r0;
            if (!nt.valid) break;
            ct = nt;
            nt = ct;
            tile_next(a, g, n_jobs, nt);
            c_off = n_off;
            c_U = n_U;
            c_Upad = (c_U + 3) & ~3;
            n_valid = nt.valid;
            if (n_valid) {
                n_off = (size_t)nt.bh * head_elems * 2;
                n_U = tile_units(nt.qt, N);
            }
        }
        // closing step: P V of the last unit and the rows of waves still pending
        if (pending) F::gemm_half(S, s, pk, kf, 0, (STAGES - 1) * UNIT_B, [&](int) {});
        barrier_mid();
        if (pending) F::epilogue(S, Ob + (size_t)p_bh * head_elems, a.lse + (size_t)p_bh * N, p_r0, N, (int)lane_id_here());
        barrier_end();
        if (!lag) F::template barrier<0>();
        // every DMA of this wave has landed before it leaves
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1)
void attn_fwd_persist_kernel(FwdArgs a) {
    static_assert(MfmaFwdPersist<T, D, CAUSAL>::THREADS == 512, "launch bounds");
    MfmaFwdPersist<T, D, CAUSAL>::run(a);
}

}  // namespace attn
