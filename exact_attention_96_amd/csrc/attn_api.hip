// C ABI of the attention library: argument checks, kernel selection, launch.
// The operation and every argument are specified in include/attn.h.
#include "attn.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <chrono>
#include <random>
#include <utility>

#include "fwd_f32.hpp"
#include "bwd_mfma.hpp"
#include "fwd_mfma.hpp"
#include "fwd_persist.hpp"
#include "linattn.hpp"
#include "linscan.hpp"

namespace {

using attn::BwdArgs;
using attn::FwdArgs;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Half-open byte ranges [p, p + n) and [r, r + m) intersect.
bool overlaps(const void *p, uint64_t n, const void *r, uint64_t m) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(r);
    return a0 < b0 + m && b0 < a0 + n;
}

// Launch with the given kernel arguments (their types must be the kernel's parameter
// types); returns this launch's own status (not an error left behind by an earlier call).
template <typename Kernel, typename... Args>
hipError_t launch(Kernel *kernel, int grid, int threads, int lds_bytes, hipStream_t stream, Args... args) {
    void *argv[] = {&args...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(grid), dim3(threads), argv,
                           static_cast<size_t>(lds_bytes), stream);
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch_f32(const FwdArgs &a, int bh, hipStream_t stream) {
    typedef attn::F32Fwd<D, CAUSAL, MASK> K;
    FwdArgs b = a;
    b.n_qtiles = (a.Nq + K::QW - 1) / K::QW;
    b.total = bh * b.n_qtiles;  // bounded by the check in fwd_core
    return launch(&attn::attn_fwd_f32_kernel<D, CAUSAL, MASK>, b.total, K::THREADS, 0, stream, b);
}

// Opt a kernel in to its dynamic LDS size, once per device (devices 0..63; others
// every call).  Tag names the kernel: one flag set per instantiation.
template <typename Tag>
hipError_t opt_in_lds(const void *kernel, int lds_bytes) {
    static std::atomic<uint64_t> done{0};
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool tracked = dev >= 0 && dev < 64;
    if (tracked && ((done.load(std::memory_order_acquire) >> dev) & 1u)) return hipSuccess;
    const hipError_t r = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (r == hipSuccess && tracked) done.fetch_or(uint64_t(1) << dev, std::memory_order_release);
    return r;
}

template <typename T, int D, bool CAUSAL, int MODE>
hipError_t launch_mfma(const FwdArgs &a, int bh, hipStream_t stream) {
    typedef attn::MfmaFwd<T, D, CAUSAL, MODE> K;
    FwdArgs b = a;
    b.n_qtiles = (a.Nq + K::BR - 1) / K::BR;
    b.total = bh * b.n_qtiles;  // bounded by the check in fwd_core
    constexpr int lds_bytes = K::LDS_B;
    const hipError_t attr =
        opt_in_lds<K>(reinterpret_cast<const void *>(&attn::attn_fwd_mfma_kernel<T, D, CAUSAL, MODE>), lds_bytes);
    if (attr != hipSuccess) return attr;
    return launch(&attn::attn_fwd_mfma_kernel<T, D, CAUSAL, MODE>, b.total, K::THREADS, lds_bytes, stream, b);
}

// Compute units of the current device (cached for devices 0..63).
hipError_t device_cus(int *cus) {
    static std::atomic<int> cache[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool tracked = dev >= 0 && dev < 64;
    if (tracked) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    if (tracked) cache[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return hipSuccess;
}

// The persistent kernel: one workgroup per compute unit (at most one per job), each
// walking its list of jobs (pairs of causal query tiles, or single tiles).
template <typename T, int D, bool CAUSAL>
hipError_t launch_persist(const FwdArgs &a, int bh, hipStream_t stream) {
    typedef attn::MfmaFwdPersist<T, D, CAUSAL> K;
    FwdArgs b = a;
    b.n_qtiles = (a.Nq + K::BR - 1) / K::BR;
    b.total = bh * b.n_qtiles;  // bounded by the check in fwd_core
    b.p_nbh = bh;
    b.p_jph = CAUSAL ? (b.n_qtiles + 1) / 2 : b.n_qtiles;
    const long long jobs = (long long)bh * b.p_jph;
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const int grid = (int)(jobs < cus ? jobs : cus);
    b.p_grid = grid;
    b.p_xcd = (bh % 8 == 0 && grid % 8 == 0) ? 1 : 0;
    e = opt_in_lds<K>(reinterpret_cast<const void *>(&attn::attn_fwd_persist_kernel<T, D, CAUSAL>), K::LDS_B);
    if (e != hipSuccess) return e;
    return launch(&attn::attn_fwd_persist_kernel<T, D, CAUSAL>, grid, K::THREADS, K::LDS_B, stream, b);
}

// MODE: attn::kFwdPlain / kFwdOffset / kFwdBits (the fp32 kernel only tells masked
// from unmasked)
template <int D, bool CAUSAL, int MODE>
hipError_t dispatch_dtype(const FwdArgs &a, int bh, int dtype, hipStream_t stream) {
    switch (dtype) {
        case ATTN_F32: return launch_f32<D, CAUSAL, MODE == attn::kFwdBits>(a, bh, stream);
        case ATTN_F16: return launch_mfma<_Float16, D, CAUSAL, MODE>(a, bh, stream);
        default: return launch_mfma<__bf16, D, CAUSAL, MODE>(a, bh, stream);
    }
}

// Variant choice: a mask needs kFwdBits; a causal offset Nk - Nq that is not a
// multiple of 32 lets a wave's diagonal cross a unit boundary (kFwdOffset);
// everything else, including every equal-length problem, runs kFwdPlain.
template <int D>
hipError_t dispatch_mode(const FwdArgs &a, int bh, int causal, int dtype, hipStream_t stream) {
    // equal lengths, no mask, 16-bit inputs, scale >= 0: the persistent kernel
    if (!a.mask && a.Nq == a.Nk && dtype != ATTN_F32 && a.c >= 0.f) {
        if (dtype == ATTN_F16)
            return causal ? launch_persist<_Float16, D, true>(a, bh, stream)
                          : launch_persist<_Float16, D, false>(a, bh, stream);
        return causal ? launch_persist<__bf16, D, true>(a, bh, stream) : launch_persist<__bf16, D, false>(a, bh, stream);
    }
    if (a.mask)
        return causal ? dispatch_dtype<D, true, attn::kFwdBits>(a, bh, dtype, stream)
                      : dispatch_dtype<D, false, attn::kFwdBits>(a, bh, dtype, stream);
    if (!causal) return dispatch_dtype<D, false, attn::kFwdPlain>(a, bh, dtype, stream);
    if (a.off % 32 != 0) return dispatch_dtype<D, true, attn::kFwdOffset>(a, bh, dtype, stream);
    return dispatch_dtype<D, true, attn::kFwdPlain>(a, bh, dtype, stream);
}

// Packs a byte mask [rows, Nk] into bits [rows, ceil(Nk / 64)]: a wave makes
// PACK_WORDS consecutive 64-bit words per pass, each lane reading one key's byte of
// each (independent loads in flight); the wave's ballot is the word.
constexpr int PACK_WORDS = 8;
__global__ __launch_bounds__(256) void attn_mask_pack_kernel(const uint8_t *mask, uint64_t *bits, long long words,
                                                             int Nk, int w_per_row) {
    const int lane = threadIdx.x & 63;
    const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long n_waves = (long long)gridDim.x * 4;
    for (long long i0 = wave * PACK_WORDS; i0 < words; i0 += n_waves * PACK_WORDS) {
        bool on[PACK_WORDS];
#pragma unroll
        for (int t = 0; t < PACK_WORDS; ++t) {
            const long long i = i0 + t;
            const long long r = i / w_per_row;
            const int key = (int)(i - r * w_per_row) * 64 + lane;
            on[t] = i < words && key < Nk && mask[r * Nk + key] != 0;
        }
#pragma unroll
        for (int t = 0; t < PACK_WORDS; ++t) {
            const uint64_t word = __builtin_amdgcn_ballot_w64(on[t]);
            if (lane == 0 && i0 + t < words) bits[i0 + t] = word;
        }
    }
}

// Tile summary of packed bits [heads, Nq, W]: one wave per (head, query tile t, word
// wi of the summary row), lane = unit wi * 64 + lane; the lane ORs the unit's word
// over the tile's rows and the wave's ballot is the summary word.
__global__ __launch_bounds__(256) void attn_mask_tiles_kernel(const uint64_t *bits, uint64_t *tiles, long long words,
                                                              int Nq, int W, int nt, int tw) {
    const int lane = threadIdx.x & 63;
    const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long n_waves = (long long)gridDim.x * 4;
    for (long long i = wave; i < words; i += n_waves) {
        const long long ht = i / tw;  // head * nt + t
        const int wi = (int)(i - ht * tw);
        const long long head = ht / nt;
        const int t = (int)(ht - head * nt);
        const int u = wi * 64 + lane;
        uint64_t any = 0;
        if (u < W) {
            const int r0 = t * attn::kMaskTileRows, r1 = min(r0 + attn::kMaskTileRows, Nq);
            const uint64_t *col = bits + (head * Nq + r0) * (long long)W + u;
#pragma unroll 16
            for (int r = r0; r < r1; ++r, col += W) any |= *col;  // independent loads
        }
        const uint64_t word = __builtin_amdgcn_ballot_w64(any != 0);
        if (lane == 0) tiles[i] = word;
    }
}

// Backward: D_i = dO_i . O_i, then dQ and dK/dV (independent of each other).
template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs &a, int bh, hipStream_t stream) {
    typedef attn::BwdDq<T, D, CAUSAL> KQ;
    typedef attn::BwdDkv<T, D, CAUSAL> KKV;
    const size_t rows = (size_t)bh * (size_t)a.N;
    const size_t threads = rows * (D / 8);
    hipError_t e = launch(&attn::attn_bwd_delta_kernel<T, D>, (int)((threads + 255) / 256), 256, 0, stream, a.o,
                          a.dout, a.delta, rows);  // grid bounded by the check in attn_bwd
    if (e != hipSuccess) return e;
    BwdArgs b = a;
    b.n_tiles = (a.N + KQ::BR - 1) / KQ::BR;
    b.total = bh * b.n_tiles;  // bounded by the check in attn_bwd
    e = opt_in_lds<KQ>(reinterpret_cast<const void *>(&attn::attn_bwd_dq_kernel<T, D, CAUSAL>), KQ::LDS_B);
    if (e != hipSuccess) return e;
    e = launch(&attn::attn_bwd_dq_kernel<T, D, CAUSAL>, b.total, KQ::THREADS, KQ::LDS_B, stream, b);
    if (e != hipSuccess) return e;
    b.n_tiles = (a.N + KKV::BKV - 1) / KKV::BKV;
    b.total = bh * b.n_tiles;
    e = opt_in_lds<KKV>(reinterpret_cast<const void *>(&attn::attn_bwd_dkv_kernel<T, D, CAUSAL>), KKV::LDS_B);
    if (e != hipSuccess) return e;
    return launch(&attn::attn_bwd_dkv_kernel<T, D, CAUSAL>, b.total, KKV::THREADS, KKV::LDS_B, stream, b);
}

template <int D, bool CAUSAL>
hipError_t bwd_dtype(const BwdArgs &a, int bh, int dtype, hipStream_t stream) {
    return dtype == ATTN_F16 ? launch_bwd<_Float16, D, CAUSAL>(a, bh, stream)
                             : launch_bwd<__bf16, D, CAUSAL>(a, bh, stream);
}

template <int D>
hipError_t bwd_causal(const BwdArgs &a, int bh, int causal, int dtype, hipStream_t stream) {
    return causal ? bwd_dtype<D, true>(a, bh, dtype, stream) : bwd_dtype<D, false>(a, bh, dtype, stream);
}

// Checks and launch shared by attn_fwd and attn_fwd_masked (mask may be NULL).
int fwd_core(const void *q, const void *k, const void *v, const void *mask, const void *tiles, long long msb,
             long long msh, void *o, float *lse, int B, int H, int Nq, int Nk, int d, float scale, int causal,
             int dtype, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return ATTN_EINVAL;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!isfinite(scale)) return ATTN_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return ATTN_EINVAL;
    const uint64_t elt = dtype == ATTN_F32 ? 4 : 2;
    const uint64_t rows_q = (uint64_t)B * (uint64_t)H * (uint64_t)Nq;
    const uint64_t rows_k = (uint64_t)B * (uint64_t)H * (uint64_t)Nk;
    const uint64_t qb = rows_q * (uint64_t)d * elt, kb = rows_k * (uint64_t)d * elt;
    const uint64_t lbytes = rows_q * 4;
    const uint64_t mw = ((uint64_t)Nk + 63) / 64;  // mask words per row
    const uint64_t nt = ((uint64_t)Nq + attn::kMaskTileRows - 1) / attn::kMaskTileRows;  // summary tiles per head
    const uint64_t tw = (mw + 63) / 64;                                                 // summary words per tile
    uint64_t mbytes = 0, tbytes = 0;
    if (tiles && !mask) return ATTN_EINVAL;
    if (mask) {
        if (!aligned(mask, 8) || (tiles && !aligned(tiles, 8)) || msb < 0 || msh < 0) return ATTN_EINVAL;
        if ((uint64_t)msb > (1ull << 31) || (uint64_t)msh > (1ull << 31)) return ATTN_EUNSUPPORTED;
        // mask heads read: 0 .. (B-1) sb + (H-1) sh (checked in 64 bits)
        const uint64_t heads = (uint64_t)(B - 1) * (uint64_t)msb + (uint64_t)(H - 1) * (uint64_t)msh + 1;
        mbytes = heads * (uint64_t)Nq * mw * 8;
        tbytes = tiles ? heads * nt * tw * 8 : 0;
    }
    if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb) || overlaps(lse, lbytes, q, qb) ||
        overlaps(lse, lbytes, k, kb) || overlaps(lse, lbytes, v, kb) || overlaps(lse, lbytes, o, qb))
        return ATTN_EINVAL;
    if (mask && (overlaps(o, qb, mask, mbytes) || overlaps(lse, lbytes, mask, mbytes))) return ATTN_EINVAL;
    if (tiles && (overlaps(o, qb, tiles, tbytes) || overlaps(lse, lbytes, tiles, tbytes))) return ATTN_EINVAL;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    // the smallest query tile is 32 rows; the 1-D grid holds at most INT32_MAX workgroups
    if ((uint64_t)B * (uint64_t)H * (((uint64_t)Nq + 31) / 32) > (uint64_t)INT32_MAX) return ATTN_EUNSUPPORTED;
    // a head's mask rows are addressed with 32-bit byte offsets
    if (mask && (uint64_t)Nq * mw * 8 > (uint64_t)UINT32_MAX) return ATTN_EUNSUPPORTED;
    // the unit list of a query tile lives in LDS
    if (tiles && mw > (uint64_t)attn::MfmaFwd<__bf16, 128, false, attn::kFwdBits>::LIST_CAP) return ATTN_EUNSUPPORTED;

    FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.Nq = Nq;
    a.Nk = Nk;
    a.off = Nk - Nq;
    a.n_qtiles = 0;
    a.total = 0;
    a.c = (float)((double)scale * 1.4426950408889634073599);
    a.mask = static_cast<const uint64_t *>(mask);
    a.mask_sb = msb;
    a.mask_sh = msh;
    a.mask_w = (int)mw;
    a.H = H;
    a.tiles = static_cast<const uint64_t *>(tiles);
    a.tiles_w = (int)tw;
    a.tiles_nt = (int)nt;
    a.p_grid = a.p_jph = a.p_nbh = a.p_xcd = 0;
    const int bh = B * H;
    const hipError_t err = d == 64 ? dispatch_mode<64>(a, bh, causal, dtype, stream)
                                   : dispatch_mode<128>(a, bh, causal, dtype, stream);
    return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // namespace

extern "C" ATTN_API int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                                 int N, int d, float scale, int causal, int dtype, hipStream_t stream) {
    return fwd_core(q, k, v, nullptr, nullptr, 0, 0, o, lse, B, H, N, N, d, scale, causal, dtype, stream);
}

extern "C" ATTN_API int attn_fwd_masked(const void *q, const void *k, const void *v, const void *mask_bits,
                                        const void *mask_tiles, long long mask_stride_b, long long mask_stride_h,
                                        void *o, float *lse, int B, int H, int Nq, int Nk, int d, float scale,
                                        int causal, int dtype, hipStream_t stream) {
    return fwd_core(q, k, v, mask_bits, mask_tiles, mask_stride_b, mask_stride_h, o, lse, B, H, Nq, Nk, d, scale,
                    causal, dtype, stream);
}

extern "C" ATTN_API int attn_mask_pack(const void *mask, void *bits, void *tiles, long long heads, int Nq, int Nk,
                                       hipStream_t stream) {
    if (!mask || !bits || heads < 1 || Nq < 1 || Nk < 1) return ATTN_EINVAL;
    if (!aligned(bits, 8) || (tiles && !aligned(tiles, 8))) return ATTN_EINVAL;
    const uint64_t w = ((uint64_t)Nk + 63) / 64;
    const uint64_t nt = ((uint64_t)Nq + attn::kMaskTileRows - 1) / attn::kMaskTileRows, tw = (w + 63) / 64;
    if ((uint64_t)heads > (1ull << 40) / ((uint64_t)Nq * w)) return ATTN_EUNSUPPORTED;
    const uint64_t rows = (uint64_t)heads * (uint64_t)Nq;
    const uint64_t words = rows * w, twords = (uint64_t)heads * nt * tw;
    if (overlaps(bits, words * 8, mask, rows * (uint64_t)Nk)) return ATTN_EINVAL;
    if (tiles && (overlaps(tiles, twords * 8, mask, rows * (uint64_t)Nk) || overlaps(tiles, twords * 8, bits, words * 8)))
        return ATTN_EINVAL;
    const uint64_t blocks = (words + 4 * PACK_WORDS - 1) / (4 * PACK_WORDS);
    hipError_t e = launch(&attn_mask_pack_kernel, (int)(blocks < 65536 ? blocks : 65536), 256, 0, stream,
                          static_cast<const uint8_t *>(mask), static_cast<uint64_t *>(bits), (long long)words, Nk,
                          (int)w);
    if (e != hipSuccess || !tiles) return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
    const uint64_t tblocks = (twords + 3) / 4;
    e = launch(&attn_mask_tiles_kernel, (int)(tblocks < 65536 ? tblocks : 65536), 256, 0, stream,
               static_cast<const uint64_t *>(bits), static_cast<uint64_t *>(tiles), (long long)twords, Nq, (int)w,
               (int)nt, (int)tw);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

namespace {

// Checks and launches shared by attn_bwd and attn_bwd_noalloc.  delta: the caller's
// workspace (checked against every other buffer) or, with own_delta, the library's
// fixed scratch (nullptr here: it is looked up only after every check has passed).
int bwd_core(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
             void *dq, void *dk, void *dv, float *delta, bool own_delta, int B, int H, int N, int d, float scale,
             int causal, int dtype, hipStream_t stream);

}  // namespace

extern "C" ATTN_API int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                                 const void *dout, void *dq, void *dk, void *dv, float *delta, int B, int H, int N,
                                 int d, float scale, int causal, int dtype, hipStream_t stream) {
    if (!delta) return ATTN_EINVAL;
    return bwd_core(q, k, v, o, lse, dout, dq, dk, dv, delta, false, B, H, N, d, scale, causal, dtype, stream);
}

namespace {

// The scratch of attn_bwd_noalloc: D_i = dO_i . O_i for up to kScratchRows rows
// (16 MiB of fp32), one copy per GPU for the life of the process.  Host code never
// uses the symbol itself as an address: scratch_on_device() looks the device
// address up once per device (with that device current) and keeps it.
constexpr uint64_t kScratchRows = uint64_t(1) << 22;
static __device__ __align__(256) float scratch[kScratchRows];

hipError_t scratch_on_device(float **out) {
    static std::atomic<float *> addr[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool tracked = dev >= 0 && dev < 64;
    if (tracked) {
        float *p = addr[dev].load(std::memory_order_acquire);
        if (p) {
            *out = p;
            return hipSuccess;
        }
    }
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    if (tracked) addr[dev].store(static_cast<float *>(p), std::memory_order_release);
    *out = static_cast<float *>(p);
    return hipSuccess;
}

}  // namespace

extern "C" ATTN_API int attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                                         const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                                         int H, int N, int d, float scale, int causal, int dtype,
                                         hipStream_t stream) {
    return bwd_core(q, k, v, o, lse, dout, dq, dk, dv, nullptr, true, B, H, N, d, scale, causal, dtype, stream);
}

namespace {

int bwd_core(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
             void *dq, void *dk, void *dv, float *delta, bool own_delta, int B, int H, int N, int d, float scale,
             int causal, int dtype, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_EINVAL;
    if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_EINVAL;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!isfinite(scale)) return ATTN_EINVAL;
    const void *in16[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void *p : in16)
        if (!aligned(p, 16)) return ATTN_EINVAL;
    if (!aligned(lse, 4) || (!own_delta && !aligned(delta, 4))) return ATTN_EINVAL;
    const uint64_t elt = dtype == ATTN_F32 ? 4 : 2;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t tb = rows * (uint64_t)d * elt, lb = rows * 4;
    // each output against every input and every other output (the library's own
    // scratch overlaps nothing of the caller's)
    const void *outs[] = {dq, dk, dv, delta};
    const uint64_t out_b[] = {tb, tb, tb, lb};
    const int n_outs = own_delta ? 3 : 4;
    const void *ins[] = {q, k, v, o, dout, lse};
    const uint64_t in_b[] = {tb, tb, tb, tb, tb, lb};
    for (int i = 0; i < n_outs; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], out_b[i], ins[j], in_b[j])) return ATTN_EINVAL;
        for (int j = i + 1; j < n_outs; ++j)
            if (overlaps(outs[i], out_b[i], outs[j], out_b[j])) return ATTN_EINVAL;
    }
    if (dtype == ATTN_F32) return ATTN_EUNSUPPORTED;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    if ((uint64_t)B * (uint64_t)H * (((uint64_t)N + 127) / 128) > (uint64_t)INT32_MAX) return ATTN_EUNSUPPORTED;
    if ((rows * (uint64_t)d / 8 + 255) / 256 > (uint64_t)INT32_MAX) return ATTN_EUNSUPPORTED;
    if (own_delta) {
        if (rows > kScratchRows) return ATTN_ESCRATCH;
        const hipError_t e = scratch_on_device(&delta);
        if (e != hipSuccess) return ATTN_EHIP;
    }

    BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    a.N = N;
    a.n_tiles = 0;
    a.total = 0;
    a.c = (float)((double)scale * 1.4426950408889634073599);
    a.scale = scale;
    const int bh = B * H;
    const hipError_t err = d == 64 ? bwd_causal<64>(a, bh, causal, dtype, stream)
                                   : bwd_causal<128>(a, bh, causal, dtype, stream);
    return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // namespace

template <int E>
hipError_t launch_linear(const attn::LinArgs &a, int grid, hipStream_t stream) {
    typedef attn::LinFwd<E> K;
    const hipError_t e = opt_in_lds<K>(reinterpret_cast<const void *>(&attn::attn_linear_fwd_kernel<E>), K::LDS_B);
    if (e != hipSuccess) return e;
    return launch(&attn::attn_linear_fwd_kernel<E>, grid, K::THREADS, K::LDS_B, stream, a);
}

template <int E>
hipError_t launch_linear_chunked(const attn::LinChunkArgs &a, int bh, hipStream_t stream) {
    typedef attn::LinChunk<E> K;
    const int grid = bh * a.n_chunks;  // bounded by the checks in attn_linear_fwd
    const int s_lds = K::states_lds(a.M), o_lds = K::outputs_lds(a.M);
    // the LDS these kernels take depends on M: each is opted in once per device to the
    // whole 160 KB (the caller has checked that both sizes fit)
    struct StatesTag {};
    struct OutputsTag {};
    hipError_t e = opt_in_lds<std::pair<K, StatesTag>>(
        reinterpret_cast<const void *>(&attn::attn_linear_states_kernel<E>), 160 * 1024);
    if (e != hipSuccess) return e;
    e = opt_in_lds<std::pair<K, OutputsTag>>(reinterpret_cast<const void *>(&attn::attn_linear_outputs_kernel<E>),
                                             160 * 1024);
    if (e != hipSuccess) return e;
    e = launch(&attn::attn_linear_states_kernel<E>, grid, K::THREADS, s_lds, stream, a);
    if (e != hipSuccess) return e;
    const int per_chunk = E * a.M + E, bph = (per_chunk + 255) / 256;
    e = launch(&attn::attn_linear_prefix_kernel, bh * bph, 256, 0, stream, a.ws, a.n_chunks, per_chunk, bph);
    if (e != hipSuccess) return e;
    return launch(&attn::attn_linear_outputs_kernel<E>, grid, K::THREADS, o_lds, stream, a);
}

// The matrix-core chunk kernels (E >= 32) use no LDS.
template <int E>
hipError_t launch_linear_chunked_mfma(const attn::LinChunkArgs &a, int bh, hipStream_t stream) {
    const int grid = bh * a.n_chunks;  // bounded by the checks in attn_linear_fwd
    const int tiles = attn::LinChunkMfma<E>::STATE_TILES_PER_E * ((a.M + 31) / 32);
    hipError_t e = launch(&attn::attn_linear_states_mfma_kernel<E>, grid * tiles, 64, 0, stream, a);
    if (e != hipSuccess) return e;
    const int per_chunk = E * a.M + E, bph = (per_chunk + 255) / 256;
    e = launch(&attn::attn_linear_prefix_kernel, bh * bph, 256, 0, stream, a.ws, a.n_chunks, per_chunk, bph);
    if (e != hipSuccess) return e;
    return launch(&attn::attn_linear_outputs_mfma_kernel<E>, grid, 256, 0, stream, a);
}

// LDS of the larger of the chunked state and output kernels for (E, M); the LDS form
// (E = 16) is used only where both fit.
template <int E>
int linear_chunk_lds_e(int M) {
    const int s = attn::LinChunk<E>::states_lds(M), o = attn::LinChunk<E>::outputs_lds(M);
    return s > o ? s : o;
}
int linear_chunk_lds(int E, int M) { return E == 16 ? linear_chunk_lds_e<16>(M) : 0; }

// The one-pass kernel covers E, M in {32, 64}.
bool linear_scan_shape(int E, int M) { return (E == 32 || E == 64) && (M == 32 || M == 64); }

template <int E, int M>
typename attn::LinScan<E, M>::Layout linear_scan_layout_em(long long BH, int N) {
    typedef attn::LinScan<E, M> K;
    const long long S = ((long long)N + K::L - 1) / K::L, SG = (S + K::G - 1) / K::G;
    return K::layout(BH, S, SG);
}
size_t linear_scan_bytes(long long BH, int N, int E, int M) {
    if (E == 32) return M == 32 ? linear_scan_layout_em<32, 32>(BH, N).bytes : linear_scan_layout_em<32, 64>(BH, N).bytes;
    return M == 32 ? linear_scan_layout_em<64, 32>(BH, N).bytes : linear_scan_layout_em<64, 64>(BH, N).bytes;
}

extern "C" ATTN_API long long attn_linear_workspace_bytes(int B, int H, int N, int E, int M) {
    if (B < 1 || H < 1 || N < 1 || E < 1 || M < 1) return -1;
    const uint64_t chunks = ((uint64_t)N + attn::LinChunk<16>::TC - 1) / attn::LinChunk<16>::TC;
    const uint64_t chunked = (uint64_t)B * (uint64_t)H * chunks * ((uint64_t)E * (uint64_t)M + (uint64_t)E) * 4;
    if (!linear_scan_shape(E, M)) return (long long)chunked;
    const uint64_t scan = linear_scan_bytes((long long)B * H, N, E, M);
    return (long long)(scan > chunked ? scan : chunked);
}

// A fresh nonzero 64-bit flag value per call of the one-pass kernel: a counter from a
// random start, so that flags left in a workspace by earlier calls (or by whatever the
// memory held before) do not match.
unsigned long long next_epoch() {
    static std::atomic<unsigned long long> counter{[] {
        std::random_device rd;
        const unsigned long long t = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
        return ((unsigned long long)rd() << 32 ^ (unsigned long long)rd()) ^ (t * 0x9e3779b97f4a7c15ull);
    }()};
    unsigned long long e;
    do e = counter.fetch_add(1, std::memory_order_relaxed) + 1; while (e == 0);
    return e;
}

template <int E, int M>
hipError_t launch_linear_scan(const float *q, const float *k, const float *v, float *o, void *ws, int BH, int N,
                              int feature_map, float eps, hipStream_t stream) {
    typedef attn::LinScan<E, M> K;
    struct ScanTag {};
    const hipError_t e = opt_in_lds<std::pair<K, ScanTag>>(
        reinterpret_cast<const void *>(&attn::attn_linear_scan_kernel<E, M>), K::LDS_B);
    if (e != hipSuccess) return e;
    const long long S = ((long long)N + K::L - 1) / K::L, SG = (S + K::G - 1) / K::G;
    const typename K::Layout l = K::layout(BH, S, SG);
    char *base = static_cast<char *>(ws);
    attn::LinScanArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.flag_agg = reinterpret_cast<unsigned long long *>(base + l.flag_agg);
    a.flag_incl = reinterpret_cast<unsigned long long *>(base + l.flag_incl);
    a.agg = reinterpret_cast<float *>(base + l.agg);
    a.incl = reinterpret_cast<float *>(base + l.incl);
    a.epoch = next_epoch();
    a.N = N;
    a.BH = BH;
    a.BHp = (BH + 7) / 8 * 8;
    a.S = (int)S;
    a.SG = (int)SG;
    a.eps = eps;
    a.feature_map = feature_map;
    return launch(&attn::attn_linear_scan_kernel<E, M>, (int)((long long)a.BHp * S), K::THREADS, K::LDS_B, stream, a);
}

extern "C" ATTN_API int attn_linear_fwd(const float *q, const float *k, const float *v, float *o, int B, int H, int N,
                                        int E, int M, int feature_map, float eps, void *workspace,
                                        long long workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o) return ATTN_EINVAL;
    if (B < 1 || H < 1 || N < 1 || E < 1 || M < 1) return ATTN_EINVAL;
    if (feature_map != 0 && feature_map != 1) return ATTN_EINVAL;
    if (!isfinite(eps) || eps < 0.f) return ATTN_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ATTN_EINVAL;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t qb = rows * (uint64_t)E * 4, vb = rows * (uint64_t)M * 4;
    if (overlaps(o, vb, q, qb) || overlaps(o, vb, k, qb) || overlaps(o, vb, v, vb)) return ATTN_EINVAL;
    const long long need = attn_linear_workspace_bytes(B, H, N, E, M);
    if (workspace) {
        if (!aligned(workspace, 16) || workspace_bytes < need) return ATTN_EINVAL;
        const void *outs[] = {q, k, v, o};
        const uint64_t ob[] = {qb, qb, vb, vb};
        for (int i = 0; i < 4; ++i)
            if (overlaps(workspace, (uint64_t)need, outs[i], ob[i])) return ATTN_EINVAL;
    }
    if (E != 16 && E != 32 && E != 64 && E != 128) return ATTN_EUNSUPPORTED;
    if (M % 16 != 0) return ATTN_EUNSUPPORTED;
    const uint64_t grid = (uint64_t)B * (uint64_t)H * (uint64_t)(M / 16);
    if (grid > (uint64_t)INT32_MAX || (uint64_t)N * (uint64_t)(E > M ? E : M) > (uint64_t)INT32_MAX)
        return ATTN_EUNSUPPORTED;
    if (workspace && linear_scan_shape(E, M) && ((uint64_t)N + 256) * 64 * 4 < (1ull << 31) &&
        ((uint64_t)B * H + 7) / 8 * 8 * (((uint64_t)N + 127) / 128) <= (uint64_t)INT32_MAX) {
        const int bh = B * H;
        hipError_t e;
        if (E == 32)
            e = M == 32 ? launch_linear_scan<32, 32>(q, k, v, o, workspace, bh, N, feature_map, eps, stream)
                        : launch_linear_scan<32, 64>(q, k, v, o, workspace, bh, N, feature_map, eps, stream);
        else
            e = M == 32 ? launch_linear_scan<64, 32>(q, k, v, o, workspace, bh, N, feature_map, eps, stream)
                        : launch_linear_scan<64, 64>(q, k, v, o, workspace, bh, N, feature_map, eps, stream);
        return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
    }
    const uint64_t chunks = ((uint64_t)N + 63) / 64;
    // the matrix-core chunk kernels address a head's v and o, and a chunk's state, with
    // 32-bit byte offsets below 2^31 (rows up to one chunk past the end included)
    const uint64_t wide = (uint64_t)(E > M ? E : M);
    const bool mfma_ok = E >= 32 && ((uint64_t)N + 128) * wide * 4 < (1ull << 31) &&
                         ((uint64_t)E * M + E) * 4 < (1ull << 31) &&
                         (uint64_t)B * H * chunks * (E / 32) * ((M + 31) / 32) <= (uint64_t)INT32_MAX;
    if (workspace && (mfma_ok || (E == 16 && linear_chunk_lds(E, M) <= 160 * 1024)) && (uint64_t)B * (uint64_t)H * chunks <= (uint64_t)INT32_MAX &&
        (uint64_t)B * (uint64_t)H * (((uint64_t)E * M + E + 255) / 256) <= (uint64_t)INT32_MAX) {
        attn::LinChunkArgs c;
        c.q = q;
        c.k = k;
        c.v = v;
        c.o = o;
        c.ws = static_cast<float *>(workspace);
        c.N = N;
        c.M = M;
        c.n_chunks = (int)chunks;
        c.eps = eps;
        c.feature_map = feature_map;
        const int bh = B * H;
        hipError_t e;
        switch (E) {
            case 16: e = launch_linear_chunked<16>(c, bh, stream); break;
            case 32: e = launch_linear_chunked_mfma<32>(c, bh, stream); break;
            case 64: e = launch_linear_chunked_mfma<64>(c, bh, stream); break;
            default: e = launch_linear_chunked_mfma<128>(c, bh, stream); break;
        }
        return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
    }
    attn::LinArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.N = N;
    a.M = M;
    a.n_mslices = M / 16;
    a.eps = eps;
    a.feature_map = feature_map;
    hipError_t e;
    switch (E) {
        case 16: e = launch_linear<16>(a, (int)grid, stream); break;
        case 32: e = launch_linear<32>(a, (int)grid, stream); break;
        case 64: e = launch_linear<64>(a, (int)grid, stream); break;
        default: e = launch_linear<128>(a, (int)grid, stream); break;
    }
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

extern "C" ATTN_API const char *attn_strerror(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_EINVAL: return "invalid argument";
        case ATTN_EUNSUPPORTED: return "unsupported head dimension or problem size";
        case ATTN_EHIP: return "HIP runtime error at launch";
        case ATTN_ESCRATCH: return "problem larger than the fixed scratch of attn_bwd_noalloc (B*H*N above 2^22)";
        default: return "unknown status";
    }
}

extern "C" ATTN_API int attn_abi_version(void) { return ATTN_ABI_VERSION; }
