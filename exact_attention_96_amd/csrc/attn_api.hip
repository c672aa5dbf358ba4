// C ABI of the attention library: argument checks, kernel selection, launch.
// The operation and every argument are specified in include/attn.h.
#include "attn.h"

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "fwd_f32.hpp"
#include "bwd_mfma.hpp"
#include "fwd_mfma.hpp"

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

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdArgs &a, int bh, hipStream_t stream) {
    constexpr int QW = attn::F32Fwd<D, CAUSAL>::QW;
    FwdArgs b = a;
    b.n_qtiles = (a.N + QW - 1) / QW;
    b.total = bh * b.n_qtiles;  // bounded by the check in attn_fwd
    return launch(&attn::attn_fwd_f32_kernel<D, CAUSAL>, b.total, attn::F32Fwd<D, CAUSAL>::THREADS, 0, stream, b);
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

template <typename T, int D, bool CAUSAL>
hipError_t launch_mfma(const FwdArgs &a, int bh, hipStream_t stream) {
    typedef attn::MfmaFwd<T, D, CAUSAL> K;
    FwdArgs b = a;
    b.n_qtiles = (a.N + K::BR - 1) / K::BR;
    b.total = bh * b.n_qtiles;  // bounded by the check in attn_fwd
    constexpr int lds_bytes = K::LDS_B;
    const hipError_t attr =
        opt_in_lds<K>(reinterpret_cast<const void *>(&attn::attn_fwd_mfma_kernel<T, D, CAUSAL>), lds_bytes);
    if (attr != hipSuccess) return attr;
    return launch(&attn::attn_fwd_mfma_kernel<T, D, CAUSAL>, b.total, K::THREADS, lds_bytes, stream, b);
}

template <int D, bool CAUSAL>
hipError_t dispatch_dtype(const FwdArgs &a, int bh, int dtype, hipStream_t stream) {
    switch (dtype) {
        case ATTN_F32: return launch_f32<D, CAUSAL>(a, bh, stream);
        case ATTN_F16: return launch_mfma<_Float16, D, CAUSAL>(a, bh, stream);
        default: return launch_mfma<__bf16, D, CAUSAL>(a, bh, stream);
    }
}

template <int D>
hipError_t dispatch_causal(const FwdArgs &a, int bh, int causal, int dtype, hipStream_t stream) {
    return causal ? dispatch_dtype<D, true>(a, bh, dtype, stream)
                  : dispatch_dtype<D, false>(a, bh, dtype, stream);
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

}  // namespace

extern "C" ATTN_API int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                        int N, int d, float scale, int causal, int dtype, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
    if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_EINVAL;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!isfinite(scale)) return ATTN_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return ATTN_EINVAL;
    const uint64_t elt = dtype == ATTN_F32 ? 4 : 2;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t tbytes = rows * (uint64_t)d * elt;
    const uint64_t lbytes = rows * 4;
    if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) || overlaps(o, tbytes, v, tbytes) ||
        overlaps(lse, lbytes, q, tbytes) || overlaps(lse, lbytes, k, tbytes) ||
        overlaps(lse, lbytes, v, tbytes) || overlaps(lse, lbytes, o, tbytes))
        return ATTN_EINVAL;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    // the smallest query tile is 32 rows; the 1-D grid holds at most INT32_MAX workgroups
    if ((uint64_t)B * (uint64_t)H * (((uint64_t)N + 31) / 32) > (uint64_t)INT32_MAX) return ATTN_EUNSUPPORTED;

    FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.N = N;
    a.n_qtiles = 0;
    a.total = 0;
    a.c = (float)((double)scale * 1.4426950408889634073599);
    const int bh = B * H;
    const hipError_t err = d == 64 ? dispatch_causal<64>(a, bh, causal, dtype, stream)
                                   : dispatch_causal<128>(a, bh, causal, dtype, stream);
    return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

extern "C" ATTN_API int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                                 const void *dout, void *dq, void *dk, void *dv, float *delta, int B, int H, int N,
                                 int d, float scale, int causal, int dtype, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return ATTN_EINVAL;
    if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_EINVAL;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!isfinite(scale)) return ATTN_EINVAL;
    const void *in16[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void *p : in16)
        if (!aligned(p, 16)) return ATTN_EINVAL;
    if (!aligned(lse, 4) || !aligned(delta, 4)) return ATTN_EINVAL;
    const uint64_t elt = dtype == ATTN_F32 ? 4 : 2;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t tb = rows * (uint64_t)d * elt, lb = rows * 4;
    // each output against every input and every other output
    const void *outs[] = {dq, dk, dv, delta};
    const uint64_t out_b[] = {tb, tb, tb, lb};
    const void *ins[] = {q, k, v, o, dout, lse};
    const uint64_t in_b[] = {tb, tb, tb, tb, tb, lb};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], out_b[i], ins[j], in_b[j])) return ATTN_EINVAL;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], out_b[i], outs[j], out_b[j])) return ATTN_EINVAL;
    }
    if (dtype == ATTN_F32) return ATTN_EUNSUPPORTED;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    if ((uint64_t)B * (uint64_t)H * (((uint64_t)N + 127) / 128) > (uint64_t)INT32_MAX) return ATTN_EUNSUPPORTED;
    if ((rows * (uint64_t)d / 8 + 255) / 256 > (uint64_t)INT32_MAX) return ATTN_EUNSUPPORTED;

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

extern "C" ATTN_API const char *attn_strerror(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_EINVAL: return "invalid argument";
        case ATTN_EUNSUPPORTED: return "unsupported head dimension or problem size";
        case ATTN_EHIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

extern "C" ATTN_API int attn_abi_version(void) { return ATTN_ABI_VERSION; }
