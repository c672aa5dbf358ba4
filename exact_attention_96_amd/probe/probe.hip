// Sustained-rate probes for the measurement harness (libattn_probe.so): the matrix
// cores and LDS reads at whatever clock the board holds under the load.  The C ABI is
// declared, with argument meanings and errors, in include/attn_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Four independent accumulator chains, eight products per iteration, each with another
// pair of operand registers, so that consecutive products see different data.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void probe_mfma_kernel(const u32x4_t *ops, float *out, int iters) {
    const int t = threadIdx.x;
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        a[f] = __builtin_bit_cast(bf16x8_t, ops[8 * t + f]);
        b[f] = __builtin_bit_cast(bf16x8_t, ops[8 * t + 4 + f]);
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[2], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[3], c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[0], c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(size_t)blockIdx.x * 256 + t] = s;
}

constexpr int kLdsBytes = 65536;

// Every read of a wave covers one window of consecutive pieces (1 KiB for 16-byte
// reads, 512 bytes for 8-byte ones); the window moves with every read and with the
// wave.  The compiler barrier at the top of each iteration makes every iteration read
// the LDS again; each value read is consumed by an empty asm statement (so that the
// reads are neither narrowed nor dropped, and no vector ALU work competes with them).
template <int MODE>
__global__ __launch_bounds__(512) void probe_lds_kernel(unsigned *out, int iters) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
    for (int p = 0; p < kLdsBytes / 4 / 512; ++p) lds[p * 512 + t] = (uint32_t)(p * 512 + t) * 2654435761u;
    __syncthreads();
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t *)lds;
    constexpr uint32_t piece = MODE == 0 ? 16 : 8, window = 64 * piece, nwin = kLdsBytes / window;
    typedef typename std::conditional<MODE == 0, u32x4_t, u32x2_t>::type piece_t;
    piece_t x[8];
    for (int i = 0; i < iters; ++i) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t win = (uint32_t)(w * 8 + i * 8 + u) % nwin;
            const uint32_t addr = base + win * window + (uint32_t)lane * piece;
            if constexpr (MODE == 0)
                x[u] = *(const lds_u32x4_t *)(uintptr_t)addr;
            else if constexpr (MODE == 1)
                x[u] = *(const lds_u32x2_t *)(uintptr_t)addr;
            else
                x[u] = __builtin_bit_cast(u32x2_t,
                                          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)addr));
        }
        // (the eight reads of an iteration are in flight together)
        asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
    }
    const uint32_t last = iters > 0 ? x[7][1] : 0u;
    out[(size_t)blockIdx.x * 512 + t] = last;
}

}  // namespace

extern "C" ATTN_PROBE_API int attn_probe_mfma_bf16(const void *ops, float *out, int blocks, int iters,
                                                   hipStream_t stream) {
    if (!ops || !out) return -1;
    if (blocks < 1 || iters < 1) return -2;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, stream, (const u32x4_t *)ops, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" ATTN_PROBE_API int attn_probe_lds_read(unsigned *out, int blocks, int iters, int mode, hipStream_t stream) {
    if (!out) return -1;
    if (blocks < 1 || iters < 1) return -2;
    switch (mode) {
    case 0: hipLaunchKernelGGL(probe_lds_kernel<0>, dim3(blocks), dim3(512), 0, stream, out, iters); break;
    case 1: hipLaunchKernelGGL(probe_lds_kernel<1>, dim3(blocks), dim3(512), 0, stream, out, iters); break;
    case 2: hipLaunchKernelGGL(probe_lds_kernel<2>, dim3(blocks), dim3(512), 0, stream, out, iters); break;
    default: return -3;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
