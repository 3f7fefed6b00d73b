// calib.hip -- calibration kernels for the measurements beside the library:
// what one MI355X actually reaches for a plain streaming read, a streaming
// copy and back-to-back bf16 matrix-core instructions, and the cost of an
// empty launch.  They hold none of the quantized method and are built into a
// separate library (libqmx_calib.so, include/qmx_calib.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmx_calib.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Grid-stride read of n16 16-byte chunks, sixteen loads in flight per thread
// (measured: four in flight stay near 4.9 TB/s at 512 MiB, sixteen reach 6).
// The xor of everything read is stored only when it equals a value the
// caller passes and no input contains, so the loads cannot be dropped.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink, uint32_t never) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 15 * stride < n16; i += 16 * stride) {
        u32x4 v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = src[i + j * stride];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc ^= v[j];
    }
    for (; i < n16; i += stride) acc ^= src[i];
    const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (v == never) sink[0] = v;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n16) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

// Eight independent accumulation chains of v_mfma_f32_16x16x32_bf16 per
// wave, `iters` rounds; each wave stores its chain sums so that none is dead.
__global__ __launch_bounds__(256) void mfma16_kernel(float* __restrict__ out, int iters) {
    const uint32_t l = threadIdx.x;
    u32x4 ai = {0x3f803f80u ^ (l & 1u), 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    u32x4 bi = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u ^ (l & 2u)};
    const bf16x8 a = __builtin_bit_cast(bf16x8, ai), b = __builtin_bit_cast(bf16x8, bi);
    f32x4 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
    f32x4 s = c[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) s += c[j];
    out[(size_t)blockIdx.x * 256 + l] = s.x + s.y + s.z + s.w;
}

// Four independent chains of v_mfma_f32_32x32x16_bf16 (32768 flops each).
__global__ __launch_bounds__(256) void mfma32_kernel(float* __restrict__ out, int iters) {
    const uint32_t l = threadIdx.x;
    u32x4 ai = {0x3f803f80u ^ (l & 1u), 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const bf16x8 a = __builtin_bit_cast(bf16x8, ai);
    f32x16 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    out[(size_t)blockIdx.x * 256 + l] = s;
}

// Co-issue of the matrix core and the vector ALU: four independent chains of
// v_mfma_f32_32x32x16_bf16, each instruction followed by F independent
// v_fmac_f32 (16 chains, an SGPR multiplier, no literal), `iters` rounds.
template <int F>
__global__ __launch_bounds__(256) void mfma_valu_kernel(float* __restrict__ out, int iters, float m) {
    const uint32_t l = threadIdx.x;
    u32x4 ai = {0x3f803f80u ^ (l & 1u), 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const bf16x8 a = __builtin_bit_cast(bf16x8, ai);
    f32x16 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
    float f[16], g[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        f[j] = (float)(l + j) * 1e-3f;
        g[j] = (float)(l ^ j) * 1e-4f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c[q], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < F; ++j) f[(q * F + j) % 16] = fmaf(m, g[(q * F + j) % 16], f[(q * F + j) % 16]);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += f[j];
    out[(size_t)blockIdx.x * 256 + l] = s;
}

// The same F float FMAs per round without the matrix instructions.
template <int F>
__global__ __launch_bounds__(256) void valu_kernel(float* __restrict__ out, int iters, float m) {
    const uint32_t l = threadIdx.x;
    float f[16], g[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        f[j] = (float)(l + j) * 1e-3f;
        g[j] = (float)(l ^ j) * 1e-4f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < F; ++j) f[(q * F + j) % 16] = fmaf(m, g[(q * F + j) % 16], f[(q * F + j) % 16]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += f[j];
    out[(size_t)blockIdx.x * 256 + l] = s;
}

template <int F>
int mfma_valu_go(float* out, int iters, int blocks, int with_mfma, hipStream_t st) {
    if (with_mfma)
        hipLaunchKernelGGL(mfma_valu_kernel<F>, dim3(blocks), dim3(256), 0, st, out, iters, 0.999f);
    else
        hipLaunchKernelGGL(valu_kernel<F>, dim3(blocks), dim3(256), 0, st, out, iters, 0.999f);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void empty_kernel() {}

int status(hipError_t e) { return e == hipSuccess ? 0 : -1; }

}  // namespace

extern "C" {

int qmxc_read(const void* src, size_t bytes, uint32_t* sink, uint32_t never, int blocks, void* stream) {
    if (!src || !sink || bytes % 16 != 0 || blocks <= 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, sink, never);
    return status(hipGetLastError());
}

int qmxc_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
    if (!src || !dst || bytes % 16 != 0 || blocks <= 0 ||
        ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
        return -1;
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return status(hipGetLastError());
}

int qmxc_mfma(float* out, int iters, int blocks, int shape, void* stream) {
    if (!out || iters < 0 || blocks <= 0 || (shape != 16 && shape != 32)) return -1;
    if (shape == 16)
        hipLaunchKernelGGL(mfma16_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    else
        hipLaunchKernelGGL(mfma32_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    return status(hipGetLastError());
}

int qmxc_mfma_valu(float* out, int iters, int blocks, int fmas, int with_mfma, void* stream) {
    if (!out || iters < 0 || blocks <= 0) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (fmas) {
        case 0: return mfma_valu_go<0>(out, iters, blocks, with_mfma, st);
        case 2: return mfma_valu_go<2>(out, iters, blocks, with_mfma, st);
        case 4: return mfma_valu_go<4>(out, iters, blocks, with_mfma, st);
        case 6: return mfma_valu_go<6>(out, iters, blocks, with_mfma, st);
        case 8: return mfma_valu_go<8>(out, iters, blocks, with_mfma, st);
        case 10: return mfma_valu_go<10>(out, iters, blocks, with_mfma, st);
        case 12: return mfma_valu_go<12>(out, iters, blocks, with_mfma, st);
        case 16: return mfma_valu_go<16>(out, iters, blocks, with_mfma, st);
        default: return -1;
    }
}

int qmxc_empty(int blocks, void* stream) {
    if (blocks <= 0) return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(64), 0, static_cast<hipStream_t>(stream));
    return status(hipGetLastError());
}

}  // extern "C"
