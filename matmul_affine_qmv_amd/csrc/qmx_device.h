// qmx_device.h -- device-side helpers shared by the gfx950 kernels of libqmx.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmx {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- scalar conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Round a float to bfloat16, to nearest even (NaN stays a quiet NaN).  Both
// results are formed and one is selected, so the conversion takes no branch.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Storage element of dtype DT at p[i], as float.
template <int DT>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
    if constexpr (DT == DT_F32) {
        return static_cast<const float*>(p)[i];
    } else if constexpr (DT == DT_F16) {
        return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    } else {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
}

template <int DT>
__device__ __forceinline__ void store_elem(void* p, size_t i, float v) {
    if constexpr (DT == DT_F32) {
        static_cast<float*>(p)[i] = v;
    } else if constexpr (DT == DT_F16) {
        static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_f16_bits(v);
    } else {
        static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// Low / high 16-bit half of a packed pair of 16-bit storage values, as float.
template <int DT>
__device__ __forceinline__ float half_lo(uint32_t w) {
    return DT == DT_F16 ? f16_bits_to_f32(w & 0xffffu) : __uint_as_float(w << 16);
}
template <int DT>
__device__ __forceinline__ float half_hi(uint32_t w) {
    return DT == DT_F16 ? f16_bits_to_f32(w >> 16) : __uint_as_float(w & 0xffff0000u);
}

// ---------------------------------------------------------------- buffer loads
// Buffer resource over [p, p + bytes) (bytes clamped to 32 bits); the kernels
// keep every offset inside the array, so the range check never trims a load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                             (int)(bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes),
                                             0x00020000);
}

// ---------------------------------------------------------------- code pairs
// The magic exponent bytes above a pair of 16-bit codes (0x43 for bf16: the
// value 128 + q; 0x64 for f16: 1024 + q) as an opaque register value.  With
// the field mask and the magic both constants, the vector ALU (one scalar
// operand and no literal in its three-operand forms) needs a separate and and
// or; with the magic in a register they are one and-or.
template <int DT>
__device__ __forceinline__ uint32_t magic_bytes() {
    uint32_t mb = DT == DT_F16 ? 0x64006400u : 0x43004300u;
    asm volatile("" : "+v"(mb));
    return mb;
}

// ---------------------------------------------------------------- wave reductions
// Sum over all 64 lanes with a fixed butterfly; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace qmx
