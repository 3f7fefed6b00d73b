// q8_i8.hip -- integer-activation matvec: int8 weights times int8 activations
// with one float32 scale per 32-element block of a weight row.
//
// Method (page "hanzo-kernel src/quant.rs", packed-int8 dp4a matvec and its
// block-per-row form): both operands are packed four int8 to a word, each
// group of four is one hardware 4-way integer dot, a block's integer sum is
// exact, and out[n] = sum_b wd[n,b] * dot_b is accumulated in float32.
//
// gfx950 mapping: a wave owns 2 rows and lane l takes blocks l, l + 64, ... of
// them, so a load instruction reads 2 KB contiguous per row; the block's 32
// activations are loaded once per lane and used by both rows.  A wave keeps
// one round of loads in flight, so many small waves (8 per SIMD, the whole
// grid resident at once) hide the round trips better than fewer wide ones.  Each block is
// eight v_dot4_i32_i8 into an int32 (|sum| <= 32 * 128 * 128), then one float32
// fma with the row's block scale.  All loads are buffer loads whose per-round
// advance is a scalar offset.  The rows' sums end in the fixed xor butterfly,
// so results do not change from run to run.
#include "qmx_device.h"
#include "qmx_internal.h"

namespace qmx {

constexpr int I8_ROWS = 2;     // rows per wave
constexpr int I8_WAVES = 4;    // waves per work-group

__device__ __forceinline__ int dot8x4(const u32x4& a, const u32x4& b, int c) {
    c = __builtin_amdgcn_sdot4((int)a.x, (int)b.x, c, false);
    c = __builtin_amdgcn_sdot4((int)a.y, (int)b.y, c, false);
    c = __builtin_amdgcn_sdot4((int)a.z, (int)b.z, c, false);
    return __builtin_amdgcn_sdot4((int)a.w, (int)b.w, c, false);
}

__global__ __launch_bounds__(64 * I8_WAVES) void q8_i8_kernel(const uint32_t* __restrict__ wq,
                                                             const uint32_t* __restrict__ xq,
                                                             const float* __restrict__ wd,
                                                             float* __restrict__ out, int N, int K) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = (blockIdx.x * I8_WAVES + wave) * I8_ROWS;
    if (n0 >= N) return;
    const int nb = K / 32;
    // rows past N repeat row N - 1 and are not stored
    const __amdgpu_buffer_rsrc_t rw = buffer_over(reinterpret_cast<const unsigned char*>(wq) + (size_t)n0 * K,
                                                  (size_t)(N - n0) * K);
    const __amdgpu_buffer_rsrc_t rx = buffer_over(xq, (size_t)K);
    const __amdgpu_buffer_rsrc_t rd = buffer_over(wd + (size_t)n0 * nb, (size_t)(N - n0) * nb * 4);
    int vw[I8_ROWS], vd[I8_ROWS];
#pragma unroll
    for (int r = 0; r < I8_ROWS; ++r) {
        const int rr = min(n0 + r, N - 1) - n0;
        vw[r] = rr * K + 32 * lane;
        vd[r] = (rr * nb + lane) * 4;
    }
    const int vx = 32 * lane;
    float acc[I8_ROWS] = {};
    for (int c = lane, round = 0; c < nb; c += 64, ++round) {
        const int sw = round * 64 * 32, sd = round * 64 * 4;
        const u32x4 x0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, vx, sw, 0));
        const u32x4 x1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, vx + 16, sw, 0));
        u32x4 w0[I8_ROWS], w1[I8_ROWS];
        float d[I8_ROWS];
#pragma unroll
        for (int r = 0; r < I8_ROWS; ++r) {
            w0[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw[r], sw, 0));
            w1[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw[r] + 16, sw, 0));
        }
#pragma unroll
        for (int r = 0; r < I8_ROWS; ++r)
            d[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, vd[r], sd, 0));
#pragma unroll
        for (int r = 0; r < I8_ROWS; ++r) acc[r] = fmaf(d[r], (float)dot8x4(w1[r], x1, dot8x4(w0[r], x0, 0)), acc[r]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int r = 0; r < I8_ROWS; ++r) acc[r] += __shfl_xor(acc[r], off, 64);
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < I8_ROWS; ++r)
        if (lane == r) mine = acc[r];
    if (lane < I8_ROWS && n0 + lane < N) out[n0 + lane] = mine;
}

hipError_t launch_q8_i8(const uint32_t* wq, const uint32_t* xq, const float* wd, float* out, int N, int K,
                        hipStream_t st) {
    const int rows_per_group = I8_ROWS * I8_WAVES;
    const dim3 grid((N + rows_per_group - 1) / rows_per_group);
    hipLaunchKernelGGL(q8_i8_kernel, grid, dim3(64 * I8_WAVES), 0, st, wq, xq, wd, out, N, K);
    return hipGetLastError();
}

}  // namespace qmx
