// blocks.hip -- llama.cpp-style Q8_0 and Q4_K block matvecs (M = 1) on gfx950.
//
// Formats and arithmetic follow page "hanzo-kernel src/quant.rs" (Q8_0
// packed layout: 9 words per 32 weights; Q4_K: 144-byte super-blocks with
// 6-bit sub-block scales and mins).  Both kernels are weight-bandwidth
// bound; each wave owns 4 output rows so every x value it loads is used
// four times, accumulates in float32 and ends with a fixed-order wave
// reduction.
#include "qmx_device.h"
#include "qmx_internal.h"

namespace qmx {

constexpr int BLK_ROWS = 4;

// ---------------------------------------------------------------- Q8_0
// Lane l takes blocks l, l+64, ... of its rows.  A signed byte q is read as
// the unsigned byte q ^ 0x80 = q + 128, and the 128 * sum(x) it adds is taken
// off once per block: sum_i q_i x_i = sum_i (q_i + 128) x_i - 128 sum_i x_i.
__global__ __launch_bounds__(64) void q8_0_kernel(const uint32_t* __restrict__ wb,
                                                  const float* __restrict__ x,
                                                  float* __restrict__ out, int N, int K) {
    const int lane = threadIdx.x;
    const int n0 = blockIdx.x * BLK_ROWS;
    const int nb = K / 32;
    float acc[BLK_ROWS] = {0.f, 0.f, 0.f, 0.f};

    for (int b = lane; b < nb; b += 64) {
        float xv[32];
        const u32x4* xp = reinterpret_cast<const u32x4*>(x + 32 * (size_t)b);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x4 d = xp[i];
            xv[4 * i + 0] = __uint_as_float(d.x);
            xv[4 * i + 1] = __uint_as_float(d.y);
            xv[4 * i + 2] = __uint_as_float(d.z);
            xv[4 * i + 3] = __uint_as_float(d.w);
        }
        float xs = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) xs += xv[i];
#pragma unroll
        for (int r = 0; r < BLK_ROWS; ++r) {
            const int n = min(n0 + r, N - 1);
            const uint32_t* blk = wb + ((size_t)n * nb + b) * 9;
            const float d = f16_bits_to_f32(blk[0] & 0xffffu);
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t wd = blk[1 + j] ^ 0x80808080u;
#pragma unroll
                for (int i = 0; i < 4; ++i) s = fmaf((float)((wd >> (8 * i)) & 0xffu), xv[4 * j + i], s);
            }
            acc[r] = fmaf(d, fmaf(-128.f, xs, s), acc[r]);
        }
    }

    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < BLK_ROWS; ++r) {
        const float t = wave_sum(acc[r]);
        if (lane == r) mine = t;
    }
    if (lane < BLK_ROWS && n0 + lane < N) out[n0 + lane] = mine;
}

// ---------------------------------------------------------------- Q4_K
// Eight lanes share a super-block: lane part j (0..7) reads quant bytes
// [16j, 16j+16), i.e. g = j/2 and i in [16(j%2), 16(j%2)+16): low nibbles
// are elements 64g+i of sub-block 2g, high nibbles elements 64g+32+i of
// sub-block 2g+1.  Per sub-block part the sum of q*x and the sum of x are
// formed once; the weight d*sc*q - dmin*m is applied as
// d*sc*sum(q x) - dmin*m*sum(x).
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j,
                                              uint32_t& sc, uint32_t& mn) {
    // s0, s1, s2: scale bytes 0-3, 4-7, 8-11.
    const int jj = j & 3;
    const uint32_t lo_sc = (s0 >> (8 * jj)) & 63u;
    const uint32_t lo_mn = (s1 >> (8 * jj)) & 63u;
    const uint32_t hi_sc = ((s2 >> (8 * jj)) & 15u) | (((s0 >> (8 * jj + 6)) & 3u) << 4);
    const uint32_t hi_mn = ((s2 >> (8 * jj + 4)) & 15u) | (((s1 >> (8 * jj + 6)) & 3u) << 4);
    sc = j < 4 ? lo_sc : hi_sc;
    mn = j < 4 ? lo_mn : hi_mn;
}

__global__ __launch_bounds__(64) void q4_k_kernel(const uint32_t* __restrict__ wb,
                                                  const float* __restrict__ x,
                                                  float* __restrict__ out, int N, int K) {
    const int lane = threadIdx.x;
    const int slot = lane >> 3, part = lane & 7;
    const int g = part >> 1, t0 = (part & 1) * 16;
    const int n0 = blockIdx.x * BLK_ROWS;
    const int nb = K / 256;
    float acc[BLK_ROWS] = {0.f, 0.f, 0.f, 0.f};

    for (int b = slot; b < nb; b += 8) {
        float xl[16], xh[16];
        const float* xb = x + 256 * (size_t)b + 64 * g + t0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 dl = reinterpret_cast<const u32x4*>(xb)[i];
            const u32x4 dh = reinterpret_cast<const u32x4*>(xb + 32)[i];
            xl[4 * i + 0] = __uint_as_float(dl.x); xl[4 * i + 1] = __uint_as_float(dl.y);
            xl[4 * i + 2] = __uint_as_float(dl.z); xl[4 * i + 3] = __uint_as_float(dl.w);
            xh[4 * i + 0] = __uint_as_float(dh.x); xh[4 * i + 1] = __uint_as_float(dh.y);
            xh[4 * i + 2] = __uint_as_float(dh.z); xh[4 * i + 3] = __uint_as_float(dh.w);
        }
        float xsl = 0.f, xsh = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) { xsl += xl[i]; xsh += xh[i]; }

#pragma unroll
        for (int r = 0; r < BLK_ROWS; ++r) {
            const int n = min(n0 + r, N - 1);
            const uint32_t* blk = wb + ((size_t)n * nb + b) * 36;
            const u32x4 hdr = *reinterpret_cast<const u32x4*>(blk);
            const u32x4 qw = *reinterpret_cast<const u32x4*>(blk + 4 + 4 * part);
            const float d = f16_bits_to_f32(hdr.x & 0xffffu);
            const float dmin = f16_bits_to_f32(hdr.x >> 16);
            uint32_t sc_lo, mn_lo, sc_hi, mn_hi;
            q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * g, sc_lo, mn_lo);
            q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * g + 1, sc_hi, mn_hi);
            float sl = 0.f, sh = 0.f;
            const uint32_t qws[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = qws[k] & 0x0f0f0f0fu, hi = (qws[k] >> 4) & 0x0f0f0f0fu;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sl = fmaf((float)((lo >> (8 * i)) & 0xffu), xl[4 * k + i], sl);
                    sh = fmaf((float)((hi >> (8 * i)) & 0xffu), xh[4 * k + i], sh);
                }
            }
            const float qpart = fmaf((float)sc_lo, sl, (float)sc_hi * sh);
            const float mpart = fmaf((float)mn_lo, xsl, (float)mn_hi * xsh);
            acc[r] = fmaf(d, qpart, fmaf(-dmin, mpart, acc[r]));
        }
    }

    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < BLK_ROWS; ++r) {
        const float t = wave_sum(acc[r]);
        if (lane == r) mine = t;
    }
    if (lane < BLK_ROWS && n0 + lane < N) out[n0 + lane] = mine;
}

hipError_t launch_q8_0(const uint32_t* w, const float* x, float* out, int N, int K, hipStream_t st) {
    const dim3 grid((N + BLK_ROWS - 1) / BLK_ROWS);
    hipLaunchKernelGGL(q8_0_kernel, grid, dim3(64), 0, st, w, x, out, N, K);
    return hipGetLastError();
}

hipError_t launch_q4_k(const uint32_t* w, const float* x, float* out, int N, int K, hipStream_t st) {
    const dim3 grid((N + BLK_ROWS - 1) / BLK_ROWS);
    hipLaunchKernelGGL(q4_k_kernel, grid, dim3(64), 0, st, w, x, out, N, K);
    return hipGetLastError();
}

}  // namespace qmx
