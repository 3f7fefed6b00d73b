// qmv.hip -- group-wise affine quantized matvec (small M) on the gfx950 vector ALUs.
//
// Method (page "metaltile-std src/mlx/quantized.rs", qmv kernel): per group
// g of row n, out += scale[n,g] * sum q*x + bias[n,g] * sum x, with the sum
// of x formed once per group part and shared by every row (bias hoist), x
// held in registers and reused across the rows a wave owns, float32
// accumulators, and a cross-lane reduction followed by one store per output.
//
// gfx950 mapping: one wave64 per work-group owns QMV_ROWS consecutive rows
// of W and up to MT rows of x.  A row of W is cut into 16-byte chunks; lane
// l takes chunks l, l+64, ... so every wave-wide load is 1 KB of one row,
// contiguous.  Small single-wave work-groups keep the per-CU load even when
// N/QMV_ROWS is not a multiple of the CU count.  The final reduction is a
// fixed xor-butterfly, so results do not change from run to run.
#include "qmx_device.h"
#include "qmx_internal.h"

namespace qmx {

// Expand one packed word into its 32/BITS codes (element order), as float.
template <int BITS>
__device__ __forceinline__ void unpack_word(uint32_t w, float (&q)[32 / BITS]) {
    if constexpr (BITS == 4) {
        const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q[2 * i] = (float)((lo >> (8 * i)) & 0xffu);
            q[2 * i + 1] = (float)((hi >> (8 * i)) & 0xffu);
        }
    } else if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (float)((w >> (8 * i)) & 0xffu);
    } else {
        static_assert(BITS == 2, "bits");
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t f = (w >> (2 * t)) & 0x03030303u;
#pragma unroll
            for (int i = 0; i < 4; ++i) q[4 * i + t] = (float)((f >> (8 * i)) & 0xffu);
        }
    }
}

// The N values of x starting at element index `idx` (idx*sizeof aligned to
// 16 bytes for f32 / 8 bytes for 16-bit types), as float.
template <int DT, int N>
__device__ __forceinline__ void load_x(const void* x, size_t idx, float (&v)[N]) {
    if constexpr (DT == DT_F32) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + idx);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const u32x4 d = p[i];
            v[4 * i + 0] = __uint_as_float(d.x);
            v[4 * i + 1] = __uint_as_float(d.y);
            v[4 * i + 2] = __uint_as_float(d.z);
            v[4 * i + 3] = __uint_as_float(d.w);
        }
    } else if constexpr (N % 8 == 0) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + idx);
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            const u32x4 d = p[i];
            const uint32_t ws[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = half_lo<DT>(ws[j]);
                v[8 * i + 2 * j + 1] = half_hi<DT>(ws[j]);
            }
        }
    } else {
        static_assert(N == 4, "x word width");
        const u32x2 d = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(x) + idx);
        v[0] = half_lo<DT>(d.x);
        v[1] = half_hi<DT>(d.x);
        v[2] = half_lo<DT>(d.y);
        v[3] = half_hi<DT>(d.y);
    }
}

template <int DT, int BITS, int GS, int MT>
__global__ __launch_bounds__(64) void qmv_kernel(const uint32_t* __restrict__ w,
                                                 const void* __restrict__ scales,
                                                 const void* __restrict__ biases,
                                                 const void* __restrict__ x,
                                                 void* __restrict__ out, int M, int N, int K) {
    constexpr int R = QMV_ROWS;
    constexpr int CPW = 32 / BITS;                 // codes per word
    constexpr int CPC = 4 * CPW;                   // codes per 16-byte chunk
    constexpr int PARTS = CPC > GS ? CPC / GS : 1; // groups touched by one chunk
    constexpr int WPP = 4 / PARTS;                 // words per group part

    const int lane = threadIdx.x;
    const int n0 = blockIdx.x * R;
    const int m0 = blockIdx.y * MT;
    const int mcount = min(MT, M - m0);
    const int G = K / GS;
    const int chunks = K / CPC;
    const size_t row_words = (size_t)(K / CPW);

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

    for (int c = lane; c < chunks; c += 64) {
        u32x4 wv[R];
        float sv[R][PARTS], bv[R][PARTS];
        const int g0 = (c * CPC) / GS;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(n0 + r, N - 1);      // rows past N compute garbage that is never stored
            wv[r] = *reinterpret_cast<const u32x4*>(w + (size_t)n * row_words + 4 * (size_t)c);
#pragma unroll
            for (int p = 0; p < PARTS; ++p) {
                const size_t gi = (size_t)n * G + g0 + p;
                sv[r][p] = load_elem<DT>(scales, gi);
                bv[r][p] = load_elem<DT>(biases, gi);
            }
        }

        float qd[R][MT][PARTS];
        float xs[MT][PARTS];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int p = 0; p < PARTS; ++p) {
                xs[m][p] = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) qd[r][m][p] = 0.f;
            }

#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = j / WPP;
            float xv[MT][CPW];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mcount) {
                    load_x<DT, CPW>(x, (size_t)(m0 + m) * K + (size_t)c * CPC + j * CPW, xv[m]);
                } else {
#pragma unroll
                    for (int e = 0; e < CPW; ++e) xv[m][e] = 0.f;
                }
                float t = 0.f;
#pragma unroll
                for (int e = 0; e < CPW; ++e) t += xv[m][e];
                xs[m][p] += t;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t word = j == 0 ? wv[r].x : j == 1 ? wv[r].y : j == 2 ? wv[r].z : wv[r].w;
                float q[CPW];
                unpack_word<BITS>(word, q);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float t = qd[r][m][p];
#pragma unroll
                    for (int e = 0; e < CPW; ++e) t = fmaf(q[e], xv[m][e], t);
                    qd[r][m][p] = t;
                }
            }
        }

#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int p = 0; p < PARTS; ++p)
                    acc[r][m] = fmaf(sv[r][p], qd[r][m][p], fmaf(bv[r][p], xs[m][p], acc[r][m]));
    }

    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float tot = wave_sum(acc[r][m]);
            if (lane == r * MT + m) mine = tot;
        }
    if (lane < R * MT) {
        const int r = lane / MT, m = lane % MT;
        if (n0 + r < N && m < mcount) store_elem<DT>(out, (size_t)(m0 + m) * N + n0 + r, mine);
    }
}

int qmv_mt_for(int M) { return M >= 4 ? 4 : (M == 3 ? 4 : (M == 2 ? 2 : 1)); }

template <int DT, int BITS, int GS>
static hipError_t qmv_mt(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                         int M, int N, int K, hipStream_t st) {
    const int mt = qmv_mt_for(M);
    const dim3 grid((N + QMV_ROWS - 1) / QMV_ROWS, (M + mt - 1) / mt);
    if (mt == 1)
        hipLaunchKernelGGL((qmv_kernel<DT, BITS, GS, 1>), grid, dim3(64), 0, st, w, s, b, x, out, M, N, K);
    else if (mt == 2)
        hipLaunchKernelGGL((qmv_kernel<DT, BITS, GS, 2>), grid, dim3(64), 0, st, w, s, b, x, out, M, N, K);
    else
        hipLaunchKernelGGL((qmv_kernel<DT, BITS, GS, 4>), grid, dim3(64), 0, st, w, s, b, x, out, M, N, K);
    return hipGetLastError();
}

template <int DT, int BITS>
static hipError_t qmv_gs(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                         int M, int N, int K, int gs, hipStream_t st) {
    switch (gs) {
        case 32: return qmv_mt<DT, BITS, 32>(w, s, b, x, out, M, N, K, st);
        case 64: return qmv_mt<DT, BITS, 64>(w, s, b, x, out, M, N, K, st);
        default: return qmv_mt<DT, BITS, 128>(w, s, b, x, out, M, N, K, st);
    }
}

template <int DT>
static hipError_t qmv_bits(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                           int M, int N, int K, int bits, int gs, hipStream_t st) {
    switch (bits) {
        case 2: return qmv_gs<DT, 2>(w, s, b, x, out, M, N, K, gs, st);
        case 4: return qmv_gs<DT, 4>(w, s, b, x, out, M, N, K, gs, st);
        default: return qmv_gs<DT, 8>(w, s, b, x, out, M, N, K, gs, st);
    }
}

hipError_t launch_qmv(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                      int M, int N, int K, int bits, int gs, int dt, hipStream_t st) {
    switch (dt) {
        case DT_F32: return qmv_bits<DT_F32>(w, s, b, x, out, M, N, K, bits, gs, st);
        case DT_F16: return qmv_bits<DT_F16>(w, s, b, x, out, M, N, K, bits, gs, st);
        default: return qmv_bits<DT_BF16>(w, s, b, x, out, M, N, K, bits, gs, st);
    }
}

}  // namespace qmx
