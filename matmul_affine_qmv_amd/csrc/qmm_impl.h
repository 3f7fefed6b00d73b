// qmm_impl.h -- the staged affine quantized x * W^T kernel for M >= 8 on the
// gfx950 matrix cores.  Included once per code width by qmm_b{2,4,8}.hip.
//
// Method (page "mlx PR 4682"): transposed affine qmm with the next K step's
// packed weights, scales/biases and activations prefetched into registers
// while the current step is consumed from a threadgroup-memory buffer, the
// prefetched step written into the other buffer, and one barrier per K step;
// split-K writes float32 partials that a separate kernel sums.
//
// gfx950 mapping:
// * A work-group of 4 waves owns an output tile of BM = 16*MT rows of x by
//   BN = 128 columns of W (each wave 2 fragments of 16 columns) and a range
//   of 128-column K blocks.  LDS holds two buffers of: the x block (BM x 128,
//   16-bit), the packed W block (128 rows x 128 codes), per-row group sums
//   of x and the block's scales/biases converted to float32.
// * Codes stay packed in LDS and are expanded in registers right before the
//   MFMA into exact 16-bit integers: (field | 0x4300) is the bf16 value
//   128 + q and (field | 0x6400) the f16 value 1024 + q, so each pair of
//   codes costs one and/or.  The constant offset OFF*sum(x) this adds is
//   removed in the group epilogue.  The codes of a word come out in the
//   order 0,4,1,5,2,6,3,7 (8-bit: 0,2,1,3); x is written to LDS in the same
//   order, and since both MFMA operands see the same permutation of k the
//   dot product is unchanged.
// * MFMA v_mfma_f32_16x16x32_{bf16,f16}: A = x fragment (16 rows of M),
//   B = W codes (16 columns of N).  A group of GS codes is GS/32 MFMA k-steps
//   accumulated into a fresh float32 tile; the epilogue then adds
//   scale * (tile) + (bias - OFF*scale) * sum(x) in float32.  Scale and bias
//   never pass through a 16-bit format, so the output's only roundings are
//   float32 accumulation and the final store.
// * Work-groups are numbered so that the ones sharing a K range (and so the
//   same x slice) are dispatched to the same XCD and share its L2.
#pragma once

#include "qmx_device.h"
#include "qmx_internal.h"

namespace qmx {

template <int DT, int BITS, int GS, int MT>
struct QmmCfg {
    static constexpr int BM = 16 * MT;
    static constexpr int GPB = QMM_KB / GS;                  // groups per K block
    static constexpr int S = GS / 4;                         // codes per lane group per group
    static constexpr int KS = GS / 32;                       // MFMA k-steps per group
    static constexpr int XP = QMM_KB + 8;                    // x LDS row pitch (elements)
    static constexpr int WROW = QMM_KB * BITS / 32;          // words per W row per block
    static constexpr int WP = WROW + 4;                      // W LDS row pitch (words)
    static constexpr int WPL = (S * BITS / 32) > 0 ? (S * BITS / 32) : 1;  // words per lane per group
    static constexpr int X_BYTES = BM * XP * 2;
    static constexpr int W_BYTES = QMM_BN * WP * 4;
    static constexpr int XS_BYTES = GPB * BM * 4;
    static constexpr int SB_BYTES = 2 * GPB * QMM_BN * 4;
    static constexpr int BUF_BYTES = X_BYTES + W_BYTES + XS_BYTES + SB_BYTES;
    static constexpr int W_PIECES = BITS / 2;                // 16-byte W pieces per thread per block
    static constexpr int SB_PER_THREAD = GPB >= 2 ? GPB / 2 : 1;
    static constexpr uint32_t MAGIC = DT == DT_F16 ? 0x64006400u : 0x43004300u;
    static constexpr float OFF = (DT == DT_F16) ? 1024.f : (BITS == 8 ? 0.f : 128.f);
    static_assert(BUF_BYTES % 16 == 0, "buffer alignment");
    static_assert(2 * BUF_BYTES <= 160 * 1024, "LDS budget");
};

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 8 codes of one unit as 16-bit MFMA operands.  4-bit: one word, pairs
// (i, i+4).  2-bit: 16 bits v, spread so codes 4..7 land in the high half.
// 8-bit: two words, pairs (0,2), (1,3), (4,6), (5,7).
template <int DT, int BITS>
__device__ __forceinline__ u32x4 unpack_unit(uint32_t w0, uint32_t w1) {
    constexpr uint32_t MAGIC = DT == DT_F16 ? 0x64006400u : 0x43004300u;
    u32x4 r;
    if constexpr (BITS == 4) {
        r.x = (w0 & 0x000f000fu) | MAGIC;
        r.y = ((w0 >> 4) & 0x000f000fu) | MAGIC;
        r.z = ((w0 >> 8) & 0x000f000fu) | MAGIC;
        r.w = ((w0 >> 12) & 0x000f000fu) | MAGIC;
    } else if constexpr (BITS == 2) {
        const uint32_t t = w0 | (w0 << 8);   // w0 holds the unit in its low 16 bits
        r.x = (t & 0x00030003u) | MAGIC;
        r.y = ((t >> 2) & 0x00030003u) | MAGIC;
        r.z = ((t >> 4) & 0x00030003u) | MAGIC;
        r.w = ((t >> 6) & 0x00030003u) | MAGIC;
    } else if constexpr (DT == DT_F16) {
        r.x = (w0 & 0x00ff00ffu) | MAGIC;
        r.y = ((w0 >> 8) & 0x00ff00ffu) | MAGIC;
        r.z = (w1 & 0x00ff00ffu) | MAGIC;
        r.w = ((w1 >> 8) & 0x00ff00ffu) | MAGIC;
    } else {
        // bf16 holds every integer up to 256 exactly: convert, keep the upper half.
        auto pair = [](uint32_t a, uint32_t b) {
            return (__float_as_uint((float)a) >> 16) | (__float_as_uint((float)b) & 0xffff0000u);
        };
        r.x = pair(w0 & 0xffu, (w0 >> 16) & 0xffu);
        r.y = pair((w0 >> 8) & 0xffu, w0 >> 24);
        r.z = pair(w1 & 0xffu, (w1 >> 16) & 0xffu);
        r.w = pair((w1 >> 8) & 0xffu, w1 >> 24);
    }
    return r;
}

// Eight consecutive x values (d = x0x1, x2x3, x4x5, x6x7) in the unit order
// used by unpack_unit.
template <int BITS>
__device__ __forceinline__ u32x4 permute_x(u32x4 d) {
    u32x4 r;
    if constexpr (BITS == 8) {
        r.x = (d.x & 0xffffu) | (d.y << 16);
        r.y = (d.x >> 16) | (d.y & 0xffff0000u);
        r.z = (d.z & 0xffffu) | (d.w << 16);
        r.w = (d.z >> 16) | (d.w & 0xffff0000u);
    } else {
        r.x = (d.x & 0xffffu) | (d.z << 16);
        r.y = (d.x >> 16) | (d.z & 0xffff0000u);
        r.z = (d.y & 0xffffu) | (d.w << 16);
        r.w = (d.y >> 16) | (d.w & 0xffff0000u);
    }
    return r;
}

template <int DT>
__device__ __forceinline__ float sum8(u32x4 d) {
    float t = half_lo<DT>(d.x) + half_hi<DT>(d.x);
    t += half_lo<DT>(d.y) + half_hi<DT>(d.y);
    t += half_lo<DT>(d.z) + half_hi<DT>(d.z);
    t += half_lo<DT>(d.w) + half_hi<DT>(d.w);
    return t;
}

template <int DT, int BITS, int GS, int MT, bool SPLIT>
__global__ __launch_bounds__(QMM_THREADS) void qmm_t_kernel(
    const uint32_t* __restrict__ w, const void* __restrict__ scales, const void* __restrict__ biases,
    const void* __restrict__ x, void* __restrict__ out, float* __restrict__ ws,
    int M, int N, int K, int splits, int ntiles, int mtiles, int total_tiles, int per_xcd) {
    using C = QmmCfg<DT, BITS, GS, MT>;
    constexpr int NB = QMM_NB;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::BUF_BYTES];

    // Hardware block h runs on XCD h % 8; give each XCD a contiguous range of tiles.
    const int h = blockIdx.x;
    const int L = (h & 7) * per_xcd + (h >> 3);
    if (L >= total_tiles) return;
    const int ntile = L % ntiles;
    const int rest = L / ntiles;
    const int mtile = rest % mtiles;
    const int split = rest / mtiles;
    const int n0 = ntile * QMM_BN, m0 = mtile * C::BM;
    const int nkb = K / QMM_KB;
    const int kb0 = (int)((long)split * nkb / splits);
    const int kb1 = (int)((long)(split + 1) * nkb / splits);
    const int G = K / GS;
    const size_t row_words = (size_t)K * BITS / 32;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;

    u32x4 xr[MT];
    u32x4 wr[C::W_PIECES];
    float sr[C::SB_PER_THREAD], br[C::SB_PER_THREAD];
    const int sb_col = tid & 127;
    const int sb_g0 = (tid >> 7) * C::SB_PER_THREAD;
    const bool sb_active = sb_g0 < C::GPB;

    auto gload = [&](int kb) {
        const int k0 = kb * QMM_KB;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int m = m0 + (tid >> 4) + 16 * i;
            if (m < M)
                xr[i] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + (size_t)m * K +
                                                        k0 + 8 * (tid & 15));
            else
                xr[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < C::W_PIECES; ++i) {
            const int p = tid + QMM_THREADS * i;
            const int n = n0 + p / BITS;
            if (n < N)
                wr[i] = *reinterpret_cast<const u32x4*>(w + (size_t)n * row_words + (size_t)kb * C::WROW +
                                                        4 * (p % BITS));
            else
                wr[i] = u32x4{0u, 0u, 0u, 0u};
        }
        const int n = n0 + sb_col;
#pragma unroll
        for (int j = 0; j < C::SB_PER_THREAD; ++j) {
            if (sb_active && n < N) {
                const size_t gi = (size_t)n * G + (size_t)kb * C::GPB + sb_g0 + j;
                sr[j] = load_elem<DT>(scales, gi);
                br[j] = load_elem<DT>(biases, gi);
            } else {
                sr[j] = 0.f;
                br[j] = 0.f;
            }
        }
    };

    auto lstore = [&](int buf) {
        unsigned char* base = smem + buf * C::BUF_BYTES;
        uint16_t* xl = reinterpret_cast<uint16_t*>(base);
        uint32_t* wl = reinterpret_cast<uint32_t*>(base + C::X_BYTES);
        float* xsl = reinterpret_cast<float*>(base + C::X_BYTES + C::W_BYTES);
        float* sbl = reinterpret_cast<float*>(base + C::X_BYTES + C::W_BYTES + C::XS_BYTES);
        const int u = tid & 15;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int row = (tid >> 4) + 16 * i;
            *reinterpret_cast<u32x4*>(xl + row * C::XP + 8 * u) = permute_x<BITS>(xr[i]);
            float t = sum8<DT>(xr[i]);
#pragma unroll
            for (int off = 1; off < GS / 8; off <<= 1) t += __shfl_xor(t, off, 64);
            if ((u % (GS / 8)) == 0) xsl[(u / (GS / 8)) * C::BM + row] = t;
        }
#pragma unroll
        for (int i = 0; i < C::W_PIECES; ++i) {
            const int p = tid + QMM_THREADS * i;
            *reinterpret_cast<u32x4*>(wl + (p / BITS) * C::WP + 4 * (p % BITS)) = wr[i];
        }
        if (sb_active) {
#pragma unroll
            for (int j = 0; j < C::SB_PER_THREAD; ++j) {
                sbl[(sb_g0 + j) * QMM_BN + sb_col] = sr[j];
                sbl[(C::GPB + sb_g0 + j) * QMM_BN + sb_col] = fmaf(-C::OFF, sr[j], br[j]);
            }
        }
    };

    f32x4 run[MT][NB];
#pragma unroll
    for (int mf = 0; mf < MT; ++mf)
#pragma unroll
        for (int nf = 0; nf < NB; ++nf) run[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const unsigned char* base = smem + buf * C::BUF_BYTES;
        const uint16_t* xl = reinterpret_cast<const uint16_t*>(base);
        const uint32_t* wl = reinterpret_cast<const uint32_t*>(base + C::X_BYTES);
        const float* xsl = reinterpret_cast<const float*>(base + C::X_BYTES + C::W_BYTES);
        const float* sbl = reinterpret_cast<const float*>(base + C::X_BYTES + C::W_BYTES + C::XS_BYTES);
#pragma unroll
        for (int gi = 0; gi < C::GPB; ++gi) {
            uint32_t bw[NB][C::WPL];
#pragma unroll
            for (int nf = 0; nf < NB; ++nf) {
                const int row = wave * (NB * 16) + nf * 16 + lrow;
                int word;
                if constexpr (BITS == 2 && GS == 32) word = gi * 2 + (lgrp >> 1);
                else word = (gi * GS + lgrp * C::S) * BITS / 32;
#pragma unroll
                for (int i = 0; i < C::WPL; ++i) bw[nf][i] = wl[row * C::WP + word + i];
            }
            f32x4 gacc[MT][NB];
#pragma unroll
            for (int mf = 0; mf < MT; ++mf)
#pragma unroll
                for (int nf = 0; nf < NB; ++nf) gacc[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < C::KS; ++t) {
                u32x4 bf[NB];
#pragma unroll
                for (int nf = 0; nf < NB; ++nf) {
                    if constexpr (BITS == 4) {
                        bf[nf] = unpack_unit<DT, 4>(bw[nf][t], 0u);
                    } else if constexpr (BITS == 8) {
                        bf[nf] = unpack_unit<DT, 8>(bw[nf][2 * t], bw[nf][2 * t + 1]);
                    } else {
                        const int half = (GS == 32) ? (lgrp & 1) : (t & 1);
                        const uint32_t wd = (GS == 32) ? bw[nf][0] : bw[nf][t >> 1];
                        bf[nf] = unpack_unit<DT, 2>((wd >> (16 * half)) & 0xffffu, 0u);
                    }
                }
#pragma unroll
                for (int mf = 0; mf < MT; ++mf) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(
                        xl + (mf * 16 + lrow) * C::XP + gi * GS + lgrp * C::S + 8 * t);
#pragma unroll
                    for (int nf = 0; nf < NB; ++nf) gacc[mf][nf] = mfma16x16x32<DT>(a, bf[nf], gacc[mf][nf]);
                }
            }
            float sv[NB], bv[NB];
#pragma unroll
            for (int nf = 0; nf < NB; ++nf) {
                const int col = wave * (NB * 16) + nf * 16 + lrow;
                sv[nf] = sbl[gi * QMM_BN + col];
                bv[nf] = sbl[(C::GPB + gi) * QMM_BN + col];
            }
#pragma unroll
            for (int mf = 0; mf < MT; ++mf) {
                const f32x4 xs4 = *reinterpret_cast<const f32x4*>(xsl + gi * C::BM + mf * 16 + 4 * lgrp);
#pragma unroll
                for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        run[mf][nf][v] = fmaf(sv[nf], gacc[mf][nf][v], fmaf(bv[nf], xs4[v], run[mf][nf][v]));
            }
        }
    };

    if (kb0 < kb1) {
        gload(kb0);
        lstore(0);
        if (kb0 + 1 < kb1) gload(kb0 + 1);
        __syncthreads();
        for (int kb = kb0; kb < kb1; ++kb) {
            const int buf = (kb - kb0) & 1;
            compute(buf);
            if (kb + 1 < kb1) {
                lstore(buf ^ 1);
                if (kb + 2 < kb1) gload(kb + 2);
            }
            __syncthreads();
        }
    }

#pragma unroll
    for (int mf = 0; mf < MT; ++mf)
#pragma unroll
        for (int nf = 0; nf < NB; ++nf)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + mf * 16 + 4 * lgrp + v;
                const int n = n0 + wave * (NB * 16) + nf * 16 + lrow;
                if (m < M && n < N) {
                    if constexpr (SPLIT)
                        ws[((size_t)split * M + m) * N + n] = run[mf][nf][v];
                    else
                        store_elem<DT>(out, (size_t)m * N + n, run[mf][nf][v]);
                }
            }
}

template <int DT, int BITS, int GS, int MT>
hipError_t qmm_launch_mt(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                         float* ws, int M, int N, int K, int splits, hipStream_t st) {
    const int ntiles = (N + QMM_BN - 1) / QMM_BN;
    const int mtiles = qmm_mtiles_for(M);
    const int total = ntiles * mtiles * splits;
    const int per_xcd = (total + 7) / 8;
    const dim3 grid(8 * per_xcd), block(QMM_THREADS);
    if (splits > 1)
        hipLaunchKernelGGL((qmm_t_kernel<DT, BITS, GS, MT, true>), grid, block, 0, st, w, s, b, x, out, ws,
                           M, N, K, splits, ntiles, mtiles, total, per_xcd);
    else
        hipLaunchKernelGGL((qmm_t_kernel<DT, BITS, GS, MT, false>), grid, block, 0, st, w, s, b, x, out, ws,
                           M, N, K, splits, ntiles, mtiles, total, per_xcd);
    return hipGetLastError();
}

template <int DT, int BITS, int GS>
hipError_t qmm_launch_gs(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                         float* ws, int M, int N, int K, int splits, hipStream_t st) {
    switch (qmm_mt_for(M)) {
        case 1: return qmm_launch_mt<DT, BITS, GS, 1>(w, s, b, x, out, ws, M, N, K, splits, st);
        case 2: return qmm_launch_mt<DT, BITS, GS, 2>(w, s, b, x, out, ws, M, N, K, splits, st);
        case 3: return qmm_launch_mt<DT, BITS, GS, 3>(w, s, b, x, out, ws, M, N, K, splits, st);
        case 4: return qmm_launch_mt<DT, BITS, GS, 4>(w, s, b, x, out, ws, M, N, K, splits, st);
        case 6: return qmm_launch_mt<DT, BITS, GS, 6>(w, s, b, x, out, ws, M, N, K, splits, st);
        default: return qmm_launch_mt<DT, BITS, GS, 8>(w, s, b, x, out, ws, M, N, K, splits, st);
    }
}

template <int BITS>
hipError_t qmm_launch_bits(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                           float* ws, int M, int N, int K, int gs, int dt, int splits, hipStream_t st) {
    if (dt == DT_F16) {
        switch (gs) {
            case 32: return qmm_launch_gs<DT_F16, BITS, 32>(w, s, b, x, out, ws, M, N, K, splits, st);
            case 64: return qmm_launch_gs<DT_F16, BITS, 64>(w, s, b, x, out, ws, M, N, K, splits, st);
            default: return qmm_launch_gs<DT_F16, BITS, 128>(w, s, b, x, out, ws, M, N, K, splits, st);
        }
    }
    switch (gs) {
        case 32: return qmm_launch_gs<DT_BF16, BITS, 32>(w, s, b, x, out, ws, M, N, K, splits, st);
        case 64: return qmm_launch_gs<DT_BF16, BITS, 64>(w, s, b, x, out, ws, M, N, K, splits, st);
        default: return qmm_launch_gs<DT_BF16, BITS, 128>(w, s, b, x, out, ws, M, N, K, splits, st);
    }
}

hipError_t qmm_launch_b2(const uint32_t*, const void*, const void*, const void*, void*, float*, int, int,
                         int, int, int, int, hipStream_t);
hipError_t qmm_launch_b4(const uint32_t*, const void*, const void*, const void*, void*, float*, int, int,
                         int, int, int, int, hipStream_t);
hipError_t qmm_launch_b8(const uint32_t*, const void*, const void*, const void*, void*, float*, int, int,
                         int, int, int, int, hipStream_t);

}  // namespace qmx
