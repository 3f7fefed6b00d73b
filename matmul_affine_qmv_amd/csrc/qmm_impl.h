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
// * A work-group of 8 waves owns an output tile of BM = 16*MT rows of x by
//   BN = 128 columns of W and a range of 128-column K blocks (4 MFMA k-steps
//   each).  Waves 0-3 each own 2 fragments of 16 columns and take k-steps
//   0-1 of every block; waves 4-7 own the same columns and take k-steps 2-3.
//   The two halves add their float32 tiles through LDS once at the end, so a
//   CU runs two waves per SIMD without splitting K further across
//   work-groups (which would cost HBM traffic for partials).
// * Packed weights are used by exactly one wave, so they go straight from
//   HBM into that wave's MFMA B-operand registers through a 4-deep register
//   ring (three blocks in flight while one is consumed); they never touch LDS.
// * x is shared by the 4 waves: it is prefetched two blocks ahead into
//   registers, written to one of two LDS buffers in the k order the code
//   expansion produces, and read back as MFMA A operands; the block's
//   scales/biases are staged alongside in float32.  One barrier per K block.
// * Codes are expanded in registers right before the MFMA into exact 16-bit
//   integers: one v_perm per pair of codes sets a magic exponent byte above
//   two byte-aligned fields (0x43qq is the bf16 value 128 + q, 0x64qq the f16
//   value 1024 + q).  The constant offset OFF*sum(x) this adds is removed in
//   the group epilogue.  The codes come out in a fixed permutation of k; x
//   is written to LDS in the same order, and since both MFMA operands see the
//   same permutation the dot product is unchanged.
// * MFMA v_mfma_f32_16x16x32_{bf16,f16}: A = x fragment (16 rows of M),
//   B = W codes (16 columns of N).  A group of GS codes is GS/32 MFMA k-steps
//   accumulated into a fresh float32 tile; the same A fragments against an
//   all-ones B give the group's row sums of x in a matching tile, and the
//   epilogue adds scale * (tile) + (bias - OFF*scale) * (row sums) in float32.  Scale and bias
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
    static constexpr int WPS = BITS == 8 ? 2 : 1;            // words a lane loads per k-step
    static constexpr int WRING = 4;                          // register ring depth for W
    static constexpr int XPR = QMM_KB / 8;                   // 16-byte x pieces per row per block
    static constexpr int XPT = (MT * 16 * XPR + QMM_THREADS - 1) / QMM_THREADS;  // pieces per thread
    static constexpr int XROWS = XPT * QMM_THREADS / XPR;    // x rows held in LDS (>= BM)
    static constexpr int X_BYTES = XROWS * XP * 2;
    static constexpr int SB_BYTES = 2 * GPB * QMM_BN * 4;
    static constexpr int BUF_BYTES = X_BYTES + SB_BYTES;
    static constexpr int SB_SLICES = QMM_THREADS / QMM_BN;   // thread slices over the groups of a block
    static constexpr float OFF = (DT == DT_F16) ? 1024.f : (BITS == 8 ? 0.f : 128.f);
    static constexpr int RED_BYTES = QMM_WAVES_N * MT * QMM_NB * 4 * 64 * 4;
    static_assert(BUF_BYTES % 16 == 0, "buffer alignment");
    static_assert(2 * BUF_BYTES <= 160 * 1024, "LDS budget");
    static_assert(RED_BYTES <= 2 * BUF_BYTES, "end reduction reuses the LDS buffers");
    static_assert(GPB <= SB_SLICES, "one scale/bias slice per group");
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

// 8 codes of one unit as 16-bit MFMA operands (exact integers).  The word
// is split into byte-aligned fields and one v_perm per pair puts two field
// bytes under the magic exponent byte: 0x43qq is the bf16 value 128 + q and
// 0x64qq the f16 value 1024 + q.  Element orders of the 8 operand slots:
//   4-bit: 0,2,4,6,1,3,5,7   (low nibbles, then high nibbles, of one word)
//   2-bit: 0,4,1,5,2,6,3,7   (fields t of the unit's two bytes)
//   8-bit: 0..7              (bytes of two words; bf16 converts, since 128 + q
//                             would overflow the bf16 mantissa for q >= 128)
__device__ constexpr uint32_t perm_sel(int i, int j) {   // bytes i, j of the field word under the magic byte
    return (uint32_t)i | (4u << 8) | ((uint32_t)j << 16) | (4u << 24);
}

template <int DT, int BITS>
__device__ __forceinline__ u32x4 unpack_unit(uint32_t w0, uint32_t w1) {
    constexpr uint32_t MB = DT == DT_F16 ? 0x64646464u : 0x43434343u;
    u32x4 r;
    if constexpr (BITS == 4) {
        const uint32_t lo = w0 & 0x0f0f0f0fu, hi = (w0 >> 4) & 0x0f0f0f0fu;
        r.x = __builtin_amdgcn_perm(MB, lo, perm_sel(0, 1));
        r.y = __builtin_amdgcn_perm(MB, lo, perm_sel(2, 3));
        r.z = __builtin_amdgcn_perm(MB, hi, perm_sel(0, 1));
        r.w = __builtin_amdgcn_perm(MB, hi, perm_sel(2, 3));
    } else if constexpr (BITS == 2) {
        // w0 holds the unit in its low 16 bits: byte 0 = codes 0-3, byte 1 = codes 4-7
        r.x = __builtin_amdgcn_perm(MB, w0 & 0x0303u, perm_sel(0, 1));
        r.y = __builtin_amdgcn_perm(MB, (w0 >> 2) & 0x0303u, perm_sel(0, 1));
        r.z = __builtin_amdgcn_perm(MB, (w0 >> 4) & 0x0303u, perm_sel(0, 1));
        r.w = __builtin_amdgcn_perm(MB, (w0 >> 6) & 0x0303u, perm_sel(0, 1));
    } else if constexpr (DT == DT_F16) {
        r.x = __builtin_amdgcn_perm(MB, w0, perm_sel(0, 1));
        r.y = __builtin_amdgcn_perm(MB, w0, perm_sel(2, 3));
        r.z = __builtin_amdgcn_perm(MB, w1, perm_sel(0, 1));
        r.w = __builtin_amdgcn_perm(MB, w1, perm_sel(2, 3));
    } else {
        // bf16 holds every integer up to 256 exactly: convert, keep the upper half.
        auto pair = [](uint32_t a, uint32_t b) {
            return __builtin_amdgcn_perm(__float_as_uint((float)b), __float_as_uint((float)a), 0x07060302u);
        };
        r.x = pair(w0 & 0xffu, (w0 >> 8) & 0xffu);
        r.y = pair((w0 >> 16) & 0xffu, w0 >> 24);
        r.z = pair(w1 & 0xffu, (w1 >> 8) & 0xffu);
        r.w = pair((w1 >> 16) & 0xffu, w1 >> 24);
    }
    return r;
}

// Eight consecutive 16-bit x values (d = x0x1, x2x3, x4x5, x6x7) in the
// slot order unpack_unit uses for BITS.
template <int BITS>
__device__ __forceinline__ u32x4 permute_x(u32x4 d) {
    if constexpr (BITS == 8) {
        return d;
    } else if constexpr (BITS == 4) {
        // (x0,x2) (x4,x6) (x1,x3) (x5,x7)
        return u32x4{__builtin_amdgcn_perm(d.y, d.x, 0x05040100u), __builtin_amdgcn_perm(d.w, d.z, 0x05040100u),
                     __builtin_amdgcn_perm(d.y, d.x, 0x07060302u), __builtin_amdgcn_perm(d.w, d.z, 0x07060302u)};
    } else {
        // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
        return u32x4{__builtin_amdgcn_perm(d.z, d.x, 0x05040100u), __builtin_amdgcn_perm(d.z, d.x, 0x07060302u),
                     __builtin_amdgcn_perm(d.w, d.y, 0x05040100u), __builtin_amdgcn_perm(d.w, d.y, 0x07060302u)};
    }
}

// WPL consecutive words at p (WPL = 1, 2, 4 or 8; 16-byte aligned for 4 and 8).
template <int WPL>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&v)[WPL]) {
    if constexpr (WPL == 1) {
        v[0] = p[0];
    } else if constexpr (WPL == 2) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(p);
        v[0] = a.x; v[1] = a.y;
    } else {
#pragma unroll
        for (int i = 0; i < WPL / 4; ++i) {
            const u32x4 a = reinterpret_cast<const u32x4*>(p)[i];
            v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
        }
    }
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
    const int nk = kb1 - kb0;
    const int G = K / GS;
    const size_t row_words = (size_t)K * BITS / 32;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & (QMM_WAVES_N - 1);   // column slice of this wave
    const int wk = wave / QMM_WAVES_N;          // k-step pair of this wave: steps 2wk, 2wk+1 of each block
    const int lrow = lane & 15, lgrp = lane >> 4;

    // ---- x (+ scales/biases) ring: 2 register slots -> 2 LDS buffers.
    // Every prefetch load is unconditional, with the block index and the row
    // and column indices clamped into range: rows of x past M and columns
    // past N then only feed outputs that are never stored.  Loaded values are
    // left untouched until they are written to LDS two blocks later, so the
    // compiler never has to wait on a load it has just issued.
    u32x4 xr[2][C::XPT];
    uint32_t sr[2], br[2];
    const int sb_col = tid % QMM_BN;
    const int sb_g = tid / QMM_BN;
    const bool sb_active = sb_g < C::GPB;
    const int sb_n = min(n0 + sb_col, N - 1);
    const int sb_gl = min(sb_g, C::GPB - 1);   // in-range group for inactive slices

    auto x_gload = [&](int kb_req, int slot) {
        const int kb = min(kb_req, kb1 - 1);
        const int k0 = kb * QMM_KB;
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) {
            const int p = tid + QMM_THREADS * i;              // piece p: row p / XPR, unit p % XPR
            const int m = min(m0 + p / C::XPR, M - 1);
            xr[slot][i] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + (size_t)m * K + k0 +
                                                          8 * (p % C::XPR));
        }
        const size_t gi = (size_t)sb_n * G + (size_t)kb * C::GPB + sb_gl;
        sr[slot] = static_cast<const uint16_t*>(scales)[gi];
        br[slot] = static_cast<const uint16_t*>(biases)[gi];
    };

    auto x_lstore = [&](int slot, int buf) {
        unsigned char* base = smem + buf * C::BUF_BYTES;
        uint16_t* xl = reinterpret_cast<uint16_t*>(base);
        float* sbl = reinterpret_cast<float*>(base + C::X_BYTES);
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) {
            const int p = tid + QMM_THREADS * i;
            *reinterpret_cast<u32x4*>(xl + (p / C::XPR) * C::XP + 8 * (p % C::XPR)) = permute_x<BITS>(xr[slot][i]);
        }
        if (sb_active) {
            const float sv = DT == DT_F16 ? f16_bits_to_f32(sr[slot]) : bf16_bits_to_f32(sr[slot]);
            const float bv = DT == DT_F16 ? f16_bits_to_f32(br[slot]) : bf16_bits_to_f32(br[slot]);
            sbl[sb_g * QMM_BN + sb_col] = sv;
            sbl[(C::GPB + sb_g) * QMM_BN + sb_col] = fmaf(-C::OFF, sv, bv);
        }
    };

    // ---- W ring: WRING register slots of this wave's B-operand words (2 k-steps)
    // code offset (within the block) of this lane's unit in k-step s
    auto unit_code = [&](int s) { return (s / C::KS) * GS + lgrp * C::S + 8 * (s % C::KS); };
    uint32_t wr[C::WRING][NB][2][C::WPS];
    auto w_gload = [&](int kb_req, int slot) {
        const int kb = min(kb_req, kb1 - 1);
#pragma unroll
        for (int nf = 0; nf < NB; ++nf) {
            const int n = min(n0 + wn * (NB * 16) + nf * 16 + lrow, N - 1);
            const uint32_t* row = w + (size_t)n * row_words + (size_t)kb * C::WROW;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int word = unit_code(2 * wk + st) * BITS / 32;
                if constexpr (C::WPS == 2) {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(row + word);
                    wr[slot][nf][st][0] = v.x;
                    wr[slot][nf][st][1] = v.y;
                } else {
                    wr[slot][nf][st][0] = row[word];
                }
            }
        }
    };

    f32x4 run[MT][NB];
#pragma unroll
    for (int mf = 0; mf < MT; ++mf)
#pragma unroll
        for (int nf = 0; nf < NB; ++nf) run[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr uint32_t ONE2 = DT == DT_F16 ? 0x3c003c00u : 0x3f803f80u;
    const u32x4 ones = u32x4{ONE2, ONE2, ONE2, ONE2};

    auto compute = [&](int buf, int wslot) {
        const unsigned char* base = smem + buf * C::BUF_BYTES;
        const uint16_t* xl = reinterpret_cast<const uint16_t*>(base);
        const float* sbl = reinterpret_cast<const float*>(base + C::X_BYTES);
        // expand this wave's two k-steps of codes once
        u32x4 bf[2][NB];
        int off[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int c = unit_code(2 * wk + st);
            off[st] = c;
#pragma unroll
            for (int nf = 0; nf < NB; ++nf) {
                const uint32_t* bw = wr[wslot][nf][st];
                if constexpr (BITS == 4) {
                    bf[st][nf] = unpack_unit<DT, 4>(bw[0], 0u);
                } else if constexpr (BITS == 8) {
                    bf[st][nf] = unpack_unit<DT, 8>(bw[0], bw[1]);
                } else {
                    bf[st][nf] = unpack_unit<DT, 2>((bw[0] >> (16 * ((c >> 3) & 1))) & 0xffffu, 0u);
                }
            }
        }
        // the two k-steps share one group unless a group is a single k-step
        constexpr int NG = C::KS >= 2 ? 1 : 2;
        float sv[NG][NB], bv[NG][NB];
#pragma unroll
        for (int gp = 0; gp < NG; ++gp) {
            const int g = (2 * wk + gp) / C::KS;
#pragma unroll
            for (int nf = 0; nf < NB; ++nf) {
                const int col = wn * (NB * 16) + nf * 16 + lrow;
                sv[gp][nf] = sbl[g * QMM_BN + col];
                bv[gp][nf] = sbl[(C::GPB + g) * QMM_BN + col];
            }
        }
        // one 16-row fragment of x at a time keeps one row of group tiles live; the
        // group's row sums of x come from one more MFMA against ones
#pragma unroll
        for (int mf = 0; mf < MT; ++mf) {
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(xl + (mf * 16 + lrow) * C::XP + off[0]);
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(xl + (mf * 16 + lrow) * C::XP + off[1]);
#pragma unroll
            for (int gp = 0; gp < NG; ++gp) {
                f32x4 gacc[NB];
#pragma unroll
                for (int nf = 0; nf < NB; ++nf) {
                    if constexpr (NG == 1) {
                        gacc[nf] = mfma16x16x32<DT>(a0, bf[0][nf], f32x4{0.f, 0.f, 0.f, 0.f});
                        gacc[nf] = mfma16x16x32<DT>(a1, bf[1][nf], gacc[nf]);
                    } else {
                        gacc[nf] = mfma16x16x32<DT>(gp ? a1 : a0, bf[gp][nf], f32x4{0.f, 0.f, 0.f, 0.f});
                    }
                }
                f32x4 gxs;
                if constexpr (NG == 1) {
                    gxs = mfma16x16x32<DT>(a0, ones, f32x4{0.f, 0.f, 0.f, 0.f});
                    gxs = mfma16x16x32<DT>(a1, ones, gxs);
                } else {
                    gxs = mfma16x16x32<DT>(gp ? a1 : a0, ones, f32x4{0.f, 0.f, 0.f, 0.f});
                }
#pragma unroll
                for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        run[mf][nf][v] = fmaf(sv[gp][nf], gacc[nf][v], fmaf(bv[gp][nf], gxs[v], run[mf][nf][v]));
            }
        }
    };

    if (nk > 0) {
        x_gload(kb0, 0);
        x_gload(kb0 + 1, 1);
#pragma unroll
        for (int i = 0; i < C::WRING; ++i) w_gload(kb0 + i, i);
        x_lstore(0, 0);
        x_gload(kb0 + 2, 0);
        __syncthreads();
        // Block i: compute from LDS buffer i%2 and W slot i%4; then stage x(i+1)
        // into the other buffer and request x(i+3) and W(i+4) into the freed
        // slots.  Past the last block the requests repeat the last block and
        // the staged data is never read.
        for (int base = 0; base < nk; base += C::WRING) {
#pragma unroll
            for (int j = 0; j < C::WRING; ++j) {
                const int i = base + j;
                if (i < nk) compute(j & 1, j);
                x_lstore((j + 1) & 1, (j + 1) & 1);
                x_gload(kb0 + i + 3, (j + 1) & 1);
                w_gload(kb0 + i + C::WRING, j);
                __syncthreads();
            }
        }
    }

    // add the second half's tiles to the first half's, then store
    float* red = reinterpret_cast<float*>(smem);
    if (wk == 1) {
#pragma unroll
        for (int mf = 0; mf < MT; ++mf)
#pragma unroll
            for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[(((wn * MT + mf) * NB + nf) * 4 + v) * 64 + lane] = run[mf][nf][v];
    }
    __syncthreads();
    if (wk == 1) return;
#pragma unroll
    for (int mf = 0; mf < MT; ++mf)
#pragma unroll
        for (int nf = 0; nf < NB; ++nf)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float r = run[mf][nf][v] + red[(((wn * MT + mf) * NB + nf) * 4 + v) * 64 + lane];
                const int m = m0 + mf * 16 + 4 * lgrp + v;
                const int n = n0 + wn * (NB * 16) + nf * 16 + lrow;
                if (m < M && n < N) {
                    if constexpr (SPLIT)
                        ws[((size_t)split * M + m) * N + n] = r;
                    else
                        store_elem<DT>(out, (size_t)m * N + n, r);
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
