// qmv.hip -- group-wise affine quantized matvec (small M) on the gfx950 vector ALUs.
//
// Method (page "metaltile-std src/mlx/quantized.rs", qmv kernel): per group
// g of row n, out += scale[n,g] * sum q*x + bias[n,g] * sum x, with the sum
// of x formed once per group part and shared by every row (bias hoist), x
// held in registers and reused across the rows a wave owns, float32
// accumulators, and a cross-lane reduction followed by one store per output.
//
// gfx950 mapping:
// * A row group is QMV_ROWS consecutive rows of W, served with up to MT rows
//   of x.  A wave owns RG row groups (64/RG lanes each) and a contiguous range
//   of their chunks (16 bytes for 2-, 4- and 8-bit codes, BITS words = 32
//   codes for 1, 3, 5 and 6 bits); lane l of a row group takes chunks l,
//   l + 64/RG, ... of that range, so each load instruction reads 256 B-1.5 KB
//   contiguous per row.  KSPLIT waves of one work-group may split the chunks of the same
//   rows; their partial sums are added in LDS in a fixed order.  The split
//   (KSPLIT, RG) comes from qmv_split_for.
// * Loads are buffer loads through resources based at the work-group's first
//   row; per-lane offsets are fixed for the loop and each round adds one
//   scalar offset, so the loop does no address arithmetic on the vector ALU.
// * 16-bit x: a word is split into byte-aligned fields and one v_perm per
//   pair of codes sets a magic exponent byte above two of them (0x43qq is the
//   bf16 value 128+q, 0x64qq the f16 value 1024+q; f16 then subtracts 1024
//   exactly), so codes become exact 16-bit integers contracted with
//   v_dot2_f32_{bf16,f16} two at a time.  The bf16 offset adds 128*sum(x),
//   removed by using bias - 128*scale in the group epilogue.  x is paired in
//   the same element order with v_perm.  float32 x (and 8-bit codes with
//   bf16 x) use per-code conversion and float32 FMA.
// * 1, 3, 5 and 6 bits: codes 2k and 2k+1 of a chunk are cut as one window
//   and moved under the magic bytes with a shift-or and an and-or (the magic
//   held in a register), pairing with x dword k as loaded.
// * A batch of problems is the third grid dimension (pointers offset by the
//   problem's strides or index-picked matrices at the start).  A gather at
//   M = 1 may group consecutive problems on one weight matrix into the x rows
//   of one tile, so that matrix streams once for all of them.
// * The final reductions are fixed xor-butterflies, so results do not change
//   from run to run.
#include <algorithm>

#include "qmx_device.h"
#include "qmx_internal.h"

namespace qmx {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a), __builtin_bit_cast(b2_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}

// The 16-bit code pairs of a word.  The word is first split into
// byte-aligned fields (4-bit: low nibbles = codes 0,2,4,6 and high nibbles =
// codes 1,3,5,7; 2-bit: field t of every byte = codes t, t+4, t+8, t+12;
// 8-bit: the bytes themselves), then one v_perm per pair puts two field bytes
// under the magic exponent byte: 0x43 makes the bf16 value 128 + q, 0x64 the
// f16 value 1024 + q, from which f16 subtracts 1024 exactly.
template <int BITS>
struct PairOrder {
    // element index (within the word) of the first / second code of pair k
    __device__ static constexpr int first(int k) {
        return BITS == 4 ? (k < 2 ? 4 * k : 4 * (k - 2) + 1)
             : BITS == 2 ? ((k & 1) ? 8 + (k >> 1) : (k >> 1))
             : 2 * k;
    }
    __device__ static constexpr int second(int k) { return first(k) + (BITS == 4 ? 2 : BITS == 2 ? 4 : 1); }
};

// v_perm_b32 selector taking bytes i and j of the second operand (the field
// word) and byte 0 of the first (the magic byte), as (lo16, hi16) = (i, j).
__device__ constexpr uint32_t magic_sel(int i, int j) {
    return (uint32_t)i | (4u << 8) | ((uint32_t)j << 16) | (4u << 24);
}

template <int DT, int BITS>
__device__ __forceinline__ void code_pairs(uint32_t w, uint32_t (&q)[16 / BITS]) {
    constexpr uint32_t MB = DT == DT_BF16 ? 0x43434343u : 0x64646464u;
    if constexpr (BITS == 4) {
        const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
        q[0] = __builtin_amdgcn_perm(MB, lo, magic_sel(0, 1));
        q[1] = __builtin_amdgcn_perm(MB, lo, magic_sel(2, 3));
        q[2] = __builtin_amdgcn_perm(MB, hi, magic_sel(0, 1));
        q[3] = __builtin_amdgcn_perm(MB, hi, magic_sel(2, 3));
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t f = (w >> (2 * t)) & 0x03030303u;
            q[2 * t] = __builtin_amdgcn_perm(MB, f, magic_sel(0, 1));
            q[2 * t + 1] = __builtin_amdgcn_perm(MB, f, magic_sel(2, 3));
        }
    } else {
        q[0] = __builtin_amdgcn_perm(MB, w, magic_sel(0, 1));
        q[1] = __builtin_amdgcn_perm(MB, w, magic_sel(2, 3));
    }
    if constexpr (DT == DT_F16) {
#pragma unroll
        for (int k = 0; k < 16 / BITS; ++k) {
            const h2_t v = __builtin_bit_cast(h2_t, q[k]) - h2_t{(_Float16)1024.f, (_Float16)1024.f};
            q[k] = __builtin_bit_cast(uint32_t, v);
        }
    }
}

// x values a and b (element indices within the word, whose 16-bit values sit
// two per dword in d) as one (lo, hi) pair.
__device__ __forceinline__ uint32_t x_pair(const uint32_t* d, int a, int b) {
    const uint32_t sa = (a & 1) ? 2u : 0u, sb = (b & 1) ? 6u : 4u;
    const uint32_t sel = sa | ((sa + 1) << 8) | (sb << 16) | ((sb + 1) << 24);
    return __builtin_amdgcn_perm(d[b >> 1], d[a >> 1], sel);
}

// Offset that code_pairs leaves on every code.
template <int DT>
constexpr float code_offset() { return DT == DT_BF16 ? 128.f : 0.f; }

template <int DT, int BITS>
constexpr bool use_dot2() { return DT != DT_F32 && (BITS != 8 || DT == DT_F16); }

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

// Registers of one chunk: the RR rows' weight chunks (CW words each), their
// scales and biases (raw storage bits), and the MT rows' x values under the
// chunk.
template <int DT, int BITS, int GS, int MT, int RR = QMV_ROWS>
struct QmvStage {
    static constexpr int R = RR;
    static constexpr int CW = qmv_chunk_words(BITS);
    static constexpr int CPC = qmv_chunk_codes(BITS);
    static constexpr int PARTS = CPC > GS ? CPC / GS : 1;
    static constexpr int XQ = CPC * (DT == DT_F32 ? 4 : 2) / 16;   // 16-byte x pieces per chunk
    uint32_t w[R][CW];
    uint32_t s[R][PARTS], b[R][PARTS];
    u32x4 x[MT][XQ];
};

template <int DT>
__device__ __forceinline__ uint32_t buffer_raw(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (DT == DT_F32) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Where a lane's loads come from.  Every array is addressed through a buffer
// resource based at the work-group's first row; a lane's byte offsets for its
// first chunk are fixed (voffset) and each round adds the same scalar offset to
// all lanes (soffset), so no per-round address arithmetic runs on the vector ALU.
template <int DT, int BITS, int GS, int MT>
struct QmvAddr {
    static constexpr int R = QMV_ROWS;
    static constexpr int EB = DT == DT_F32 ? 4 : 2;
    __amdgpu_buffer_rsrc_t w, s, b, x;
    int vw[R], vsb[R], vx[MT];
};

template <int DT, int BITS, int GS, int MT>
__device__ __forceinline__ void qmv_load(QmvStage<DT, BITS, GS, MT>& st, const QmvAddr<DT, BITS, GS, MT>& ad,
                                         int sw, int ssb, int sx) {
    using S = QmvStage<DT, BITS, GS, MT>;
    constexpr int EB = QmvAddr<DT, BITS, GS, MT>::EB;
    // issued in the order the arithmetic first needs them (x, then the rows, then
    // the group epilogue's scales and biases), so its waits can be partial
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < S::XQ; ++i)
            st.x[m][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad.x, ad.vx[m] + 16 * i, sx, 0));
#pragma unroll
    for (int r = 0; r < S::R; ++r) {
        if constexpr (S::CW == 1) {
            st.w[r][0] = __builtin_amdgcn_raw_buffer_load_b32(ad.w, ad.vw[r], sw, 0);
        } else if constexpr (S::CW == 3) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b96(ad.w, ad.vw[r], sw, 0);
            st.w[r][0] = v[0]; st.w[r][1] = v[1]; st.w[r][2] = v[2];
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(ad.w, ad.vw[r], sw, 0);
            st.w[r][0] = v[0]; st.w[r][1] = v[1]; st.w[r][2] = v[2]; st.w[r][3] = v[3];
            if constexpr (S::CW == 5) {
                st.w[r][4] = __builtin_amdgcn_raw_buffer_load_b32(ad.w, ad.vw[r] + 16, sw, 0);
            } else if constexpr (S::CW == 6) {
                const auto u = __builtin_amdgcn_raw_buffer_load_b64(ad.w, ad.vw[r] + 16, sw, 0);
                st.w[r][4] = u[0]; st.w[r][5] = u[1];
            }
        }
    }
#pragma unroll
    for (int r = 0; r < S::R; ++r)
#pragma unroll
        for (int p = 0; p < S::PARTS; ++p) {
            st.s[r][p] = buffer_raw<DT>(ad.s, ad.vsb[r] + p * EB, ssb);
            st.b[r][p] = buffer_raw<DT>(ad.b, ad.vsb[r] + p * EB, ssb);
        }
}

template <int DT>
__device__ __forceinline__ float raw_to_f32(uint32_t v) {
    if constexpr (DT == DT_F32) return __uint_as_float(v);
    else if constexpr (DT == DT_F16) return f16_bits_to_f32(v);
    else return bf16_bits_to_f32(v);
}

// Word j (0..3) of a 16-byte piece.
__device__ __forceinline__ uint32_t word_of(const u32x4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Code e of a chunk of CW words that holds its codes as one little-endian
// bit stream (e and so the bit position are compile-time constants after
// unrolling: one bit-field extract, or a funnel shift where the field
// straddles two words).
template <int BITS, int CW>
__device__ __forceinline__ uint32_t stream_code(const uint32_t (&w)[CW], int e) {
    const int bit = BITS * e, i = bit >> 5, sh = bit & 31;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    if (sh + BITS <= 32) return (w[i] >> sh) & MASK;
    return __builtin_amdgcn_alignbit(w[i + 1], w[i], sh) & MASK;
}

// Codes e and e + 1 of such a chunk as a pair of exact 16-bit values under
// the magic exponent (128 + q in bf16, q in f16 after removing 1024).
// The two fields are taken as one 2*BITS-bit window t (code e in its low
// BITS bits); t | t << (16 - BITS) puts code e + 1 at bit 16, and one mask
// keeps both codes under the magic bytes.
// mb holds the magic bytes in a register (see magic_bytes) so that the mask
// and the magic go into one and-or.
template <int DT, int BITS, int CW>
__device__ __forceinline__ uint32_t stream_pair(const uint32_t (&w)[CW], int e, uint32_t mb) {
    constexpr uint32_t MASK = (1u << BITS) - 1u, WIN = (1u << (2 * BITS)) - 1u;
    const int bit = BITS * e, i = bit >> 5, sh = bit & 31;
    const uint32_t t = (sh + 2 * BITS <= 32 ? w[i] >> sh : __builtin_amdgcn_alignbit(w[i + 1], w[i], sh)) & WIN;
    uint32_t p = (((t << (16 - BITS)) | t) & (MASK | (MASK << 16))) | mb;
    if constexpr (DT == DT_F16) {
        const h2_t v = __builtin_bit_cast(h2_t, p) - h2_t{(_Float16)1024.f, (_Float16)1024.f};
        p = __builtin_bit_cast(uint32_t, v);
    }
    return p;
}

template <int DT, int BITS, int GS, int MT, int RR>
__device__ __forceinline__ void qmv_consume(const QmvStage<DT, BITS, GS, MT, RR>& st, float (&acc)[RR][MT]) {
    using S = QmvStage<DT, BITS, GS, MT, RR>;
    constexpr int R = S::R;
    constexpr int PARTS = S::PARTS;
    constexpr int WPP = 4 / PARTS;          // words per group part
    constexpr int CPW = 32 / BITS;          // codes per word

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

    if constexpr (S::CW != 4) {
        // 1-, 3-, 5- and 6-bit codes: 32 per chunk in natural order, so codes
        // 2k and 2k+1 pair with x dword k as it is loaded.
        static_assert(PARTS == 1 && S::CPC == 32, "one group part of 32 codes per chunk");
        if constexpr (DT != DT_F32) {
            constexpr uint32_t ONES = DT == DT_BF16 ? 0x3f803f80u : 0x3c003c00u;
            uint32_t xp[MT][16];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float t = 0.f;
#pragma unroll
                for (int i = 0; i < S::XQ; ++i) {
                    xp[m][4 * i] = st.x[m][i].x; xp[m][4 * i + 1] = st.x[m][i].y;
                    xp[m][4 * i + 2] = st.x[m][i].z; xp[m][4 * i + 3] = st.x[m][i].w;
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) t = dot2<DT>(xp[m][k], ONES, t);
                xs[m][0] = t;
            }
            const uint32_t mb = magic_bytes<DT>();
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t q = stream_pair<DT, BITS>(st.w[r], 2 * k, mb);
#pragma unroll
                    for (int m = 0; m < MT; ++m) qd[r][m][0] = dot2<DT>(q, xp[m][k], qd[r][m][0]);
                }
        } else {
            float xv[MT][32];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float t = 0.f;
#pragma unroll
                for (int i = 0; i < S::XQ; ++i) {
                    xv[m][4 * i] = __uint_as_float(st.x[m][i].x); xv[m][4 * i + 1] = __uint_as_float(st.x[m][i].y);
                    xv[m][4 * i + 2] = __uint_as_float(st.x[m][i].z); xv[m][4 * i + 3] = __uint_as_float(st.x[m][i].w);
                }
#pragma unroll
                for (int e = 0; e < 32; ++e) t += xv[m][e];
                xs[m][0] = t;
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const float q = (float)stream_code<BITS>(st.w[r], e);
#pragma unroll
                    for (int m = 0; m < MT; ++m) qd[r][m][0] = fmaf(q, xv[m][e], qd[r][m][0]);
                }
        }
    } else if constexpr (use_dot2<DT, BITS>()) {
        // Each word is split into byte-aligned fields (one code per byte); a
        // v_perm places two of those bytes under the magic exponent byte,
        // giving a pair of exact 16-bit codes, and x is paired the same way.
        constexpr int PPW = CPW / 2;                       // pairs per word
        constexpr uint32_t ONES = DT == DT_BF16 ? 0x3f803f80u : 0x3c003c00u;
        uint32_t xp[MT][4][PPW];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            uint32_t d[S::XQ * 4];
#pragma unroll
            for (int i = 0; i < S::XQ; ++i) {
                d[4 * i] = st.x[m][i].x; d[4 * i + 1] = st.x[m][i].y;
                d[4 * i + 2] = st.x[m][i].z; d[4 * i + 3] = st.x[m][i].w;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t* dj = d + j * (CPW / 2);   // CPW values = CPW/2 dwords per word
                float t = xs[m][j / WPP];
#pragma unroll
                for (int k = 0; k < PPW; ++k) {
                    xp[m][j][k] = x_pair(dj, PairOrder<BITS>::first(k), PairOrder<BITS>::second(k));
                    t = dot2<DT>(xp[m][j][k], ONES, t);
                }
                xs[m][j / WPP] = t;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t q[PPW];
                code_pairs<DT, BITS>(st.w[r][j], q);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float t = qd[r][m][j / WPP];
#pragma unroll
                    for (int k = 0; k < PPW; ++k) t = dot2<DT>(q[k], xp[m][j][k], t);
                    qd[r][m][j / WPP] = t;
                }
            }
        }
    } else {
        // float32 path: x converted once per chunk, codes converted one by one
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float xv[MT][CPW];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
                for (int e = 0; e < CPW; ++e) {
                    const int idx = j * CPW + e;       // element within the chunk
                    if constexpr (DT == DT_F32) {
                        const u32x4 q4 = st.x[m][idx / 4];
                        xv[m][e] = __uint_as_float(word_of(q4, idx % 4));
                    } else {
                        const u32x4 q4 = st.x[m][idx / 8];
                        const uint32_t d = word_of(q4, (idx % 8) / 2);
                        xv[m][e] = (idx & 1) ? half_hi<DT>(d) : half_lo<DT>(d);
                    }
                }
                float t = 0.f;
#pragma unroll
                for (int e = 0; e < CPW; ++e) t += xv[m][e];
                xs[m][j / WPP] += t;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float q[CPW];
                unpack_word<BITS>(st.w[r][j], q);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float t = qd[r][m][j / WPP];
#pragma unroll
                    for (int e = 0; e < CPW; ++e) t = fmaf(q[e], xv[m][e], t);
                    qd[r][m][j / WPP] = t;
                }
            }
        }
    }

    constexpr float OFF = use_dot2<DT, BITS>() ? code_offset<DT>() : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int p = 0; p < PARTS; ++p) {
            const float s = raw_to_f32<DT>(st.s[r][p]);
            const float b = fmaf(-OFF, s, raw_to_f32<DT>(st.b[r][p]));
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = fmaf(s, qd[r][m][p], fmaf(b, xs[m][p], acc[r][m]));
        }
}

template <int DT, int BITS, int GS, int MT, int KSPLIT, int RG, int GROUP>
__global__ __launch_bounds__(64 * KSPLIT) void qmv_kernel(const uint32_t* __restrict__ w,
                                                          const void* __restrict__ scales,
                                                          const void* __restrict__ biases,
                                                          const void* __restrict__ x,
                                                          void* __restrict__ out, QmxStrides sd, int M, int N,
                                                          int K) {
    constexpr int R = QMV_ROWS;
    constexpr int LP = 64 / RG;   // lanes per row group
    using S = QmvStage<DT, BITS, GS, MT>;
    // problem blockIdx.z of the batch
    const long long bz = blockIdx.z;
    // Grouped gather (GROUP > 1, M = 1): problem bz leads a tile when it sits at
    // a multiple of GROUP or picks another weight matrix than problem bz - 1;
    // its tile then takes the following problems up to the next such leader,
    // as x rows 1, 2, ... (their outputs are the rows that follow in `out`).
    // Every other problem belongs to a leader's tile and its work-group exits.
    int gcount = 1;
    {
        constexpr int E = DT == DT_F32 ? 4 : 2;
        const long long wz = qmx_w_matrix(sd, bz);
        if constexpr (GROUP > 1) {
            if (bz % GROUP != 0 && qmx_w_matrix(sd, bz - 1) == wz) return;
            while (gcount < GROUP && bz + gcount < (long long)gridDim.z && (bz + gcount) % GROUP != 0 &&
                   qmx_w_matrix(sd, bz + gcount) == wz)
                ++gcount;
        }
        w += wz * sd.w;
        scales = static_cast<const unsigned char*>(scales) + wz * sd.sb * E;
        biases = static_cast<const unsigned char*>(biases) + wz * sd.sb * E;
        if constexpr (GROUP == 1) x = static_cast<const unsigned char*>(x) + qmx_x_matrix(sd, bz) * sd.x * E;
        out = static_cast<unsigned char*>(out) + bz * M * (long long)N * E;
    }
    const int XR = (int)sd.x_row;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lp = lane / LP, ll = lane % LP;
    const int nw = blockIdx.x * RG * R;          // first row of the work-group
    const int n0 = nw + lp * R;                   // first row of this lane's row group
    const int m0 = blockIdx.y * MT;
    const int mcount = GROUP > 1 ? gcount : min(MT, M - m0);
    const int G = K / GS;
    const int chunks = K / S::CPC;
    const size_t row_bytes = (size_t)K * BITS / 8;
    const int c1 = (int)((long)(wave + 1) * chunks / KSPLIT);
    int c = (int)((long)wave * chunks / KSPLIT) + ll;

    // rows past N repeat row N - 1 and x rows past M repeat row m0; neither is stored
    using A = QmvAddr<DT, BITS, GS, MT>;
    constexpr int EB = A::EB;
    A ad;
    ad.w = buffer_over(reinterpret_cast<const unsigned char*>(w) + (size_t)nw * row_bytes, (size_t)(N - nw) * row_bytes);
    ad.s = buffer_over(static_cast<const unsigned char*>(scales) + (size_t)nw * G * EB, (size_t)(N - nw) * G * EB);
    ad.b = buffer_over(static_cast<const unsigned char*>(biases) + (size_t)nw * G * EB, (size_t)(N - nw) * G * EB);
    if constexpr (GROUP > 1) {
        // x rows of the tile's problems, addressed from the first x matrix
        const long long nx = sd.x_index ? sd.num_x : (long long)gridDim.z;
        ad.x = buffer_over(x, (size_t)((nx - 1) * sd.x + K) * EB);
    } else {
        ad.x = buffer_over(static_cast<const unsigned char*>(x) + (size_t)m0 * XR * EB,
                           ((size_t)(M - m0 - 1) * XR + K) * EB);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int rr = min(n0 + r, N - 1) - nw;
        ad.vw[r] = (int)((size_t)rr * row_bytes) + 4 * S::CW * c;
        ad.vsb[r] = (rr * G + (c * S::CPC) / GS) * EB;
    }
    if constexpr (GROUP > 1) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            ad.vx[m] = (int)((qmx_x_matrix(sd, bz + (m < mcount ? m : 0)) * sd.x + c * S::CPC) * EB);
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) ad.vx[m] = ((m < mcount ? m : 0) * XR + c * S::CPC) * EB;
    }
    // per-round scalar steps
    constexpr int STEP_W = LP * 4 * S::CW, STEP_SB = LP * S::CPC / GS * EB, STEP_X = LP * S::CPC * EB;
    static_assert((LP * S::CPC) % GS == 0, "a round advances by whole groups");

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

    // One chunk round in flight per wave: the register budget goes to
    // occupancy (about 7 waves per SIMD), which overlaps loads and arithmetic
    // better on this kernel than a second register set at lower occupancy.
    for (int round = 0; c < c1; c += LP, ++round) {
        S a;
        qmv_load(a, ad, round * STEP_W, round * STEP_SB, round * STEP_X);
        qmv_consume(a, acc);
    }

    // sums over the LP lanes of each row group (fixed xor butterflies); the step
    // loop is outermost so the R*MT independent exchanges of a step share a wait
#pragma unroll
    for (int off = LP / 2; off >= 1; off >>= 1)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] += __shfl_xor(acc[r][m], off, 64);
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (ll == r * MT + m) mine = acc[r][m];
    if constexpr (KSPLIT > 1) {
        __shared__ float part[KSPLIT][RG * R * MT];
        if (ll < R * MT) part[wave][lp * R * MT + ll] = mine;
        __syncthreads();
        if (wave != 0) return;
        if (ll < R * MT) {
            float t = part[0][lp * R * MT + ll];
#pragma unroll
            for (int k = 1; k < KSPLIT; ++k) t += part[k][lp * R * MT + ll];
            mine = t;
        }
    }
    if (ll < R * MT) {
        const int r = ll / MT, m = ll % MT;
        if (n0 + r < N && m < mcount) store_elem<DT>(out, (size_t)(m0 + m) * N + n0 + r, mine);
    }
}

// ---------------------------------------------------------------- deep M = 1 form
// M = 1, 4-bit codes, short rows (at most NR rounds of 64 chunks of 32 codes).
// A work-group of QMV_DEEP_WAVES waves owns QMV_DEEP_WAVES row groups of RW
// rows, one per wave, and stages the row of x in LDS once.  Every wave issues
// the weight, scale and bias loads of all NR of its rounds before it consumes
// the first, so all its rounds are in flight at once: NR is a template
// parameter and the rounds are straight-line code, with no loop join at which
// the compiler would wait for every outstanding load.  A lane whose chunk lies
// past the row takes scale and bias from outside the buffer (they read 0) and
// x = 0, so it adds exactly 0.
constexpr int QMV_DEEP_WAVES = 4;

template <int DT, int GS, int NR, int RW>
__global__ __launch_bounds__(64 * QMV_DEEP_WAVES) void qmv_deep_kernel(
    const uint32_t* __restrict__ w, const void* __restrict__ scales, const void* __restrict__ biases,
    const void* __restrict__ x, void* __restrict__ out, int N, int K) {
    constexpr int R = RW, BITS = 4;
    using S = QmvStage<DT, BITS, GS, 1, RW>;
    static_assert(S::CW == 4 && S::PARTS == 1 && S::CPC == 32, "4-bit chunks of 32 codes, one group part");
    constexpr int EB = DT == DT_F32 ? 4 : 2;               // bytes of an x, scale or bias value
    constexpr int THREADS = 64 * QMV_DEEP_WAVES;
    constexpr int XPIECES = NR * 64 * S::CPC * EB / 16;   // 16-byte pieces of the longest row of x
    constexpr int XPT = XPIECES / THREADS;                 // x pieces per thread
    static_assert(XPIECES % THREADS == 0, "x copies per thread");
    static_assert(NR * 3 * R + XPT < 64, "memory counter range");
    constexpr int OUTSIDE = 0x7ff00000;   // past the scale and bias ranges below (a load there reads 0)
    __shared__ __attribute__((aligned(16))) u32x4 xl[XPIECES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockIdx.x * QMV_DEEP_WAVES * R;      // first row of the work-group
    const int n0 = nw + wave * R;                         // first row of this wave
    const int G = K / GS, chunks = K / S::CPC;
    const size_t row_bytes = (size_t)K / 2;

    // 1. the row of x as 16-byte pieces (piece v at LDS slot v) into registers
    //    first; pieces past the row repeat its last one.  They go to LDS once the
    //    weights below are requested, so only the x loads are waited for there.
    const int xp = K * EB / 16;
    const __amdgpu_buffer_rsrc_t rx = buffer_over(x, (size_t)K * EB);
    u32x4 xv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j)
        xv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, 16 * min(j * THREADS + tid, xp - 1), 0, 0));

    // 2. every round's weights, scales and biases; rows past N repeat row N - 1.
    //    The resources cover the work-group's own rows only, so OUTSIDE is past them.
    const size_t rows = (size_t)min(N - nw, QMV_DEEP_WAVES * R);
    const __amdgpu_buffer_rsrc_t rw =
        buffer_over(reinterpret_cast<const unsigned char*>(w) + (size_t)nw * row_bytes, rows * row_bytes);
    const __amdgpu_buffer_rsrc_t rs =
        buffer_over(static_cast<const unsigned char*>(scales) + (size_t)nw * G * EB, rows * G * EB);
    const __amdgpu_buffer_rsrc_t rb =
        buffer_over(static_cast<const unsigned char*>(biases) + (size_t)nw * G * EB, rows * G * EB);
    uint32_t wr[NR][R][4], sr[NR][R], br[NR][R];
#pragma unroll
    for (int rd = 0; rd < NR; ++rd) {
        const int cr = lane + 64 * rd;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = min(n0 + r, N - 1) - nw;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)((size_t)rr * row_bytes) + 16 * min(cr, chunks - 1), 0, 0);
            wr[rd][r][0] = v[0]; wr[rd][r][1] = v[1]; wr[rd][r][2] = v[2]; wr[rd][r][3] = v[3];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = min(n0 + r, N - 1) - nw;
            const int at = cr < chunks ? (rr * G + (cr * S::CPC) / GS) * EB : OUTSIDE;
            sr[rd][r] = buffer_raw<DT>(rs, at, 0);
            br[rd][r] = buffer_raw<DT>(rb, at, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) xl[j * THREADS + tid] = xv[j];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // 3. the rounds, in order
    float acc[R][1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = 0.f;
#pragma unroll
    for (int rd = 0; rd < NR; ++rd) {
        S a;
        const int cr = lane + 64 * rd;
        const int xc = min(cr, chunks - 1);
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < S::XQ; ++i) a.x[0][i] = cr < chunks ? xl[S::XQ * xc + i] : zero;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) a.w[r][j] = wr[rd][r][j];
            a.s[r][0] = sr[rd][r];
            a.b[r][0] = br[rd][r];
        }
        qmv_consume(a, acc);
    }

    // 4. sums over the wave (fixed xor butterflies)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][0] += __shfl_xor(acc[r][0], off, 64);
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (lane == r) mine = acc[r][0];
    if (lane < R && n0 + lane < N) store_elem<DT>(out, (size_t)n0 + lane, mine);
}

// The deep form's rounds and rows per wave for an M = 1 call (rounds 0: not
// used).  Measured on the chip against the looped kernel:
// * 16-bit x (4-bit gs 64 bf16, N in 1024..14336, K in 1024..6144): with 4
//   rows per wave the deep form wins (5-14%) while the grid holds at most one
//   work-group per CU and a wave takes one round, or two rounds with at least
//   one work-group per two CUs; elsewhere the looped kernel's occupancy serves
//   better (also with 1 or 2 rows per wave: 3-20% slower at N = 14336, 27648).
// * float32 x (two or three rounds): 4 rows per wave from two work-groups per
//   CU on (11008 x 4096: 11.6 -> 9.6 us, 27648 x 5120: 29.4 -> 26.6 us), 2 rows
//   per wave from two work-groups of 8 rows per CU (5120 x 5120: 9.0 ->
//   8.6 us); seven rounds (K = 14336) lost with 1 and 2 rows per wave.
struct QmvDeep {
    int nr, rw;
};
QmvDeep qmv_deep_for(int M, int N, int K, int bits, int dt, int batch, bool plain, const void* x, int cus) {
    if (M != 1 || bits != 4 || batch != 1 || !plain || K <= 0 || N <= 0 || cus <= 0 ||
        (reinterpret_cast<uintptr_t>(x) & 15) != 0)
        return {0, 0};
    const int nr = (K / 32 + 63) / 64;
    const long long n = N;
    if (dt == DT_F32 && (nr == 2 || nr == 3)) {
        if (n >= 2LL * cus * QMV_DEEP_WAVES * 4) return {nr, 4};
        if (n >= 2LL * cus * QMV_DEEP_WAVES * 2) return {nr, 2};
    }
    const long long wgs = (n + QMV_DEEP_WAVES * 4 - 1) / (QMV_DEEP_WAVES * 4);
    if (nr > 2 || wgs > cus || (nr == 2 && 2 * wgs < cus)) return {0, 0};
    return {nr, 4};
}

template <int DT, int GS, int NR, int RW>
static void qmv_deep_go(int N, int K, const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                        hipStream_t st) {
    const dim3 grid((N + QMV_DEEP_WAVES * RW - 1) / (QMV_DEEP_WAVES * RW));
    hipLaunchKernelGGL((qmv_deep_kernel<DT, GS, NR, RW>), grid, dim3(64 * QMV_DEEP_WAVES), 0, st, w, s, b, x, out, N,
                       K);
}

template <int DT, int GS>
static bool qmv_deep_launch(QmvDeep d, int N, int K, const uint32_t* w, const void* s, const void* b, const void* x,
                            void* out, hipStream_t st) {
    if (d.nr == 1 && d.rw == 4) qmv_deep_go<DT, GS, 1, 4>(N, K, w, s, b, x, out, st);
    else if (d.nr == 2 && d.rw == 4) qmv_deep_go<DT, GS, 2, 4>(N, K, w, s, b, x, out, st);
    else if constexpr (DT == DT_F32) {
        if (d.nr == 3 && d.rw == 4) qmv_deep_go<DT, GS, 3, 4>(N, K, w, s, b, x, out, st);
        else if (d.nr == 2 && d.rw == 2) qmv_deep_go<DT, GS, 2, 2>(N, K, w, s, b, x, out, st);
        else if (d.nr == 3 && d.rw == 2) qmv_deep_go<DT, GS, 3, 2>(N, K, w, s, b, x, out, st);
        else return false;
    } else {
        return false;
    }
    return true;
}

int qmv_mt_for(int M) { return M >= 3 ? 4 : (M == 2 ? 2 : 1); }

// Work split of an M = 1 matvec: KS waves of one work-group split the chunks of
// the same rows, and RG row groups of QMV_ROWS rows share one wave (64 / RG
// lanes each).  Each wave walks its chunks in rounds of 64 / RG (one per lane),
// every round a dependent memory round trip.

// Measured on the chip (sweeps of every split on the four 4-bit shapes with K =
// 5120 or 14336): a wave-round (one round of one wave, whatever its lane use)
// costs about 1 us of a SIMD's time when the loads stream, 10% more per extra
// row group (its loads touch more rows at once); a wave's rounds run one after
// another at about 1.6 us each when few waves are in flight; a launch of more
// waves than stay resident (about 7 per SIMD) pays about 0.5 us per extra
// generation.  When the rows alone give about 6 waves per SIMD, sharing a wave
// between row groups measured slower, so only RG = 1 is considered.  The split
// with the lowest max(wave-rounds per SIMD * (1 + 0.1 (RG - 1)) us, rounds *
// 1.6 us) + 0.5 us * (generations - 1) wins; ties go to fewer rounds, then to
// fewer waves per row tile.
QmvSplit qmv_split_for(int M, long long N, int K, int bits) {
    if (qmv_mt_for(M) != 1) return {1, 1};
    static constexpr QmvSplit kCands[] = {{1, 1}, {1, 2}, {1, 4}, {2, 1}, {4, 1}, {5, 2}, {5, 4}};
    constexpr long kResident = 7 * 1024;
    const long chunks = (long)K / qmv_chunk_codes(bits);
    const bool rows_fill = (long)(N + QMV_ROWS - 1) / QMV_ROWS >= 6000;
    QmvSplit best = {1, 1};
    double best_t = -1.0;
    long best_rounds = 0;
    for (const QmvSplit& c : kCands) {
        if (rows_fill && c.rg != 1) continue;
        const long per_wave = (chunks + c.ks - 1) / c.ks;
        if (c.ks > 1 && per_wave < 16) continue;
        const long lanes = 64 / c.rg;
        const long rounds = (per_wave + lanes - 1) / lanes;
        const long waves = (long)((N + QMV_ROWS * c.rg - 1) / (QMV_ROWS * c.rg)) * c.ks;
        const long gens = (waves + kResident - 1) / kResident;
        const double t = std::max((double)(waves * rounds) / 1024.0 * (1.0 + 0.1 * (c.rg - 1)), 1.6 * (double)rounds) +
                         0.5 * (double)(gens > 1 ? gens - 1 : 0);
        if (best_t < 0 || t < best_t - 1e-9 || (t < best_t + 1e-9 && rounds < best_rounds)) {
            best = c;
            best_t = t;
            best_rounds = rounds;
        }
    }
    return best;
}

template <int DT, int BITS, int GS, int MT, int KS, int RG, int GROUP = 1>
static void qmv_go(int batch, QmxStrides sd, int M, int N, int K, const uint32_t* w, const void* s, const void* b,
                   const void* x, void* out, hipStream_t st) {
    const dim3 grid((N + QMV_ROWS * RG - 1) / (QMV_ROWS * RG), (M + MT - 1) / MT, batch);
    hipLaunchKernelGGL((qmv_kernel<DT, BITS, GS, MT, KS, RG, GROUP>), grid, dim3(64 * KS), 0, st, w, s, b, x, out,
                       sd, M, N, K);
}

template <int DT, int BITS, int GS>
static hipError_t qmv_mt(const uint32_t* w, const void* s, const void* b, const void* x, void* out, int batch,
                         QmxStrides sd, int M, int N, int K, int group, hipStream_t st) {
#define QMV_GO(MT_, KS_, RG_) qmv_go<DT, BITS, GS, MT_, KS_, RG_>(batch, sd, M, N, K, w, s, b, x, out, st)
    // grouped gathers: a tile of `group` x rows, one per problem
    if (group == 2) {
        qmv_go<DT, BITS, GS, 2, 1, 1, 2>(batch, sd, M, N, K, w, s, b, x, out, st);
        return hipGetLastError();
    }
    if (group == 4) {
        qmv_go<DT, BITS, GS, 4, 1, 1, 4>(batch, sd, M, N, K, w, s, b, x, out, st);
        return hipGetLastError();
    }
    const int mt = qmv_mt_for(M);
    if constexpr (BITS == 4) {
        const QmvDeep d = qmv_deep_for(M, N, K, BITS, DT, batch, !sd.w_index && !sd.x_index, x, device_cu_count());
        if (d.nr > 0 && qmv_deep_launch<DT, GS>(d, N, K, w, s, b, x, out, st)) return hipGetLastError();
    }
    if (mt == 1) {
        const QmvSplit sp = qmv_split_for(M, (long long)N * batch, K, BITS);
        switch (sp.ks * 8 + sp.rg) {
            case 1 * 8 + 2: QMV_GO(1, 1, 2); break;
            case 1 * 8 + 4: QMV_GO(1, 1, 4); break;
            case 2 * 8 + 1: QMV_GO(1, 2, 1); break;
            case 4 * 8 + 1: QMV_GO(1, 4, 1); break;
            case 5 * 8 + 2: QMV_GO(1, 5, 2); break;
            case 5 * 8 + 4: QMV_GO(1, 5, 4); break;
            default: QMV_GO(1, 1, 1); break;
        }
    } else if (mt == 2) {
        QMV_GO(2, 1, 1);
    } else {
        QMV_GO(4, 1, 1);
    }
#undef QMV_GO
    return hipGetLastError();
}

template <int DT, int BITS>
static hipError_t qmv_gs(const uint32_t* w, const void* s, const void* b, const void* x, void* out, int batch,
                         QmxStrides sd, int M, int N, int K, int gs, int group, hipStream_t st) {
    switch (gs) {
        case 32: return qmv_mt<DT, BITS, 32>(w, s, b, x, out, batch, sd, M, N, K, group, st);
        case 64: return qmv_mt<DT, BITS, 64>(w, s, b, x, out, batch, sd, M, N, K, group, st);
        default: return qmv_mt<DT, BITS, 128>(w, s, b, x, out, batch, sd, M, N, K, group, st);
    }
}

template <int DT>
static hipError_t qmv_bits(const uint32_t* w, const void* s, const void* b, const void* x, void* out, int batch,
                           QmxStrides sd, int M, int N, int K, int bits, int gs, int group, hipStream_t st) {
    switch (bits) {
        case 1: return qmv_gs<DT, 1>(w, s, b, x, out, batch, sd, M, N, K, gs, group, st);
        case 2: return qmv_gs<DT, 2>(w, s, b, x, out, batch, sd, M, N, K, gs, group, st);
        case 3: return qmv_gs<DT, 3>(w, s, b, x, out, batch, sd, M, N, K, gs, group, st);
        case 4: return qmv_gs<DT, 4>(w, s, b, x, out, batch, sd, M, N, K, gs, group, st);
        case 5: return qmv_gs<DT, 5>(w, s, b, x, out, batch, sd, M, N, K, gs, group, st);
        case 6: return qmv_gs<DT, 6>(w, s, b, x, out, batch, sd, M, N, K, gs, group, st);
        default: return qmv_gs<DT, 8>(w, s, b, x, out, batch, sd, M, N, K, gs, group, st);
    }
}

hipError_t launch_qmv(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                      int batch, QmxStrides sd, int M, int N, int K, int bits, int gs, int dt,
                      hipStream_t st, int group) {
    // grouping is defined for single-row gathers only, in tiles of 2 or 4 problems
    if (M != 1 || !sd.w_index || (group != 2 && group != 4)) group = 1;
    switch (dt) {
        case DT_F32: return qmv_bits<DT_F32>(w, s, b, x, out, batch, sd, M, N, K, bits, gs, group, st);
        case DT_F16: return qmv_bits<DT_F16>(w, s, b, x, out, batch, sd, M, N, K, bits, gs, group, st);
        default: return qmv_bits<DT_BF16>(w, s, b, x, out, batch, sd, M, N, K, bits, gs, group, st);
    }
}

// Strided rows -> contiguous rows (for activations whose rows are not 16-byte
// aligned): work-groups stride over the batch*M rows, threads over a row's
// elements, one element each (the source alignment rules out wider loads).
template <int E>
__global__ __launch_bounds__(256) void copy_rows_kernel(const unsigned char* __restrict__ x,
                                                        unsigned char* __restrict__ dst, long long xs,
                                                        long long xr, int M, int K, long long rows) {
    for (long long row = blockIdx.x; row < rows; row += gridDim.x) {
        const long long bz = row / M, m = row - bz * M;
        const unsigned char* src = x + (bz * xs + m * xr) * E;
        unsigned char* d = dst + row * K * E;
        for (int i = threadIdx.x; i < K; i += 256) {
            if constexpr (E == 4) reinterpret_cast<uint32_t*>(d)[i] = reinterpret_cast<const uint32_t*>(src)[i];
            else reinterpret_cast<uint16_t*>(d)[i] = reinterpret_cast<const uint16_t*>(src)[i];
        }
    }
}

hipError_t launch_copy_rows(const void* x, void* dst, int batch, long long xs, long long xr, int M, int K,
                            int elem, hipStream_t st) {
    const long long rows = (long long)batch * M;
    const dim3 grid((unsigned)(rows < 8192 ? rows : 8192));
    if (elem == 4)
        hipLaunchKernelGGL(copy_rows_kernel<4>, grid, dim3(256), 0, st, static_cast<const unsigned char*>(x),
                           static_cast<unsigned char*>(dst), xs, xr, M, K, rows);
    else
        hipLaunchKernelGGL(copy_rows_kernel<2>, grid, dim3(256), 0, st, static_cast<const unsigned char*>(x),
                           static_cast<unsigned char*>(dst), xs, xr, M, K, rows);
    return hipGetLastError();
}

}  // namespace qmx
