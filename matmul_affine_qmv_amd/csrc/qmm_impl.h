// qmm_impl.h -- the staged affine quantized x * W^T kernel on the gfx950
// matrix cores (M >= 8, and M = 2..7 for large weights).  Included once per
// code width by qmm_b{1,2,3,4,5,6,8}.hip.
//
// Method (page "mlx PR 4682"): transposed affine qmm in which the next K
// steps' packed weights, scales/biases and activations are fetched while the
// current step is consumed from threadgroup memory, with one barrier per K
// step; split-K writes float32 partials that a separate kernel sums.
//
// gfx950 mapping:
// * A work-group of 8 waves owns an output tile of BM = 16*MT rows of x by
//   BN = 128 columns of W and a range of 128-column K blocks (4 MFMA k-steps
//   each).  Waves 0-3 each own 2 fragments of 16 columns and take k-steps
//   0-1 of every block; waves 4-7 own the same columns and take k-steps 2-3.
//   The two halves add their float32 tiles through LDS once at the end.
//   Narrower tiles regroup the same 8 waves along K (WK groups): 64-column
//   tiles over 256-column blocks (WK = 4, split-K partials) and 32- or
//   16-column tiles over 512-column blocks (WK = 8, unsplit).
// * A split-K partition covers whole segments of K: 256 columns when K is a
//   multiple of 256, else 128, the same segments on every tile width.
// * Every operand of a K block (x rows, packed W rows, raw 16-bit scales and
//   biases) is copied from HBM straight into an LDS stage by the global-to-LDS
//   form of the load (no register staging, no conversion on the way in),
//   through a ring of NS stages: NS - 1 blocks are in flight while one is
//   consumed.  Each thread issues the same number of copies per stage, so a
//   single wait on the per-wave memory counter plus one barrier per block
//   makes a stage visible to the whole work-group.
// * The copies land at consecutive LDS slots per lane; bank conflicts on the
//   MFMA operand reads are avoided by choosing which global chunk each lane
//   fetches (an XOR swizzle of the chunk index by the row), not by padding.
// * Codes are expanded in registers right before the MFMA into exact 16-bit
//   integers in natural k order: fields are split into bytes, interleaved,
//   and one v_perm per pair of codes sets a magic exponent byte above each
//   (0x43qq is the bf16 value 128 + q, 0x64qq the f16 value 1024 + q).  For
//   1, 3, 5 and 6 bits a lane's 8 codes are a byte-aligned field of BITS
//   bytes, cut pair by pair from a two-word window.  f16 pairs then drop the
//   1024 with one exact packed f16 subtraction; for bf16 the constant offset
//   128*sum(x) is removed in the group epilogue.
// * MFMA v_mfma_f32_16x16x32_{bf16,f16}: A = x fragment (16 rows of M),
//   B = W codes (16 columns of N).  A group of GS codes is GS/32 k-steps
//   accumulated into a fresh float32 tile; the same A fragments against an
//   all-ones B give the group's row sums of x in a matching tile, and the
//   epilogue adds scale * (tile) + (bias - OFF*scale) * (row sums) in
//   float32.  Scale and bias are used exactly as stored, so the output's
//   only roundings are float32 accumulation and the final store.
// * Work-groups are numbered so that the ones sharing a K range (and so the
//   same x slice) are dispatched to the same XCD and share its L2.
// * A batch of problems of one shape is the second grid dimension: each
//   work-group offsets its operand pointers by its problem's strides (or by
//   the matrices an index array picks) before anything else.
#pragma once

#include "qmx_device.h"
#include "qmx_internal.h"

namespace qmx {

// WK: groups of waves along K.  Each of the 8 waves takes two k-steps (64
// columns) of every K block, so a block is KB = 64 * WK columns, and the
// 8 / WK waves of one group own NB fragments of 16 columns each: WK = 2 is the
// 128-column tile, WK = 4 a 64-column tile of 256-column K blocks (split-K with
// half the partitions of the 128-column plan), WK = 8 a 32-column (NB = 2) or
// 16-column (NB = 1) tile for narrow problems (more work-groups from few
// columns, every K group summed in the work-group).
template <int DT, int BITS, int GS, int MT, bool SBV, int WK = 2, int NBT = QMM_NB>
struct QmmCfg {
    static constexpr int BM = 16 * MT;
    static constexpr int WN = 8 / WK;                         // waves along N
    static constexpr int NB = NBT;                            // 16-column fragments per wave
    static constexpr int BN = WN * NB * 16;                   // columns per tile
    static constexpr int KB = 64 * WK;                        // columns per K block
    static constexpr int GPB = KB / GS;                       // groups per K block
    static constexpr int KS = GS / 32;                        // MFMA k-steps per group
    // x: rows of KB 16-bit values (XRB bytes); each wave-wide 16-byte copy fills
    // 1 KB = XRPC rows.
    static constexpr int XRB = 2 * KB;
    static constexpr int XRPC = 1024 / XRB;
    static constexpr int XPT = (BM + 8 * XRPC - 1) / (8 * XRPC);   // x copies per thread per block
    static constexpr int XROWS = 8 * XRPC * XPT;
    static constexpr int X_BYTES = XROWS * XRB;
    // W: 16*BITS bytes per row per block.  1- and 2-bit rows are copied 4
    // bytes per lane (one and two copies per thread), the others 16 bytes per
    // lane.  For 3, 5 and 6 bits (fields may straddle words) the 128*BITS
    // pieces are not a whole number of copies per thread: the spare copies
    // repeat pieces already covered, writing the same bytes to the same place,
    // so that every wave still issues the same number of copies.
    static constexpr bool ODD = !(BITS == 2 || BITS == 4 || BITS == 8);
    static constexpr bool W4B = BITS == 1 || BITS == 2;       // 4-byte W copies
    static constexpr bool WREP = ODD && !W4B;                 // 16-byte copies with repeats
    static constexpr int W_ROW = KB * BITS / 8;
    static constexpr int W_BYTES = BN * W_ROW;
    // copy slots per W row: 4-byte words for 1- and 2-bit codes, else 16-byte pieces
    static constexpr int W_SLOTS = W4B ? W_ROW / 4 : W_ROW / 16;
    static constexpr int W_PIECES = W_BYTES / 16;
    // wave-wide W copies per stage (2, 4, 8 bits); fewer than 8 (16-column tiles of
    // 4-bit codes) are made by waves 0 .. W_WAVES - 1 only
    static constexpr int W_WCOPIES = W_BYTES / (64 * (W4B ? 4 : 16));
    static constexpr int W_WAVES = (WREP || BITS == 1 || W_WCOPIES >= 8) ? 8 : W_WCOPIES;
    static constexpr int WPT = W4B && BITS == 1 ? W_BYTES / (4 * QMM_THREADS)
                             : WREP ? (W_PIECES + QMM_THREADS - 1) / QMM_THREADS
                             : (W_WCOPIES + 7) / 8;
    // Scales then biases.  Staged per block, one 16-bit value per lane
    // (zero-extended to 4 bytes in LDS), unless SBV: then the work-group's whole
    // K range of both is copied once, before the ring, in 16-byte chunks.
    static constexpr int SB_VALUES = 2 * BN * GPB;
    static constexpr int SBPT = SBV ? 0 : (SB_VALUES + QMM_THREADS - 1) / QMM_THREADS;
    static constexpr int SB_BYTES = SBPT * QMM_THREADS * 4;
    static constexpr int STAGE = X_BYTES + W_BYTES + SB_BYTES;
    // ring depth: up to 4 stages, leaving SBV at least 12 KB for its chunks; the
    // 64-column tiles (split partitions twice as long as on 128-column tiles)
    // leave room for 12 chunks where three stages still fit
    static constexpr int RING_W4 = 160 * 1024 - 12 * 2 * BN * 16;
    static constexpr int RING_LDS = (SBV && WK == 4 && RING_W4 / STAGE >= 3) ? RING_W4
                                  : 160 * 1024 - (SBV ? 12 * 1024 : 0);
    static constexpr int NS = RING_LDS / STAGE < 4 ? RING_LDS / STAGE : 4;
    static constexpr int LPS = XPT + WPT + SBPT;              // copies per thread per stage
    static constexpr int LPS_NW = XPT + SBPT;                 // ... in waves that copy no W
    // SBV: 16-byte chunks (8 groups) per (scale/bias, column) held in LDS
    static constexpr int SBV_CHUNKS = SBV ? ((160 * 1024 - NS * STAGE) / (2 * BN * 16) > 15
                                                 ? 15 : (160 * 1024 - NS * STAGE) / (2 * BN * 16))
                                          : 0;
    static constexpr int SBV_BYTES = SBV_CHUNKS * 2 * BN * 16;
    static constexpr bool CVT8 = DT == DT_BF16 && BITS == 8;  // 128 + q is not exact in bf16
    // Offset the expanded bf16 codes carry: 128 + q (q < 128); 8-bit bf16 codes are
    // converted instead, and f16 codes have their 1024 removed exactly before the MFMA.
    static constexpr float OFF = (CVT8 || DT == DT_F16) ? 0.f : 128.f;
    static constexpr int RED_FLOATS = WN * MT * NB * 4 * 64;   // one K group's tiles
    static constexpr int RED_BYTES = (WK - 1) * RED_FLOATS * 4;
    // every K group's tiles fit the stages at once: the end sum is shared by all waves
    static constexpr bool RED_ALL = WK * RED_FLOATS * 4 <= NS * STAGE && (WN * MT * NB * 4) % 8 == 0;
    static_assert(WK == 2 || ((WK == 4 || WK == 8) && (BITS == 2 || BITS == 4 || BITS == 8)), "64- and 32/16-column tiles: 2, 4, 8 bits");
    static_assert(NS >= 3, "at least two stages in flight");
    static_assert(RED_BYTES <= NS * STAGE, "end reduction reuses the stages");
    static_assert(LPS * (NS - 2) < 64, "memory counter range");
    static_assert(STAGE % 1024 == 0 && X_BYTES % 1024 == 0, "stage alignment");
    static_assert(WREP ? W_PIECES % 64 == 0 && WPT * QMM_THREADS >= W_PIECES
                       : WPT * W_WAVES * 64 * (W4B ? 4 : 16) == W_BYTES, "W copies per thread");
    static_assert(NB == QMM_NB || (WK == 8 && NB == 1 && !WREP && BITS != 1), "16-column tiles: narrow, 2/4/8 bits");
    static_assert(!SBV || SBV_CHUNKS >= 3, "room for the staged scales and biases");
};

// Largest chunk count the staged scale/bias copy of one work-group may need.
template <int DT, int BITS, int GS, int MT, int WK = 2, int NBT = QMM_NB>
constexpr int qmm_sbv_chunks() { return QmmCfg<DT, BITS, GS, MT, true, WK, NBT>::SBV_CHUNKS; }

// Bank spread of 2-, 4- and 8-bit W rows of SLOTS copy slots: slot p of row R
// holds piece (or word) p ^ w_swz(R) of the row.  Rows of 4 or 8 16-byte slots
// (64 or 128 bytes) XOR the row bits above the ones that already separate the
// banks of a fragment's 16 rows (2 and 1 of them), so that those rows read
// distinct banks; rows of 16 or more slots the low 4 bits of the row.
template <int BITS, int SLOTS>
__device__ __forceinline__ int w_swz(int R) {
    if constexpr (SLOTS >= 16) return R & 15;
    else if constexpr (BITS == 4) return SLOTS == 8 ? (R >> 1) & 7 : (R >> 2) & 3;
    else if constexpr (BITS == 8) return (R >> 1) & 7;
    else return (R >> 3) & 7;
}

// 8-value chunk of the K block that lane group g feeds at k-step s.
// Each step's 32 values lie inside one group of GS.  2-bit codes with GS >= 64
// pair steps so that a lane's two steps are the two halves of one W word.
template <int BITS, int GS>
__device__ __forceinline__ constexpr int kchunk(int s, int g) {
    if constexpr (BITS == 2 && GS >= 64)
        return 8 * (s / 2) + 2 * g + (s % 2);
    else
        return 4 * s + g;
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// v_perm selector: byte i of the low source, then the magic byte (byte 0 of
// the high source), then byte j, then the magic byte again.
__device__ constexpr uint32_t perm_sel(int i, int j) {
    return (uint32_t)i | (4u << 8) | ((uint32_t)j << 16) | (4u << 24);
}

// f16 pairs 1024 + q -> q, exactly (packed f16 subtraction).  Keeping the
// offset would leave s * 1024 * sum(x) to cancel against the bias term in
// float32, costing about ten bits of the group partial's precision.
__device__ __forceinline__ uint32_t drop1024(uint32_t v) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 r = __builtin_bit_cast(h2, v) - h2{(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, r);
}

template <int DT>
__device__ __forceinline__ u32x4 finish(u32x4 r) {
    if constexpr (DT == DT_F16) return u32x4{drop1024(r.x), drop1024(r.y), drop1024(r.z), drop1024(r.w)};
    else return r;
}

// Eight byte-held codes (bytes of e = c0 c1 c4 c5 and f = c2 c3 c6 c7) as
// four pairs of 16-bit MFMA operands in natural order.
template <int DT>
__device__ __forceinline__ u32x4 magic_pairs(uint32_t e, uint32_t f) {
    constexpr uint32_t MB = DT == DT_F16 ? 0x64646464u : 0x43434343u;
    return finish<DT>(u32x4{__builtin_amdgcn_perm(MB, e, perm_sel(0, 1)), __builtin_amdgcn_perm(MB, f, perm_sel(0, 1)),
                            __builtin_amdgcn_perm(MB, e, perm_sel(2, 3)), __builtin_amdgcn_perm(MB, f, perm_sel(2, 3))});
}

// 8 consecutive 4-bit codes of one word (code i at bits 4i).
template <int DT>
__device__ __forceinline__ u32x4 expand4(uint32_t w) {
    const uint32_t lo = w & 0x0f0f0f0fu;          // c0 c2 c4 c6
    const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;   // c1 c3 c5 c7
    const uint32_t c0123 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    const uint32_t c4567 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    constexpr uint32_t MB = DT == DT_F16 ? 0x64646464u : 0x43434343u;
    return finish<DT>(u32x4{__builtin_amdgcn_perm(MB, c0123, perm_sel(0, 1)), __builtin_amdgcn_perm(MB, c0123, perm_sel(2, 3)),
                            __builtin_amdgcn_perm(MB, c4567, perm_sel(0, 1)), __builtin_amdgcn_perm(MB, c4567, perm_sel(2, 3))});
}

// 8 consecutive codes of a 1-, 3-, 5- or 6-bit stream: they fill exactly BITS
// bytes, starting at byte sh (0..3) of word lo (hi the next word).  One byte
// shift brings them to bit 0; each pair is cut as one 2*BITS-bit window t,
// and t | t << (16 - BITS) puts its second code at bit 16 under the magic
// bytes.
template <int DT, int BITS>
__device__ __forceinline__ u32x4 expand_stream(uint32_t lo, uint32_t hi, int sh) {
    const uint32_t MB = magic_bytes<DT>();
    constexpr uint32_t MASK = (1u << BITS) - 1u, WIN = (1u << (2 * BITS)) - 1u;
    uint32_t p[4];
    if constexpr (8 * BITS <= 32) {
        const uint32_t u = __builtin_amdgcn_alignbyte(hi, lo, sh);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t t = (u >> (2 * BITS * j)) & WIN;
            p[j] = (((t << (16 - BITS)) | t) & (MASK | (MASK << 16))) | MB;
        }
    } else {
        // 40 or 48 bits: the low and high 32-bit halves of the shifted window
        const uint32_t u0 = __builtin_amdgcn_alignbyte(hi, lo, sh);
        const uint32_t u1 = __builtin_amdgcn_alignbyte(0u, hi, sh);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 2 * BITS * j;
            const uint32_t t = (b + 2 * BITS <= 32 ? u0 >> b : b >= 32 ? u1 >> (b - 32)
                                                             : __builtin_amdgcn_alignbit(u1, u0, b)) & WIN;
            p[j] = (((t << (16 - BITS)) | t) & (MASK | (MASK << 16))) | MB;
        }
    }
    return finish<DT>(u32x4{p[0], p[1], p[2], p[3]});
}

// 8 consecutive 2-bit codes held in the low 16 bits of h (code i at bits 2i).
template <int DT>
__device__ __forceinline__ u32x4 expand2(uint32_t h) {
    const uint32_t a = h & 0x0303u, b = (h >> 2) & 0x0303u;          // c0 c4, c1 c5
    const uint32_t c = (h >> 4) & 0x0303u, d = (h >> 6) & 0x0303u;   // c2 c6, c3 c7
    return magic_pairs<DT>(__builtin_amdgcn_perm(b, a, 0x05010400u), __builtin_amdgcn_perm(d, c, 0x05010400u));
}

// 8 consecutive 8-bit codes of two words.
template <int DT>
__device__ __forceinline__ u32x4 expand8(uint32_t w0, uint32_t w1) {
    if constexpr (DT == DT_F16) {
        constexpr uint32_t MB = 0x64646464u;
        return finish<DT>(u32x4{__builtin_amdgcn_perm(MB, w0, perm_sel(0, 1)), __builtin_amdgcn_perm(MB, w0, perm_sel(2, 3)),
                                __builtin_amdgcn_perm(MB, w1, perm_sel(0, 1)), __builtin_amdgcn_perm(MB, w1, perm_sel(2, 3))});
    } else {
        // bf16 holds every integer up to 256 exactly: convert, keep the upper halves.
        auto pair = [](uint32_t a, uint32_t b) {
            return __builtin_amdgcn_perm(__float_as_uint((float)b), __float_as_uint((float)a), 0x07060302u);
        };
        return u32x4{pair(w0 & 0xffu, (w0 >> 8) & 0xffu), pair((w0 >> 16) & 0xffu, w0 >> 24),
                     pair(w1 & 0xffu, (w1 >> 8) & 0xffu), pair((w1 >> 16) & 0xffu, w1 >> 24)};
    }
}

// Copy BYTES (2, 4 or 16) per lane from g into LDS at the wave-uniform address
// l: lane i's data lands at l + 16 * i for 16-byte copies and at l + 4 * i
// (zero-extended) for the smaller ones.
template <int BYTES>
__device__ __forceinline__ void dma(const void* g, unsigned char* l) {
    if constexpr (BYTES == 16)
        __builtin_amdgcn_global_load_lds(g, reinterpret_cast<void*>(l), 16, 0, 0);
    else if constexpr (BYTES == 4)
        __builtin_amdgcn_global_load_lds(g, reinterpret_cast<void*>(l), 4, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(g, reinterpret_cast<void*>(l), 2, 0, 0);
}

// Wait until at most N of this wave's copies are in flight and its LDS reads
// are done, then meet the other waves.  The memory clobber keeps the
// compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int DT, int BITS, int GS, int MT, bool SPLIT, bool SBV, int WK, int NBT>
__global__ __launch_bounds__(QMM_THREADS) void qmm_t_kernel(
    const uint32_t* __restrict__ w, const void* __restrict__ scales, const void* __restrict__ biases,
    const void* __restrict__ x, void* __restrict__ out, float* __restrict__ ws, QmxStrides sd,
    int M, int N, int K, int splits, int ntiles, int mtiles, int total_tiles, int per_xcd) {
    using C = QmmCfg<DT, BITS, GS, MT, SBV, WK, NBT>;
    // problem blockIdx.y of the batch (16-bit x, scales, biases and out)
    const long long bz = blockIdx.y, wz = qmx_w_matrix(sd, bz), xz = qmx_x_matrix(sd, bz);
    w += wz * sd.w;
    scales = static_cast<const uint16_t*>(scales) + wz * sd.sb;
    biases = static_cast<const uint16_t*>(biases) + wz * sd.sb;
    x = static_cast<const uint16_t*>(x) + xz * sd.x;
    if constexpr (!SPLIT) out = static_cast<uint16_t*>(out) + bz * M * (long long)N;
    const long long XR = sd.x_row;
    constexpr int NB = C::NB;
    constexpr int NS = C::NS;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * C::STAGE + C::SBV_BYTES];

    // Hardware block h runs on XCD h % 8; give each XCD a contiguous range of tiles.
    const int h = blockIdx.x;
    const int L = (h & 7) * per_xcd + (h >> 3);
    if (L >= total_tiles) return;
    // unsigned 32-bit divisions throughout: every value is non-negative, and
    // split * nkb < 2^31 (split < 16 and nkb <= K / 128)
    const int ntile = (int)((unsigned)L % (unsigned)ntiles);
    const int rest = (int)((unsigned)L / (unsigned)ntiles);
    const int mtile = (int)((unsigned)rest % (unsigned)mtiles);
    const int split = (int)((unsigned)rest / (unsigned)mtiles);
    const int n0 = ntile * C::BN, m0 = mtile * C::BM;
    // K partitions in segments of 256 columns (128 when K is not a multiple of
    // 256), whatever the block size: partition p covers segments
    // [floor(p * nseg / splits), floor((p + 1) * nseg / splits))
    const int seg = (K & 255) == 0 ? 256 : 128, nseg = K / seg;
    const int kb0 = (int)((unsigned)(split * nseg) / (unsigned)splits) * seg / C::KB;
    const int kb1 = (int)((unsigned)((split + 1) * nseg) / (unsigned)splits) * seg / C::KB;
    const int nk = kb1 - kb0;
    const int G = K / GS;
    const size_t row_words = (size_t)K * BITS / 32;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & (C::WN - 1);   // column slice of this wave
    const int wk = wave / C::WN;          // k-step pair of this wave: steps 2wk, 2wk+1 of each block
    const int lrow = lane & 15, lgrp = lane >> 4;

    // ---- per-thread sources of the stage copies at block 0 (block kb adds a fixed stride)
    // x: copy i of this thread fills row r = XRPC*(8i + wave) + lane/(64/XRPC) of the
    // stage at 16-byte slot lane%(64/XRPC), with chunk slot ^ (r & 15) of that row of x.
    const uint16_t* xsrc[C::XPT];
#pragma unroll
    for (int i = 0; i < C::XPT; ++i) {
        const int r = C::XRPC * (8 * i + wave) + lane / (64 / C::XRPC);
        const int c = (lane % (64 / C::XRPC)) ^ (r & 15);
        xsrc[i] = static_cast<const uint16_t*>(x) + min(m0 + r, M - 1) * XR + 8 * c;
    }
    // W: tile rows R in 16-byte chunks (4-byte words for 2-bit codes); the chunk a
    // slot holds is its index XOR a few bits of R, so B-operand reads spread over banks.
    const uint32_t* wsrc[C::WPT];
#pragma unroll
    for (int j = 0; j < C::WPT; ++j) {
        int R, q;
        if constexpr (BITS == 1) {
            // word v = 512j + tid of the block, row-major [R][4] in LDS
            const int v = QMM_THREADS * j + tid;
            R = v / 4;
            q = v % 4;
        } else if constexpr (C::WREP) {
            // 16-byte piece v of the block (row v / BITS, piece v % BITS of the row)
            const int v = (QMM_THREADS * j + tid) % C::W_PIECES;
            R = v / BITS;
            q = 4 * (v % BITS);
        } else {
            // 2, 4, 8 bits: copy j of the wave fills 64 / W_SLOTS whole rows, lane l
            // slot l % W_SLOTS of its row, with the piece (or word) the slot holds
            constexpr int SL = C::W_SLOTS;
            R = (64 / SL) * (8 * j + wave) + lane / SL;
            const int piece = (lane % SL) ^ w_swz<BITS, SL>(R);
            q = C::W4B ? piece : 4 * piece;
        }
        wsrc[j] = w + (size_t)min(n0 + R, N - 1) * row_words + q;
    }
    // SBV: the K range's scales and biases as 16-byte chunks of 8 groups, chunk
    // sb_c0 + c of every column at LDS slot (which*BN + col)*sb_nch + c.  An odd slot
    // stride keeps the 16 columns a wave reads on distinct banks.
    // When the range has an even chunk count, one more slot per column repeats its
    // last chunk, so that the slot stride is odd.
    int sb_c0 = 0, sb_nch = 0, sb_last = 0;
    if constexpr (SBV) {
        if (nk > 0) {
            sb_c0 = (kb0 * C::GPB) / 8;
            sb_last = (kb1 * C::GPB + 7) / 8 - 1 - sb_c0;
            sb_nch = (sb_last + 1) | 1;
        }
    }
    // scales/biases: value v = 512j + tid (modulo the value count) is the scale (then
    // the bias) of column (v % (BN*GPB)) / GPB, group v % GPB, and lands at LDS word v.
    const uint16_t* sbsrc[C::SBPT > 0 ? C::SBPT : 1];
#pragma unroll
    for (int j = 0; j < C::SBPT; ++j) {
        const int v = (QMM_THREADS * j + tid) % C::SB_VALUES;
        const int which = v / (C::BN * C::GPB);
        const int rem = v % (C::BN * C::GPB);
        const int col = rem / C::GPB, g = rem % C::GPB;
        sbsrc[j] = static_cast<const uint16_t*>(which ? biases : scales) + (size_t)min(n0 + col, N - 1) * G + g;
    }

    auto stage_load = [&](int kb, int buf) {
        unsigned char* X = smem + buf * C::STAGE;
        unsigned char* Wl = X + C::X_BYTES;
        unsigned char* SB = Wl + C::W_BYTES;
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) dma<16>(xsrc[i] + (size_t)kb * C::KB, X + (8 * i + wave) * 1024);
#pragma unroll
        for (int j = 0; j < C::WPT; ++j) {
            if (C::W_WAVES < 8 && wave >= C::W_WAVES) continue;   // wave-uniform
            if constexpr (C::W4B)
                dma<4>(wsrc[j] + (size_t)kb * (C::W_ROW / 4), Wl + (8 * j + wave) * 256);
            else if constexpr (C::WREP)
                dma<16>(wsrc[j] + (size_t)kb * (C::W_ROW / 4), Wl + ((8 * j + wave) * 1024) % C::W_BYTES);
            else
                dma<16>(wsrc[j] + (size_t)kb * (C::W_ROW / 4), Wl + (8 * j + wave) * 1024);
        }
#pragma unroll
        for (int j = 0; j < C::SBPT; ++j)
            dma<2>(sbsrc[j] + (size_t)kb * C::GPB, SB + (QMM_THREADS * j + 64 * wave) * 4);
    };

    f32x4 run[MT][NB];
#pragma unroll
    for (int mf = 0; mf < MT; ++mf)
#pragma unroll
        for (int nf = 0; nf < NB; ++nf) run[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr uint32_t ONE2 = DT == DT_F16 ? 0x3c003c00u : 0x3f803f80u;
    const u32x4 ones = u32x4{ONE2, ONE2, ONE2, ONE2};

    auto compute = [&](int buf, int kb) {
        const unsigned char* X = smem + buf * C::STAGE;
        const unsigned char* Wl = X + C::X_BYTES;
        const uint32_t* SB = reinterpret_cast<const uint32_t*>(Wl + C::W_BYTES);
        const uint16_t* SBVl = reinterpret_cast<const uint16_t*>(smem + NS * C::STAGE);
        // expand this wave's two k-steps of codes
        u32x4 bf[2][NB];
#pragma unroll
        for (int nf = 0; nf < NB; ++nf) {
            const int R = wn * (NB * 16) + nf * 16 + lrow;
            if constexpr (BITS == 2 && GS >= 64) {
                const int c = kchunk<BITS, GS>(2 * wk, lgrp);   // both steps share word c / 2
                const uint32_t word = *reinterpret_cast<const uint32_t*>(
                    Wl + R * C::W_ROW + (((c >> 1) ^ w_swz<BITS, C::W_SLOTS>(R)) << 2));
                bf[0][nf] = expand2<DT>(word & 0xffffu);
                bf[1][nf] = expand2<DT>(word >> 16);
            } else {
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int c = kchunk<BITS, GS>(2 * wk + st, lgrp);
                    if constexpr (C::ODD) {
                        // chunk c's 8 codes are bytes [BITS*c, BITS*c + BITS) of the row's
                        // block; the word after them may lie past the row (BITS = 1, 3), but
                        // stays inside the LDS allocation and is then not used
                        const int o = BITS * c;
                        const uint32_t* rw = reinterpret_cast<const uint32_t*>(Wl + R * C::W_ROW);
                        bf[st][nf] = expand_stream<DT, BITS>(rw[o >> 2], BITS > 1 ? rw[(o >> 2) + 1] : 0u, o & 3);
                    } else if constexpr (BITS == 4) {
                        const uint32_t word = *reinterpret_cast<const uint32_t*>(
                            Wl + R * C::W_ROW + (((c >> 2) ^ w_swz<BITS, C::W_SLOTS>(R)) << 4) + 4 * (c & 3));
                        bf[st][nf] = expand4<DT>(word);
                    } else if constexpr (BITS == 8) {
                        const u32x2 wv = *reinterpret_cast<const u32x2*>(
                            Wl + R * C::W_ROW + (((c >> 1) ^ w_swz<BITS, C::W_SLOTS>(R)) << 4) + 8 * (c & 1));
                        bf[st][nf] = expand8<DT>(wv.x, wv.y);
                    } else {
                        const uint32_t word = *reinterpret_cast<const uint32_t*>(
                            Wl + R * C::W_ROW + (((c >> 1) ^ w_swz<BITS, C::W_SLOTS>(R)) << 2));
                        bf[st][nf] = expand2<DT>((word >> (16 * (c & 1))) & 0xffffu);
                    }
                }
            }
        }
        // the two k-steps share one group unless a group is a single k-step
        constexpr int NG = C::KS >= 2 ? 1 : 2;
        float sv[NG][NB], bv[NG][NB];
#pragma unroll
        for (int gp = 0; gp < NG; ++gp) {
            const int g = (32 * (2 * wk + gp)) / GS;
#pragma unroll
            for (int nf = 0; nf < NB; ++nf) {
                const int col = wn * (NB * 16) + nf * 16 + lrow;
                uint32_t sr, br;
                if constexpr (SBV) {
                    const int ga = kb * C::GPB + g;                   // group index within the row
                    const int at = (col * sb_nch + (ga >> 3) - sb_c0) * 8 + (ga & 7);
                    sr = SBVl[at];
                    br = SBVl[C::BN * sb_nch * 8 + at];
                } else {
                    sr = SB[col * C::GPB + g];
                    br = SB[C::BN * C::GPB + col * C::GPB + g];
                }
                const float s = DT == DT_F16 ? f16_bits_to_f32(sr) : bf16_bits_to_f32(sr);
                const float b = DT == DT_F16 ? f16_bits_to_f32(br) : bf16_bits_to_f32(br);
                sv[gp][nf] = s;
                bv[gp][nf] = fmaf(-C::OFF, s, b);
            }
        }
        const int c0 = kchunk<BITS, GS>(2 * wk, lgrp), c1 = kchunk<BITS, GS>(2 * wk + 1, lgrp);
        if constexpr (NG == 1) {
            // One group per block and wave: every MFMA of the block first (the group
            // tiles, and the row sums of x as one more MFMA against ones), then the
            // float32 epilogue, so the two waves that share a SIMD spend less of the
            // block issuing the same kind of work at once (measured 1-2% faster).
            f32x4 gacc[MT][NB], gxs[MT];
#pragma unroll
            for (int mf = 0; mf < MT; ++mf) {
                const int r = mf * 16 + lrow;
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(X + r * C::XRB + ((c0 ^ (r & 15)) << 4));
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(X + r * C::XRB + ((c1 ^ (r & 15)) << 4));
#pragma unroll
                for (int nf = 0; nf < NB; ++nf) {
                    gacc[mf][nf] = mfma16x16x32<DT>(a0, bf[0][nf], f32x4{0.f, 0.f, 0.f, 0.f});
                    gacc[mf][nf] = mfma16x16x32<DT>(a1, bf[1][nf], gacc[mf][nf]);
                }
                gxs[mf] = mfma16x16x32<DT>(a0, ones, f32x4{0.f, 0.f, 0.f, 0.f});
                gxs[mf] = mfma16x16x32<DT>(a1, ones, gxs[mf]);
            }
#pragma unroll
            for (int mf = 0; mf < MT; ++mf)
#pragma unroll
                for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        run[mf][nf][v] = fmaf(sv[0][nf], gacc[mf][nf][v], fmaf(bv[0][nf], gxs[mf][v], run[mf][nf][v]));
            return;
        }
        // two groups per block and wave (GS = 32): one 16-row fragment of x at a
        // time keeps one row of group tiles live
#pragma unroll
        for (int mf = 0; mf < MT; ++mf) {
            const int r = mf * 16 + lrow;
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(X + r * C::XRB + ((c0 ^ (r & 15)) << 4));
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(X + r * C::XRB + ((c1 ^ (r & 15)) << 4));
#pragma unroll
            for (int gp = 0; gp < NG; ++gp) {
                f32x4 gacc[NB];
#pragma unroll
                for (int nf = 0; nf < NB; ++nf)
                    gacc[nf] = mfma16x16x32<DT>(gp ? a1 : a0, bf[gp][nf], f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 gxs = mfma16x16x32<DT>(gp ? a1 : a0, ones, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        run[mf][nf][v] = fmaf(sv[gp][nf], gacc[nf][v], fmaf(bv[gp][nf], gxs[v], run[mf][nf][v]));
            }
        }
    };

    // Ring of NS stages: block i lives in stage i % NS.  Before consuming block i
    // every thread waits for its own copies of block i (the copies of the NS - 2
    // later blocks may still be in flight; near the end, where fewer were issued,
    // it waits for all), and the barrier publishes them.  The copies of block
    // i + NS - 1 then go into the stage that block i - 1 used, which every wave
    // finished reading before the barrier.
    if constexpr (SBV) {
        // one copy per (scale/bias, column, chunk), lane v at LDS slot v; issued before
        // the ring so that the first stage's wait also covers them (copies of a wave
        // complete in order)
        const int lanes = 2 * C::BN * sb_nch;
        unsigned char* base = smem + NS * C::STAGE;
        for (int j = 0; j * QMM_THREADS < lanes; ++j) {
            const int v = QMM_THREADS * j + tid;
            if (v < lanes) {
                const int which = (int)((unsigned)v / (unsigned)(C::BN * sb_nch));
                const int rem = v - which * (C::BN * sb_nch);
                const int col = (int)((unsigned)rem / (unsigned)sb_nch), ch = rem - col * sb_nch;
                const uint16_t* src = static_cast<const uint16_t*>(which ? biases : scales) +
                                      (size_t)min(n0 + col, N - 1) * G + 8 * (sb_c0 + min(ch, sb_last));
                dma<16>(src, base + (QMM_THREADS * j + 64 * wave) * 16);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nk) stage_load(kb0 + p, p);
    // unrolled by NS so that every stage address is a constant
    for (int base = 0; base < nk; base += NS) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int i = base + j;
            if (i < nk) {
                if (i + NS - 2 < nk) {
                    if (C::W_WAVES == 8 || wave < C::W_WAVES)
                        stage_barrier<C::LPS * (NS - 2)>();
                    else
                        stage_barrier<C::LPS_NW * (NS - 2)>();
                } else {
                    stage_barrier<0>();
                }
                if (i + NS - 1 < nk) stage_load(kb0 + i + NS - 1, (j + NS - 1) % NS);
                compute(j, kb0 + i);
            }
        }
    }
    stage_barrier<0>();

    // add the K groups' tiles in ascending group order, then store
    float* red = reinterpret_cast<float*>(smem);
    if constexpr (C::RED_ALL) {
        // every wave leaves its tiles in LDS; wave v then sums the values e = v,
        // v + 8, ... of one group's tiles (value e of lane l at red[e * 64 + l],
        // e = ((wn * MT + mf) * NB + nf) * 4 + v4) over the groups and stores them
        constexpr int E = C::WN * MT * NB * 4;
        static_assert(E % 8 == 0, "whole values per wave");
#pragma unroll
        for (int mf = 0; mf < MT; ++mf)
#pragma unroll
            for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[wk * C::RED_FLOATS + (((wn * MT + mf) * NB + nf) * 4 + v) * 64 + lane] = run[mf][nf][v];
        stage_barrier<0>();
        float sum[E / 8];
#pragma unroll
        for (int t = 0; t < E / 8; ++t) {
            const int e = 8 * t + wave;
            sum[t] = red[e * 64 + lane];
#pragma unroll
            for (int g = 1; g < WK; ++g) sum[t] += red[g * C::RED_FLOATS + e * 64 + lane];
        }
#pragma unroll
        for (int t = 0; t < E / 8; ++t) {
            const int e = 8 * t + wave;
            const int v = e & 3, nf = (e >> 2) % NB, mf = (e / (4 * NB)) % MT, wv = e / (4 * NB * MT);
            const int m = m0 + mf * 16 + 4 * lgrp + v;
            const int n = n0 + wv * (NB * 16) + nf * 16 + lrow;
            if (m < M && n < N) {
                if constexpr (SPLIT)
                    ws[(((size_t)split * gridDim.y + bz) * M + m) * N + n] = sum[t];
                else
                    store_elem<DT>(out, (size_t)m * N + n, sum[t]);
            }
        }
        return;
    }
    if (wk > 0) {
#pragma unroll
        for (int mf = 0; mf < MT; ++mf)
#pragma unroll
            for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[(wk - 1) * C::RED_FLOATS + (((wn * MT + mf) * NB + nf) * 4 + v) * 64 + lane] = run[mf][nf][v];
    }
    stage_barrier<0>();
    if (wk > 0) return;
    // every partner value is read before the first store, so the LDS reads share
    // one wait instead of one each in front of every (row-predicated) store
#pragma unroll
    for (int g = 1; g < WK; ++g)
#pragma unroll
        for (int mf = 0; mf < MT; ++mf)
#pragma unroll
            for (int nf = 0; nf < NB; ++nf)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    run[mf][nf][v] += red[(g - 1) * C::RED_FLOATS + (((wn * MT + mf) * NB + nf) * 4 + v) * 64 + lane];
    const int nl = n0 + wn * (NB * 16) + lrow;   // this lane's column in fragment 0
    const bool cols_ok = n0 + C::BN <= N;
#pragma unroll
    for (int mf = 0; mf < MT; ++mf)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + mf * 16 + 4 * lgrp + v;
            if (m < M) {
                const size_t row = SPLIT ? (((size_t)split * gridDim.y + bz) * M + m) * N : (size_t)m * N;
#pragma unroll
                for (int nf = 0; nf < NB; ++nf) {
                    const int n = nl + nf * 16;
                    if (cols_ok || n < N) {
                        if constexpr (SPLIT)
                            ws[row + n] = run[mf][nf][v];
                        else
                            store_elem<DT>(out, row + n, run[mf][nf][v]);
                    }
                }
            }
        }
}

template <int DT, int BITS, int GS, int MT, bool SPLIT, bool SBV, int WK, int NBT>
void qmm_go(dim3 grid, const uint32_t* w, const void* s, const void* b, const void* x, void* out, float* ws,
            QmxStrides sd, int M, int N, int K, int splits, int ntiles, int mtiles, int total, int per_xcd,
            hipStream_t st) {
    hipLaunchKernelGGL((qmm_t_kernel<DT, BITS, GS, MT, SPLIT, SBV, WK, NBT>), grid, dim3(QMM_THREADS), 0, st, w, s,
                       b, x, out, ws, sd, M, N, K, splits, ntiles, mtiles, total, per_xcd);
}

template <int DT, int BITS, int GS, int MT, int WK = 2, int NBT = QMM_NB>
hipError_t qmm_launch_mt(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                         float* ws, int batch, QmxStrides sd, int M, int N, int K, int splits, int mtiles,
                         hipStream_t st) {
    using C = QmmCfg<DT, BITS, GS, MT, false, WK, NBT>;
    const int ntiles = (N + C::BN - 1) / C::BN;
    const int total = ntiles * mtiles * splits;
    const int per_xcd = (total + 7) / 8;
    const dim3 grid(8 * per_xcd, batch);
    // Staged scales/biases need 16-byte aligned arrays, rows of whole 16-byte chunks
    // (K/GS a multiple of 8) and a K range whose chunks (plus one for alignment and
    // one for an odd count) fit the LDS left over.
    // the longest partition: whole segments of 256 columns (128 when K is not a
    // multiple of 256), ceil(nseg / splits) of them
    const int G = K / GS, seg = (K & 255) == 0 ? 256 : 128;
    const int nk_max = (K / seg + splits - 1) / splits * seg / C::KB;
    const bool aligned = ((reinterpret_cast<uintptr_t>(s) | reinterpret_cast<uintptr_t>(b)) & 15) == 0 &&
                         (sd.sb * 2) % 16 == 0;
    const bool sbv = aligned && K > 0 && G % 8 == 0 &&
                     (nk_max * C::GPB + 7) / 8 + 2 <= qmm_sbv_chunks<DT, BITS, GS, MT, WK, NBT>();
#define QMM_GO(SPLIT_, SBV_) \
    qmm_go<DT, BITS, GS, MT, SPLIT_, SBV_, WK, NBT>(grid, w, s, b, x, out, ws, sd, M, N, K, splits, ntiles, mtiles, total, per_xcd, st)
    if constexpr (WK != 8) {
        if (splits > 1) {
            if (sbv) QMM_GO(true, true);
            else QMM_GO(true, false);
            return hipGetLastError();
        }
    }
    // narrow tiles run unsplit only
    if (sbv) QMM_GO(false, true);
    else QMM_GO(false, false);
#undef QMM_GO
    return hipGetLastError();
}

template <int DT, int BITS, int GS>
hipError_t qmm_launch_gs(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                         float* ws, int batch, QmxStrides sd, int M, int N, int K, int splits, hipStream_t st) {
    if constexpr (BITS == 2 || BITS == 4 || BITS == 8) {
        // narrow tiles: one tile of 16 or 32 rows
        if (qmm_narrow(M, N, K, BITS, batch, splits, device_cu_count())) {
            // 16-column tiles while they fit one round of the chip: twice the
            // work-groups, each with half the matrix work per block (measured 11-23%
            // faster than 32-column tiles at M = 8..32, N = 1024..4096, K = 2048..8192)
            if ((long long)((N + 15) / 16) * batch <= device_cu_count()) {
                if (M <= 16) return qmm_launch_mt<DT, BITS, GS, 1, 8, 1>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, 1, st);
                return qmm_launch_mt<DT, BITS, GS, 2, 8, 1>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, 1, st);
            }
            if (M <= 16) return qmm_launch_mt<DT, BITS, GS, 1, 8>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, 1, st);
            return qmm_launch_mt<DT, BITS, GS, 2, 8>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, 1, st);
        }
    }
    if constexpr (BITS == 2 || BITS == 4 || BITS == 8) {
        // split-K on 64-column tiles of 256-column blocks while those fit one
        // round of the chip
        if (splits > 1 && qmm_wide64(M, N, K, BITS, batch, splits, device_cu_count())) {
            const int t64 = (M + 63) / 64;
#define QMM_64(MT_) qmm_launch_mt<DT, BITS, GS, MT_, 4>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, t64, st)
            switch (qmm_mt_for(M, t64)) {
                case 1: return QMM_64(1);
                case 2: return QMM_64(2);
                case 3: return QMM_64(3);
                default: return QMM_64(4);
            }
#undef QMM_64
        }
    }
    const int mt = qmm_mtiles_for(M, (long long)((N + QMM_BN - 1) / QMM_BN) * batch, device_cu_count(), K);
#define QMM_MT(MT_) qmm_launch_mt<DT, BITS, GS, MT_>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, mt, st)
    switch (qmm_mt_for(M, mt)) {
        case 1: return QMM_MT(1);
        case 2: return QMM_MT(2);
        case 3: return QMM_MT(3);
        case 4: return QMM_MT(4);
        case 6: return QMM_MT(6);
        default: return QMM_MT(8);
    }
#undef QMM_MT
}

template <int BITS>
hipError_t qmm_launch_bits(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                           float* ws, int batch, QmxStrides sd, int M, int N, int K, int gs, int dt, int splits,
                           hipStream_t st) {
    if (dt == DT_F16) {
        switch (gs) {
            case 32: return qmm_launch_gs<DT_F16, BITS, 32>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, st);
            case 64: return qmm_launch_gs<DT_F16, BITS, 64>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, st);
            default: return qmm_launch_gs<DT_F16, BITS, 128>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, st);
        }
    }
    switch (gs) {
        case 32: return qmm_launch_gs<DT_BF16, BITS, 32>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, st);
        case 64: return qmm_launch_gs<DT_BF16, BITS, 64>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, st);
        default: return qmm_launch_gs<DT_BF16, BITS, 128>(w, s, b, x, out, ws, batch, sd, M, N, K, splits, st);
    }
}

hipError_t qmm_launch_b1(const uint32_t*, const void*, const void*, const void*, void*, float*, int, QmxStrides,
                         int, int, int, int, int, int, hipStream_t);
hipError_t qmm_launch_b2(const uint32_t*, const void*, const void*, const void*, void*, float*, int, QmxStrides,
                         int, int, int, int, int, int, hipStream_t);
hipError_t qmm_launch_b3(const uint32_t*, const void*, const void*, const void*, void*, float*, int, QmxStrides,
                         int, int, int, int, int, int, hipStream_t);
hipError_t qmm_launch_b4(const uint32_t*, const void*, const void*, const void*, void*, float*, int, QmxStrides,
                         int, int, int, int, int, int, hipStream_t);
hipError_t qmm_launch_b5(const uint32_t*, const void*, const void*, const void*, void*, float*, int, QmxStrides,
                         int, int, int, int, int, int, hipStream_t);
hipError_t qmm_launch_b6(const uint32_t*, const void*, const void*, const void*, void*, float*, int, QmxStrides,
                         int, int, int, int, int, int, hipStream_t);
hipError_t qmm_launch_b8(const uint32_t*, const void*, const void*, const void*, void*, float*, int, QmxStrides,
                         int, int, int, int, int, int, hipStream_t);

}  // namespace qmx
