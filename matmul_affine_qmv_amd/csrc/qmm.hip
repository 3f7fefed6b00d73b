// qmm.hip -- tile-size choice for the staged qmm_t kernel, its launcher, and
// the split-K accumulate kernel.
#include "qmm_impl.h"

namespace qmx {

// 16-row x fragments per tile: the smallest of 1, 2, 3, 4, 6, 8 that covers
// the tile's share of M (tiles spread evenly over M).
int qmm_mt_for(int M, int mtiles) {
    static const int choices[] = {1, 2, 3, 4, 6, 8};
    const int tiles = mtiles > 0 ? mtiles : 1;
    const int rows = (M + tiles - 1) / tiles;
    const int frags = (rows + 15) / 16;
    for (int c : choices)
        if (c >= frags) return c;
    return 8;
}

// Tiles of at most 64 rows up to M = 192 (MT <= 4: measured 15-20% faster per
// call at M = 85 and 128 than one tile of 6 or 8 fragments, as the larger tiles
// lose ring depth and staged scales to LDS); 128-row tiles beyond, where the
// fewer, fuller tiles fill the chip better.  When 128-row tiles alone leave
// compute units idle, 64-row tiles are taken if, with the policy's K split,
// they launch at least as many work-groups.  Measured at N = K = 4096
// (policy route, per call): M = 384 33.7 against 37.2 us, M = 512 36.6
// against 39.7 us, and (N = 1024, M = 512) 19.7 against 25.1 us; at M = 257
// the 64-row tiles launch fewer work-groups (160 unsplit against 96 x 2) and
// were slower (34.4 against 31.5 us); at M = 1024 and 2048, where 128-row
// tiles fill the chip, 15% slower.
int qmm_mtiles_for(int M, long long col_tiles, int cus, int K) {
    const int t64 = (M + 63) / 64;
    if (M <= 192) return t64;
    const int t128 = (M + 127) / 128;
    if (cus <= 0 || col_tiles * t128 >= cus) return t128;
    const long long wg64 = col_tiles * t64 * qmm_policy_splits(col_tiles * t64, K, cus);
    const long long wg128 = col_tiles * t128 * qmm_policy_splits(col_tiles * t128, K, cus);
    return wg64 >= wg128 ? t64 : t128;
}

bool qmm_narrow(int M, int N, int K, int bits, long long batch, int splits, int cus) {
    if ((bits != 2 && bits != 4 && bits != 8) || K % 512 != 0 || M < 1 || M > 32 || splits != 1 || cus <= 0)
        return false;
    // The 128-column tiles leave compute units idle, and the narrow tiles, four
    // times as many, take at most 3 rounds of the chip: a narrow block holds the
    // columns of 4 wide blocks at the same cost per wave.  Measured unsplit at
    // M = 4..7, K = 5120: N = 14336 (448 narrow tiles, 2 rounds) 18.3 us against
    // 24.7 us on 112 wide tiles; N = 27648 (864, 4 rounds) 34.5 against 25.6 us.
    const long long wide = (long long)((N + QMM_BN - 1) / QMM_BN) * batch;
    const long long narrow = (long long)((N + 31) / 32) * batch;
    return wide < cus && narrow <= 3LL * cus;
}

// Split-K on 64-column tiles (the 8 waves as 4 K groups of 2 column waves over
// 256-column K blocks): per block the same work as a 128-column tile, so with
// half the partitions a work-group walks as many blocks, and the partials and
// their accumulate halve.  Measured against 128-column tiles at twice the
// partitions: (17408, 5120, 56) 30.8 against 32.0 us, (10752, 2048, 85) 17.5
// against 18.5, (4096, 4096, 64) 13.4 against 16.9, (4096, 4096, 128) 17.7
// against 20.3, (5120, 5120, 48) 14.3 against 16.1; taken while the tiles of
// all partitions fit one round of the chip (at twice that they lost 10-20%).
bool qmm_wide64(int M, int N, int K, int bits, long long batch, int splits, int cus) {
    if ((bits != 2 && bits != 4 && bits != 8) || K % 256 != 0 || M < 1 || M > 192 || splits < 2 || cus <= 0)
        return false;
    const long long tiles = (long long)((N + 63) / 64) * ((M + 63) / 64) * batch;
    return tiles * splits <= cus;
}

// Chunks of staged scales and biases a 64-column work-group of MT row
// fragments holds in LDS.
template <int DT, int BITS, int GS>
static int wide64_sbv_capacity(int mt) {
    switch (mt) {
        case 1: return qmm_sbv_chunks<DT, BITS, GS, 1, 4>();
        case 2: return qmm_sbv_chunks<DT, BITS, GS, 2, 4>();
        case 3: return qmm_sbv_chunks<DT, BITS, GS, 3, 4>();
        default: return qmm_sbv_chunks<DT, BITS, GS, 4, 4>();
    }
}

template <int DT, int BITS>
static int wide64_sbv_capacity_gs(int gs, int mt) {
    return gs == 32 ? wide64_sbv_capacity<DT, BITS, 32>(mt)
         : gs == 64 ? wide64_sbv_capacity<DT, BITS, 64>(mt) : wide64_sbv_capacity<DT, BITS, 128>(mt);
}

template <int DT>
static int wide64_sbv_capacity_bits(int bits, int gs, int mt) {
    return bits == 2 ? wide64_sbv_capacity_gs<DT, 2>(gs, mt)
         : bits == 4 ? wide64_sbv_capacity_gs<DT, 4>(gs, mt) : wide64_sbv_capacity_gs<DT, 8>(gs, mt);
}

// Without staged scales and biases each stage carries its block's raw values,
// which cost more than the 128-column plan's extra partitions (8-bit codes at
// (17408, 5120, 56): 38.1 us on 64-column tiles in 3 partitions without them,
// 36.8 us on 128-column tiles in 6 with them); at a given partition count the
// 64-column tiles stay ahead either way (twice the work-groups).
bool qmm_wide64_staged(int M, int K, int bits, int gs, int dt, int splits) {
    if ((bits != 2 && bits != 4 && bits != 8) || (gs != 32 && gs != 64 && gs != 128) ||
        (dt != DT_F16 && dt != DT_BF16) || K % 256 != 0 || M < 1 || M > 192 || splits < 1)
        return false;
    if ((K / gs) % 8 != 0) return true;   // staged on neither tile width
    const int mt = qmm_mt_for(M, (M + 63) / 64);
    const int groups = (K / 256 + splits - 1) / splits * (256 / gs);
    const int cap = dt == DT_F16 ? wide64_sbv_capacity_bits<DT_F16>(bits, gs, mt)
                                 : wide64_sbv_capacity_bits<DT_BF16>(bits, gs, mt);
    return (groups + 7) / 8 + 2 <= cap;
}

// A narrow work-group walks all of K (K / 512 blocks) where each partition of
// the split 128-column plan walks K / (128 S) blocks of the same cost per wave;
// the narrow call saves the accumulate kernel and its launch instead.  Both
// plans run one work-group per CU at a time, so each walks its blocks once per
// round of the chip.  Measured per call at M = 8..32, N = 1024..14336, K =
// 2048..8192 on 256 CUs: narrow is up to 1.4x faster while it walks at most 4
// blocks more than the split plan, even at 6, and 8-25% slower from 8 on at 32
// rows.  Two rounds of narrow tiles pay the work-group's fixed costs twice; they
// measured 1-5% faster than the split plan at K = 4096 and 5120 (N = 11008,
// 14336, 16384: 8-10 blocks per round) but 3-17% slower at K = 8192 and 12288
// (16384 x 8192: 29.1 against 24.9 us), so they are taken only while a
// work-group walks at most 10 blocks.  At gs 32 each wave carries two group
// epilogues per block, which weighs more on the narrow tiles: measured at M =
// 8..32 (4-bit, and 16 rows at 2 and 8 bits), 16-column tiles were 8-34%
// faster than the split plan with up to 2 blocks more (4096 x 4096: 8.1 against
// 8.9 us at M = 8; 2048 x 2048: 5.2 against 6.6), 10-16% slower with 3 or more
// (1024 x 4096, 4096 x 8192), and 32-column tiles 15-22% slower even at equal
// blocks (14336 x 4096), so at gs 32 only 16-column tiles within 2 blocks are
// taken.
bool qmm_narrow_preferred(int M, int N, int K, int bits, int gs, long long batch, int cus) {
    if (!qmm_narrow(M, N, K, bits, batch, 1, cus)) return false;
    // 16-column tiles where they fit one round, else 32-column tiles
    const long long t16 = (long long)((N + 15) / 16) * batch;
    const bool cols16 = t16 <= cus;
    if (gs < 64 && !cols16) return false;
    const long long tiles = cols16 ? t16 : (long long)((N + 31) / 32) * batch;
    if (4 * tiles < cus || tiles > 2LL * cus || (tiles > cus && K / 512 > 10)) return false;
    const long long wide = (long long)((N + QMM_BN - 1) / QMM_BN) * batch;
    const long long wide_tiles = wide * qmm_mtiles_for(M, wide, cus, K);
    const int s = qmm_policy_splits(wide_tiles, K, cus);
    // a block of a 16-column tile (half the matrix work) weighs 0.7 of a block of
    // the 128-column split plan (measured over N = 1024..4096, K = 2048..8192,
    // M = 4..32: within 3% of the best route where the blocks are close)
    const double narrow_blocks = (double)((tiles + cus - 1) / cus) * (K / 512) * (cols16 ? 0.7 : 1.0);
    const long long split_blocks = (wide_tiles * s + cus - 1) / cus * (K / (QMM_KB * s));
    return narrow_blocks <= (double)split_blocks + (gs < 64 ? 2.0 : 6.0);
}

hipError_t launch_qmm_t(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                        float* ws, int batch, QmxStrides sd, int M, int N, int K, int bits, int gs,
                        int dt, int splits, hipStream_t st) {
    switch (bits) {
        case 1: return qmm_launch_b1(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
        case 2: return qmm_launch_b2(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
        case 3: return qmm_launch_b3(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
        case 4: return qmm_launch_b4(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
        case 5: return qmm_launch_b5(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
        case 6: return qmm_launch_b6(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
        default: return qmm_launch_b8(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
    }
}

// out[i] = round(sum_{p=0}^{S-1} ws[p*MN + i]), summed in ascending p in float32
// and rounded once (page "mlx PR 4682": separate accumulate kernel, one
// rounding).  S is a template parameter so every partial load of a thread is
// issued before the first add; one wave per work-group spreads the few
// thousand threads over all CUs.
template <int DT, int S, bool VEC>
__global__ __launch_bounds__(64) void splitk_accum_kernel(const float* __restrict__ ws, void* __restrict__ out,
                                                          size_t MN) {
    const size_t i0 = ((size_t)blockIdx.x * 64 + threadIdx.x) * 4;
    if (i0 >= MN) return;
    if (VEC && i0 + 4 <= MN) {
        f32x4 v[S];
#pragma unroll
        for (int p = 0; p < S; ++p) v[p] = *reinterpret_cast<const f32x4*>(ws + (size_t)p * MN + i0);
        f32x4 acc = v[0];
#pragma unroll
        for (int p = 1; p < S; ++p) {
            acc.x += v[p].x; acc.y += v[p].y; acc.z += v[p].z; acc.w += v[p].w;
        }
        if constexpr (DT == DT_F16 || DT == DT_BF16) {
            const uint32_t lo = DT == DT_F16 ? (f32_to_f16_bits(acc.x) | (f32_to_f16_bits(acc.y) << 16))
                                             : (f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16));
            const uint32_t hi = DT == DT_F16 ? (f32_to_f16_bits(acc.z) | (f32_to_f16_bits(acc.w) << 16))
                                             : (f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16));
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + i0) = u32x2{lo, hi};
        }
    } else {
        const size_t iend = i0 + 4 < MN ? i0 + 4 : MN;
        for (size_t i = i0; i < iend; ++i) {
            float acc = ws[i];
#pragma unroll
            for (int p = 1; p < S; ++p) acc += ws[(size_t)p * MN + i];
            store_elem<DT>(out, i, acc);
        }
    }
}

template <int DT, int S>
static void accum_go(const float* ws, void* out, size_t MN, bool vec, hipStream_t st) {
    const size_t threads = (MN + 3) / 4;
    const dim3 grid((unsigned)((threads + 63) / 64)), block(64);
    if (vec) hipLaunchKernelGGL((splitk_accum_kernel<DT, S, true>), grid, block, 0, st, ws, out, MN);
    else hipLaunchKernelGGL((splitk_accum_kernel<DT, S, false>), grid, block, 0, st, ws, out, MN);
}

template <int DT>
static void accum_dt(const float* ws, void* out, int splits, size_t MN, bool vec, hipStream_t st) {
    switch (splits) {
        case 2: accum_go<DT, 2>(ws, out, MN, vec, st); break;
        case 3: accum_go<DT, 3>(ws, out, MN, vec, st); break;
        case 4: accum_go<DT, 4>(ws, out, MN, vec, st); break;
        case 5: accum_go<DT, 5>(ws, out, MN, vec, st); break;
        case 6: accum_go<DT, 6>(ws, out, MN, vec, st); break;
        case 7: accum_go<DT, 7>(ws, out, MN, vec, st); break;
        case 8: accum_go<DT, 8>(ws, out, MN, vec, st); break;
        case 9: accum_go<DT, 9>(ws, out, MN, vec, st); break;
        case 10: accum_go<DT, 10>(ws, out, MN, vec, st); break;
        case 11: accum_go<DT, 11>(ws, out, MN, vec, st); break;
        case 12: accum_go<DT, 12>(ws, out, MN, vec, st); break;
        case 13: accum_go<DT, 13>(ws, out, MN, vec, st); break;
        case 14: accum_go<DT, 14>(ws, out, MN, vec, st); break;
        case 15: accum_go<DT, 15>(ws, out, MN, vec, st); break;
        default: accum_go<DT, 16>(ws, out, MN, vec, st); break;
    }
}

hipError_t launch_splitk_accum(const float* ws, void* out, int splits, size_t MN, int dt, hipStream_t st) {
    // the vector path needs 16-byte aligned partial rows and 8-byte aligned output
    const bool vec = (MN % 4) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0;
    if (dt == DT_F16) accum_dt<DT_F16>(ws, out, splits, MN, vec, st);
    else accum_dt<DT_BF16>(ws, out, splits, MN, vec, st);
    return hipGetLastError();
}

}  // namespace qmx
