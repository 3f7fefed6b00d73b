// qmx_internal.h -- host-side launchers shared between the kernel sources and
// the C ABI in qmx_api.cpp.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmx {

// Rows of W per qmv wave, and rows of x per qmv wave tile.
constexpr int QMV_ROWS = 4;
int qmv_mt_for(int M);

// A qmv lane reads a row in chunks: 16 bytes for the widths that divide 32
// (128/bits codes), and for 1, 3, 5 and 6 bits the `bits` words that hold
// exactly 32 codes (fields may straddle words inside the chunk, never across
// chunks).
constexpr int qmv_chunk_words(int bits) { return (bits == 2 || bits == 4 || bits == 8) ? 4 : bits; }
constexpr int qmv_chunk_codes(int bits) { return 32 * qmv_chunk_words(bits) / bits; }

// qmm_t geometry: 128-column K blocks of 4 MFMA k-steps; 8 waves = 4 along N
// (2 x 16 columns each) x 2 halves that take alternate k-step pairs.
constexpr int QMM_WAVES_N = 4;
constexpr int QMM_NB = 2;
constexpr int QMM_BN = QMM_WAVES_N * QMM_NB * 16;
constexpr int QMM_KB = 128;
constexpr int QMM_THREADS = 2 * QMM_WAVES_N * 64;
// Tiles along M for M rows of x when `col_tiles` column tiles (N tiles times
// the batch) share `cus` compute units over K columns, and the 16-row x
// fragments per tile (1, 2, 3, 4, 6 or 8) for M rows in `mtiles` tiles.
// Tiles never exceed (M + 63) / 64.
int qmm_mtiles_for(int M, long long col_tiles, int cus, int K);
int qmm_mt_for(int M, int mtiles);
// Whether an unsplit qmm_t runs on 32-column tiles whose 8 waves split K among
// them (one work-group per tile, 16 or 32 rows of x) instead of 128-column
// tiles: 2-, 4- or 8-bit codes, K a multiple of 512, M <= 32, 128-column
// tiles that would leave some of the `cus` compute units idle, and at most
// 3 * cus narrow tiles.
bool qmm_narrow(int M, int N, int K, int bits, long long batch, int splits, int cus);
// Whether `splits` split-K partitions run on 64-column tiles of 256-column
// blocks: 2-, 4- or 8-bit codes, K a multiple of 256, M <= 192 and the tiles of
// all partitions within one round of the `cus` compute units.
bool qmm_wide64(int M, int N, int K, int bits, long long batch, int splits, int cus);
// Whether such a 64-column work-group can stage the longest partition's scales
// and biases in LDS (or neither tile width can: K / gs not a multiple of 8).
bool qmm_wide64_staged(int M, int K, int bits, int gs, int dt, int splits);
// Whether the dispatch policy runs such a problem unsplit on 32-column tiles
// rather than split-K on 128-column tiles: the narrow tiles launch between a
// quarter of the compute units and all of them, K is short enough for one
// work-group to walk, and groups span at least 64 codes.
bool qmm_narrow_preferred(int M, int N, int K, int bits, int gs, long long batch, int cus);
// K partitions the dispatch policy gives `tiles` output tiles on `cus`
// compute units (1: unsplit).
int qmm_policy_splits(long long tiles, int K, int cus);
// Compute units of the current device (cached per device), or -1.
int device_cu_count();

// A batch of independent problems of one shape: problem i reads weights
// `i * w` words, scales and biases `i * sb` elements and x `i * x` elements
// after the first (a stride of 0 shares that operand), x rows are `x_row`
// elements apart (>= K), and it writes output matrix i of a contiguous
// [batch][M][N] (split-K partials: [S][batch][M][N]).
// With index arrays (gather), problem i takes weight matrix w_index[i] and x
// matrix x_index[i] instead of i, each clamped to [0, count - 1].
struct QmxStrides {
    long long w, sb, x, x_row;
    const int* w_index = nullptr;
    const int* x_index = nullptr;
    int num_w = 0, num_x = 0;
};
inline QmxStrides unbatched(int K) { return QmxStrides{0, 0, 0, K}; }

// Weight and x matrix of problem `i` (device side; a wave-uniform load).
__device__ __forceinline__ long long qmx_w_matrix(const QmxStrides& sd, long long i) {
    if (!sd.w_index) return i;
    const int v = sd.w_index[i];
    return v < 0 ? 0 : v >= sd.num_w ? sd.num_w - 1 : v;
}
__device__ __forceinline__ long long qmx_x_matrix(const QmxStrides& sd, long long i) {
    if (!sd.x_index) return i;
    const int v = sd.x_index[i];
    return v < 0 ? 0 : v >= sd.num_x ? sd.num_x - 1 : v;
}

// M = 1 work split chosen for `rows` rows of W in all (N times the batch).
struct QmvSplit {
    int ks, rg;
};
QmvSplit qmv_split_for(int M, long long rows, int K, int bits);

// group > 1 (M = 1 with w_index only): one tile serves up to `group`
// consecutive problems that pick the same weight matrix, as its x rows.
hipError_t launch_qmv(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                      int batch, QmxStrides sd, int M, int N, int K, int bits, int gs, int dt,
                      hipStream_t st, int group = 1);

// splits == 1: writes `out` in dtype dt.  splits > 1: writes float32
// partials ws[p][batch][M][N] (the accumulate kernel is launched separately).
hipError_t launch_qmm_t(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                        float* ws, int batch, QmxStrides sd, int M, int N, int K, int bits, int gs,
                        int dt, int splits, hipStream_t st);

// Copies a batch of strided matrices [batch][M][K] (elements of `elem` bytes,
// matrix stride `xs`, row stride `xr`) into a contiguous array.
hipError_t launch_copy_rows(const void* x, void* dst, int batch, long long xs, long long xr, int M, int K,
                            int elem, hipStream_t st);

hipError_t launch_splitk_accum(const float* ws, void* out, int splits, size_t MN, int dt,
                               hipStream_t st);

hipError_t launch_q8_0(const uint32_t* w, const float* x, float* out, int N, int K, hipStream_t st);
hipError_t launch_q4_k(const uint32_t* w, const float* x, float* out, int N, int K, hipStream_t st);
hipError_t launch_q8_i8(const uint32_t* wq, const uint32_t* xq, const float* wd, float* out, int N, int K,
                        hipStream_t st);

}  // namespace qmx
