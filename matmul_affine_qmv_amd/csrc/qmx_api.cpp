// qmx_api.cpp -- the C ABI declared in include/qmx.h: host-side validation,
// the dispatch policy and the kernel launches.  Every check runs before any
// HIP call, so argument errors never reach the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>

#include "qmx.h"
#include "qmx_internal.h"

namespace {

using qmx::QMM_BN;
using qmx::QMM_KB;

// Largest split count the dispatch policy picks by itself.
constexpr int kPolicyMaxSplits = 16;
// Default compute-unit count for planning without a device (MI355X).
constexpr int kDefaultCUs = 256;

bool is_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t elem_bytes(int dt) { return dt == QMX_F32 ? 4 : 2; }

// Checks shared by every affine route.
int check_affine_common(int M, int N, int K, int bits, int gs, int dtype) {
    if (dtype != QMX_F32 && dtype != QMX_F16 && dtype != QMX_BF16) return QMX_ERR_DTYPE;
    if (bits < 1 || bits > 8 || bits == 7) return QMX_ERR_BITS;
    if (gs != 32 && gs != 64 && gs != 128) return QMX_ERR_GROUP;
    if (M < 0 || N < 0 || K < 0) return QMX_ERR_SHAPE;
    if (K % gs != 0) return QMX_ERR_GROUP;
    return QMX_OK;
}

int check_affine_ptrs(const uint32_t* w, const void* s, const void* b, const void* x, void* out, int K,
                      int dtype, uintptr_t w_align, uintptr_t x_align) {
    if (!out) return QMX_ERR_NULL;
    if (K > 0 && (!w || !s || !b || !x)) return QMX_ERR_NULL;
    const uintptr_t e = elem_bytes(dtype);
    if (!is_aligned(out, e)) return QMX_ERR_ALIGN;
    if (K > 0) {
        if (!is_aligned(w, w_align) || !is_aligned(x, x_align)) return QMX_ERR_ALIGN;
        if (!is_aligned(s, e) || !is_aligned(b, e)) return QMX_ERR_ALIGN;
    }
    return QMX_OK;
}

int check_qmv(const uint32_t* w, const void* s, const void* b, const void* x, void* out, int M, int N, int K,
              int bits, int gs, int dtype) {
    int rc = check_affine_common(M, N, K, bits, gs, dtype);
    if (rc) return rc;
    if (K % qmx::qmv_chunk_codes(bits) != 0) return QMX_ERR_SHAPE;
    if (M > 0 && (M + qmx::qmv_mt_for(M) - 1) / qmx::qmv_mt_for(M) > 65535) return QMX_ERR_SHAPE;
    if (M == 0 || N == 0) return QMX_OK;
    return check_affine_ptrs(w, s, b, x, out, K, dtype, 16, 16);
}

int check_qmm(const uint32_t* w, const void* s, const void* b, const void* x, void* out, int M, int N, int K,
              int bits, int gs, int dtype, int splits) {
    int rc = check_affine_common(M, N, K, bits, gs, dtype);
    if (rc) return rc;
    if (dtype == QMX_F32) return QMX_ERR_DTYPE;
    if (K % QMM_KB != 0) return QMX_ERR_SHAPE;
    // the largest tiling the launcher may choose
    const long long tiles = (long long)((N + QMM_BN - 1) / QMM_BN) * (M > 0 ? (M + 63) / 64 : 0);
    if (tiles * splits + 8 > INT_MAX) return QMX_ERR_SHAPE;
    if (M == 0 || N == 0) return QMX_OK;
    return check_affine_ptrs(w, s, b, x, out, K, dtype, 16, 16);
}

int max_splits_for(int K) {
    const int by_k = K / (2 * QMM_KB);   // every partition holds at least 256 columns
    return by_k < QMX_MAX_SPLITS ? by_k : QMX_MAX_SPLITS;
}

int launch_status(hipError_t e) { return e == hipSuccess ? QMX_OK : QMX_ERR_LAUNCH; }

// Compute units of the current device, cached per device id.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return -1;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Below M = 8 qmv reads each weight once for up to 4 rows of x, and makes a
// second pass for M > 4; a pass costs the same for 3 and 4 rows.  Measured on
// the chip (N x K from 1024 x 4096 to 14336 x 5120, M = 2..7, 4-bit gs 64):
// * where 16-column tiles apply (N / 16 tiles fit one round of the chip), the
//   matrix route walks K at about 3.4 us plus 0.8 us per 1024 columns of K and
//   beat qmv from M = 3 on at every measured shape (4096 x 4096, M = 4: 6.8
//   against 8.0 us); at M = 2 qmv costs about 2.5 us plus 0.16 us per million
//   codes, but at least 2.5 us plus 0.65 us per 1024 columns of K, and won at
//   every measured shape (2048 x 8192: 8.0 against 9.2 us);
// * otherwise qmv costs about 2.5 us plus 0.16, 0.28 or 0.45 us per million
//   codes for M = 2, 3..4 and 5..7 (at least 2.5 us plus 0.65 us, from M = 3
//   3 us plus 0.8 us, per 1024 columns of K: 2048 x 8192, M = 4: 10.3 us), and
//   the matrix route 3.5 us plus 1.1 us per
//   1024 columns of K for each round of the chip its 32-column tiles take
//   (14336 x 4096 in two rounds: 15.0-15.6 us), or, without narrow tiles,
//   about its weight bytes at 2.3 TB/s with a floor of about 9 us.
bool small_m_prefers_matrix(int M, int N, int K, int bits, int gs, int batch, int cus) {
    if (M < 2 || M >= 8) return false;
    const int b = batch > 0 ? batch : 1;
    const double mcodes = (double)N * K * b / 1e6;
    // the M = 2..7 estimates below were fitted at gs 64 and 128
    const bool narrow = gs >= 64 && qmx::qmm_narrow_preferred(M, N, K, bits, gs, b, cus);
    if (narrow && (long long)((N + 15) / 16) * b <= cus) {
        if (M >= 3) return true;
        return 3.4 + 0.8 * K / 1024.0 < std::max(2.5 + 0.16 * mcodes, 2.5 + 0.65 * K / 1024.0);
    }
    const double t_qmv = std::max(2.5 + (M == 2 ? 0.16 : M <= 4 ? 0.28 : 0.45) * mcodes,
                                  M == 2 ? 2.5 + 0.65 * K / 1024.0 : 3.0 + 0.8 * K / 1024.0);
    double t_mat = std::max(9.0, mcodes * 1e6 * bits / 8.0 / 2.3e6);
    if (narrow) {
        const long long rounds = ((long long)(N + 31) / 32 * b + cus - 1) / cus;
        t_mat = (double)rounds * (3.5 + 1.1 * K / 1024.0);
    }
    return t_mat < t_qmv;
}

int plan_impl(int M, int N, int K, int bits, int gs, int dtype, int num_cus, int* route, int* splits,
              int batch = 1) {
    int rc = check_affine_common(M, N, K, bits, gs, dtype);
    if (rc) return rc;
    if (num_cus <= 0) num_cus = kDefaultCUs;
    // float32, K that the staged kernel cannot block and M < 8 stay on qmv,
    // unless M is 2..7 and the vector-ALU work of qmv outweighs the matrix route.
    if (dtype == QMX_F32 || K % QMM_KB != 0 || (M < 8 && !small_m_prefers_matrix(M, N, K, bits, gs, batch, num_cus))) {
        if (K % qmx::qmv_chunk_codes(bits) != 0) return QMX_ERR_SHAPE;
        *route = QMX_ROUTE_QMV;
        *splits = 1;
        return QMX_OK;
    }
    const long long col_tiles = (long long)((N + QMM_BN - 1) / QMM_BN) * batch;
    const long long tiles = col_tiles * qmx::qmm_mtiles_for(M, col_tiles, num_cus, K);
    int s = qmx::qmm_policy_splits(tiles, K, num_cus);
    // where 64-column tiles take the split partitions, as many partitions as keep
    // those resident at once (about half the 128-column plan's), while they can
    // stage the partition's scales and biases
    if ((bits == 2 || bits == 4 || bits == 8) && K % 256 == 0 && M <= 192) {
        const long long tiles64 = (long long)((N + 63) / 64) * ((M + 63) / 64) * batch;
        const int s64 = qmx::qmm_policy_splits(tiles64, K, num_cus);
        if (s64 >= 2 && qmx::qmm_wide64(M, N, K, bits, batch, s64, num_cus) &&
            qmx::qmm_wide64_staged(M, K, bits, gs, dtype, s64))
            s = s64;
    }
    if (s >= 2 && qmx::qmm_narrow_preferred(M, N, K, bits, gs, batch, num_cus)) s = 1;
    *route = s >= 2 ? QMX_ROUTE_QMM_T_SPLITK : QMX_ROUTE_QMM_T;
    *splits = s;
    return QMX_OK;
}

// ---------------------------------------------------------------- batched
// Workspace layout of a batched call: the split-K partials (rounded up to 256
// bytes), then, when x must be copied, the contiguous copy of x.
size_t batched_partials_bytes(int batch, int M, int N, int route, int splits) {
    if (route != QMX_ROUTE_QMM_T_SPLITK) return 0;
    return ((size_t)splits * batch * M * N * sizeof(float) + 255) & ~(size_t)255;
}

bool x_needs_copy(const void* x, long long xs, long long xr, int dtype) {
    const long long e = (long long)elem_bytes(dtype);
    return !is_aligned(x, 16) || (xs * e) % 16 != 0 || (xr * e) % 16 != 0;
}

int check_batched(int batch, int M, int N, int K, long long ws_, long long sbs, long long xs, long long xr,
                  int bits, int gs, int dtype) {
    int rc = check_affine_common(M, N, K, bits, gs, dtype);
    if (rc) return rc;
    if (batch < 0 || batch > 65535 || ws_ < 0 || sbs < 0 || xs < 0 || xr < K) return QMX_ERR_SHAPE;
    // per-problem lane offsets of the vector-ALU route stay in 32 bits
    if (xr > ((1LL << 31) - 1) / 8 / (long long)elem_bytes(dtype)) return QMX_ERR_SHAPE;
    if (ws_ % 4 != 0) return QMX_ERR_ALIGN;   // every weight matrix starts 16-byte aligned
    return QMX_OK;
}

size_t batched_workspace(int batch, int num_x, int M, int N, int K, int bits, int gs, int dtype, const void* x,
                         long long xs, long long xr) {
    int route = 0, splits = 1;
    if (check_batched(batch, M, N, K, 0, 0, xs, xr, bits, gs, dtype) != QMX_OK) return 0;
    if (batch == 0 || M == 0 || N == 0) return 0;
    if (plan_impl(M, N, K, bits, gs, dtype, device_cus(), &route, &splits, batch) != QMX_OK) return 0;
    size_t bytes = batched_partials_bytes(batch, M, N, route, splits);
    if (K > 0 && x_needs_copy(x, xs, xr, dtype)) bytes += (size_t)num_x * M * K * elem_bytes(dtype);
    return bytes;
}

// Problems per vector-route tile for a gather whose w_index holds runs of
// equal values: the run length a balanced sorted index gives (batch / num_w,
// rounded up), as 1, 2 or 4.
int gather_group(int batch, int num_w) {
    const int run = (batch + num_w - 1) / num_w;
    return run >= 3 ? 4 : run == 2 ? 2 : 1;
}

// Shared body of the batched and gathered calls: w_index/x_index NULL means
// problem i uses matrix i (num_w = num_x = batch).  `sorted`: w_index is
// expected to hold runs of equal values (see gather_group).
int batched_impl(const uint32_t* w_packed, const void* scales, const void* biases, const void* x, void* out,
                 const int* w_index, const int* x_index, int num_w, int num_x, int batch, int M, int N, int K,
                 long long w_batch_stride, long long sb_batch_stride, long long x_batch_stride,
                 long long x_row_stride, int bits, int group_size, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream, bool sorted = false) {
    int rc = check_batched(batch, M, N, K, w_batch_stride, sb_batch_stride, x_batch_stride, x_row_stride, bits,
                           group_size, dtype);
    if (rc) return rc;
    if (num_w < 0 || num_x < 0) return QMX_ERR_SHAPE;
    if (batch == 0 || M == 0 || N == 0) return QMX_OK;
    if (num_w == 0 || num_x == 0) return QMX_ERR_SHAPE;
    const int cus = device_cus();
    if (cus <= 0) return QMX_ERR_DEVICE;
    int route = 0, splits = 1;
    rc = plan_impl(M, N, K, bits, group_size, dtype, cus, &route, &splits, batch);
    if (rc) return rc;
    if (route == QMX_ROUTE_QMV) {
        if (K % qmx::qmv_chunk_codes(bits) != 0) return QMX_ERR_SHAPE;
        if ((long long)((M + qmx::qmv_mt_for(M) - 1) / qmx::qmv_mt_for(M)) > 65535) return QMX_ERR_SHAPE;
    } else {
        const long long tiles = (long long)((N + QMM_BN - 1) / QMM_BN) * ((M + 63) / 64);
        if (tiles * splits + 8 > INT_MAX) return QMX_ERR_SHAPE;
    }
    const bool copy_x = K > 0 && x_needs_copy(x, x_batch_stride, x_row_stride, dtype);
    // pointer checks: x may be at any element offset when it is copied first
    rc = check_affine_ptrs(w_packed, scales, biases, x, out, K, dtype, 16, copy_x ? elem_bytes(dtype) : 16);
    if (rc) return rc;
    if ((w_index && !is_aligned(w_index, 4)) || (x_index && !is_aligned(x_index, 4))) return QMX_ERR_ALIGN;
    const size_t part_bytes = batched_partials_bytes(batch, M, N, route, splits);
    const size_t need = part_bytes + (copy_x ? (size_t)num_x * M * K * elem_bytes(dtype) : 0);
    if (need > 0 && (!workspace || !is_aligned(workspace, 256) || workspace_bytes < need)) return QMX_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    qmx::QmxStrides sd{w_batch_stride, sb_batch_stride, x_batch_stride, x_row_stride, w_index, x_index, num_w, num_x};
    if (copy_x) {
        void* xc = static_cast<unsigned char*>(workspace) + part_bytes;
        rc = launch_status(qmx::launch_copy_rows(x, xc, num_x, x_batch_stride, x_row_stride, M, K,
                                                 (int)elem_bytes(dtype), st));
        if (rc) return rc;
        x = xc;
        sd.x = (long long)M * K;
        sd.x_row = K;
    }
    int group = 1;
    if (sorted && w_index && route == QMX_ROUTE_QMV && M == 1) {
        // a grouped tile addresses its x rows from the first x matrix in 32 bits
        const int g = gather_group(batch, num_w);
        if (g > 1 && ((long long)(num_x - 1) * sd.x + K) * (long long)elem_bytes(dtype) < (1LL << 31)) group = g;
    }
    if (route == QMX_ROUTE_QMV)
        return launch_status(qmx::launch_qmv(w_packed, scales, biases, x, out, batch, sd, M, N, K, bits, group_size,
                                             dtype, st, group));
    if (route == QMX_ROUTE_QMM_T)
        return launch_status(qmx::launch_qmm_t(w_packed, scales, biases, x, out, nullptr, batch, sd, M, N, K, bits,
                                               group_size, dtype, 1, st));
    float* ws = static_cast<float*>(workspace);
    rc = launch_status(qmx::launch_qmm_t(w_packed, scales, biases, x, out, ws, batch, sd, M, N, K, bits, group_size,
                                         dtype, splits, st));
    if (rc) return rc;
    return launch_status(qmx::launch_splitk_accum(ws, out, splits, (size_t)batch * M * N, dtype, st));
}

}  // namespace

namespace qmx {
int device_cu_count() { return device_cus(); }

int qmm_policy_splits(long long tiles, int K, int cus) {
    // below 8 K blocks the partitions are too short to repay the accumulate
    // (measured: K = 512 and 768 unsplit 10-15% faster at M = 16, N = 4096)
    if (K < 8 * QMM_KB || tiles >= cus || tiles <= 0) return 1;
    // as many partitions as keep every work-group of the launch resident at once
    long long s = cus / tiles;
    const int cap = max_splits_for(K) < kPolicyMaxSplits ? max_splits_for(K) : kPolicyMaxSplits;
    if (s > cap) s = cap;
    return s >= 2 ? (int)s : 1;
}
}  // namespace qmx

extern "C" {

int qmx_api_version(void) { return QMX_API_VERSION; }

const char* qmx_strerror(int status) {
    switch (status) {
        case QMX_OK: return "success";
        case QMX_ERR_NULL: return "a required pointer is NULL";
        case QMX_ERR_SHAPE: return "unsupported or negative problem size for this route";
        case QMX_ERR_BITS: return "bits must be 1, 2, 3, 4, 5, 6 or 8";
        case QMX_ERR_GROUP: return "group_size must be 32, 64 or 128 and divide K";
        case QMX_ERR_DTYPE: return "unsupported dtype for this route";
        case QMX_ERR_ALIGN: return "a pointer is not aligned as the route requires";
        case QMX_ERR_WORKSPACE: return "split-K workspace is NULL, misaligned or too small";
        case QMX_ERR_SPLITS: return "split count out of range for this K";
        case QMX_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case QMX_ERR_DEVICE: return "no usable HIP device";
        case QMX_ERR_SCRATCH: return "split-K partials exceed the scratch array of qmx_qmm_t_splitk_noalloc";
        default: return "unknown status";
    }
}

int qmx_qmv(const uint32_t* w_packed, const void* scales, const void* biases, const void* x, void* out,
            int M, int N, int K, int bits, int group_size, int dtype, void* stream) {
    const int rc = check_qmv(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype);
    if (rc || M == 0 || N == 0) return rc;
    return launch_status(qmx::launch_qmv(w_packed, scales, biases, x, out, 1, qmx::unbatched(K), M, N, K, bits,
                                         group_size, dtype, static_cast<hipStream_t>(stream)));
}

int qmx_qmm_t(const uint32_t* w_packed, const void* scales, const void* biases, const void* x, void* out,
              int M, int N, int K, int bits, int group_size, int dtype, void* stream) {
    const int rc = check_qmm(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype, 1);
    if (rc || M == 0 || N == 0) return rc;
    return launch_status(qmx::launch_qmm_t(w_packed, scales, biases, x, out, nullptr, 1, qmx::unbatched(K), M, N,
                                           K, bits, group_size, dtype, 1, static_cast<hipStream_t>(stream)));
}

size_t qmx_splitk_workspace_bytes(int M, int N, int splits) {
    if (M < 0 || N < 0 || splits < 0) return 0;
    return (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

int qmx_qmm_t_partials(const uint32_t* w_packed, const void* scales, const void* biases, const void* x,
                       int M, int N, int K, int bits, int group_size, int dtype, int splits, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (splits < 2 || splits > QMX_MAX_SPLITS) return QMX_ERR_SPLITS;
    // the workspace stands in for `out` in the shared pointer checks
    int rc = check_qmm(w_packed, scales, biases, x, workspace, M, N, K, bits, group_size, dtype, splits);
    if (rc == QMX_ERR_NULL && !workspace && M > 0 && N > 0) return QMX_ERR_WORKSPACE;
    if (rc) return rc;
    if (splits > max_splits_for(K)) return QMX_ERR_SPLITS;
    if (M == 0 || N == 0) return QMX_OK;
    if (!workspace || !is_aligned(workspace, 16) || workspace_bytes < qmx_splitk_workspace_bytes(M, N, splits))
        return QMX_ERR_WORKSPACE;
    return launch_status(qmx::launch_qmm_t(w_packed, scales, biases, x, nullptr, static_cast<float*>(workspace), 1,
                                           qmx::unbatched(K), M, N, K, bits, group_size, dtype, splits,
                                           static_cast<hipStream_t>(stream)));
}

int qmx_splitk_accumulate(const void* workspace, void* out, int M, int N, int splits, int dtype, void* stream) {
    if (splits < 2 || splits > QMX_MAX_SPLITS) return QMX_ERR_SPLITS;
    if (dtype != QMX_F16 && dtype != QMX_BF16) return QMX_ERR_DTYPE;
    if (M < 0 || N < 0) return QMX_ERR_SHAPE;
    if (M == 0 || N == 0) return QMX_OK;
    if (!out) return QMX_ERR_NULL;
    if (!workspace || !is_aligned(workspace, 16)) return QMX_ERR_WORKSPACE;
    if (!is_aligned(out, 2)) return QMX_ERR_ALIGN;
    return launch_status(qmx::launch_splitk_accum(static_cast<const float*>(workspace), out, splits,
                                                  (size_t)M * N, dtype, static_cast<hipStream_t>(stream)));
}

int qmx_qmm_t_splitk(const uint32_t* w_packed, const void* scales, const void* biases, const void* x,
                     void* out, int M, int N, int K, int bits, int group_size, int dtype, int splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (splits < 2 || splits > QMX_MAX_SPLITS) return QMX_ERR_SPLITS;
    int rc = check_qmm(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype, splits);
    if (rc) return rc;
    if (splits > max_splits_for(K)) return QMX_ERR_SPLITS;
    if (M == 0 || N == 0) return QMX_OK;
    if (!workspace || !is_aligned(workspace, 16) ||
        workspace_bytes < qmx_splitk_workspace_bytes(M, N, splits))
        return QMX_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);
    rc = launch_status(qmx::launch_qmm_t(w_packed, scales, biases, x, out, ws, 1, qmx::unbatched(K), M, N, K, bits,
                                         group_size, dtype, splits, st));
    if (rc) return rc;
    return launch_status(qmx::launch_splitk_accum(ws, out, splits, (size_t)M * N, dtype, st));
}

int qmx_matvec_q8_0(const uint32_t* w_blocks, const float* x, float* out, int N, int K, void* stream) {
    if (N < 0 || K < 0) return QMX_ERR_SHAPE;
    if (K % 32 != 0) return QMX_ERR_GROUP;
    if (N == 0) return QMX_OK;
    if (!out || (K > 0 && (!w_blocks || !x))) return QMX_ERR_NULL;
    if (!is_aligned(out, 4) || (K > 0 && (!is_aligned(w_blocks, 16) || !is_aligned(x, 16))))
        return QMX_ERR_ALIGN;
    return launch_status(qmx::launch_q8_0(w_blocks, x, out, N, K, static_cast<hipStream_t>(stream)));
}

int qmx_matvec_q4_k(const uint32_t* w_blocks, const float* x, float* out, int N, int K, void* stream) {
    if (N < 0 || K < 0) return QMX_ERR_SHAPE;
    if (K % 256 != 0) return QMX_ERR_GROUP;
    if (N == 0) return QMX_OK;
    if (!out || (K > 0 && (!w_blocks || !x))) return QMX_ERR_NULL;
    if (!is_aligned(out, 4) || (K > 0 && (!is_aligned(w_blocks, 16) || !is_aligned(x, 16))))
        return QMX_ERR_ALIGN;
    return launch_status(qmx::launch_q4_k(w_blocks, x, out, N, K, static_cast<hipStream_t>(stream)));
}

int qmx_matvec_q8_i8(const uint32_t* wq, const uint32_t* xq, const float* wd, float* out, int N, int K,
                     void* stream) {
    if (N < 0 || K < 0) return QMX_ERR_SHAPE;
    if (K % 32 != 0) return QMX_ERR_GROUP;
    // per-lane offsets of one work-group's rows stay in 32 bits
    if ((long long)16 * K > INT_MAX) return QMX_ERR_SHAPE;
    if (N == 0) return QMX_OK;
    if (!out || (K > 0 && (!wq || !xq || !wd))) return QMX_ERR_NULL;
    if (!is_aligned(out, 4) || (K > 0 && (!is_aligned(wq, 16) || !is_aligned(xq, 16) || !is_aligned(wd, 4))))
        return QMX_ERR_ALIGN;
    return launch_status(qmx::launch_q8_i8(wq, xq, wd, out, N, K, static_cast<hipStream_t>(stream)));
}

int qmx_plan(int M, int N, int K, int bits, int group_size, int dtype, int num_cus, int* route, int* splits) {
    if (!route || !splits) return QMX_ERR_NULL;
    return plan_impl(M, N, K, bits, group_size, dtype, num_cus, route, splits);
}

size_t qmx_qmm_workspace_bytes(int M, int N, int K, int bits, int group_size, int dtype) {
    int route = 0, splits = 1;
    if (plan_impl(M, N, K, bits, group_size, dtype, device_cus(), &route, &splits) != QMX_OK) return 0;
    return route == QMX_ROUTE_QMM_T_SPLITK ? qmx_splitk_workspace_bytes(M, N, splits) : 0;
}

int qmx_qmm(const uint32_t* w_packed, const void* scales, const void* biases, const void* x, void* out,
            int M, int N, int K, int bits, int group_size, int dtype, void* workspace, size_t workspace_bytes,
            void* stream) {
    int route = 0, splits = 1;
    int rc = check_affine_common(M, N, K, bits, group_size, dtype);
    if (rc) return rc;
    if (M == 0 || N == 0) return QMX_OK;
    const int cus = device_cus();
    if (cus <= 0) return QMX_ERR_DEVICE;
    rc = plan_impl(M, N, K, bits, group_size, dtype, cus, &route, &splits);
    if (rc) return rc;
    if (route == QMX_ROUTE_QMV)
        return qmx_qmv(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype, stream);
    if (route == QMX_ROUTE_QMM_T)
        return qmx_qmm_t(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype, stream);
    return qmx_qmm_t_splitk(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype, splits,
                            workspace, workspace_bytes, stream);
}

int qmx_plan_batched(int batch, int M, int N, int K, int bits, int group_size, int dtype, int num_cus, int* route,
                     int* splits) {
    if (!route || !splits) return QMX_ERR_NULL;
    if (batch < 0 || batch > 65535) return QMX_ERR_SHAPE;
    return plan_impl(M, N, K, bits, group_size, dtype, num_cus, route, splits, batch > 0 ? batch : 1);
}

size_t qmx_qmm_batched_workspace_bytes(int batch, int M, int N, int K, int bits, int group_size, int dtype,
                                       const void* x, long long x_batch_stride, long long x_row_stride) {
    return batched_workspace(batch, batch, M, N, K, bits, group_size, dtype, x, x_batch_stride, x_row_stride);
}

int qmx_qmm_batched(const uint32_t* w_packed, const void* scales, const void* biases, const void* x, void* out,
                    int batch, int M, int N, int K, long long w_batch_stride, long long sb_batch_stride,
                    long long x_batch_stride, long long x_row_stride, int bits, int group_size, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return batched_impl(w_packed, scales, biases, x, out, nullptr, nullptr, batch, batch, batch, M, N, K,
                        w_batch_stride, sb_batch_stride, x_batch_stride, x_row_stride, bits, group_size, dtype,
                        workspace, workspace_bytes, stream);
}

size_t qmx_qmm_gather_workspace_bytes(int batch, int num_x, int M, int N, int K, int bits, int group_size, int dtype,
                                      const void* x, long long x_batch_stride, long long x_row_stride) {
    if (num_x < 0) return 0;
    return batched_workspace(batch, num_x, M, N, K, bits, group_size, dtype, x, x_batch_stride, x_row_stride);
}

int qmx_qmm_gather(const uint32_t* w_packed, const void* scales, const void* biases, const void* x, void* out,
                   const int32_t* w_index, const int32_t* x_index, int num_w, int num_x, int batch, int M, int N,
                   int K, long long w_batch_stride, long long sb_batch_stride, long long x_batch_stride,
                   long long x_row_stride, int bits, int group_size, int dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
    return batched_impl(w_packed, scales, biases, x, out, w_index, x_index, w_index ? num_w : batch,
                        x_index ? num_x : batch, batch, M, N, K, w_batch_stride, sb_batch_stride, x_batch_stride,
                        x_row_stride, bits, group_size, dtype, workspace, workspace_bytes, stream);
}

int qmx_qmm_gather_sorted(const uint32_t* w_packed, const void* scales, const void* biases, const void* x,
                          void* out, const int32_t* w_index, const int32_t* x_index, int num_w, int num_x,
                          int batch, int M, int N, int K, long long w_batch_stride, long long sb_batch_stride,
                          long long x_batch_stride, long long x_row_stride, int bits, int group_size, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return batched_impl(w_packed, scales, biases, x, out, w_index, x_index, w_index ? num_w : batch,
                        x_index ? num_x : batch, batch, M, N, K, w_batch_stride, sb_batch_stride, x_batch_stride,
                        x_row_stride, bits, group_size, dtype, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
