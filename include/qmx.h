/*
 * qmx.h -- C ABI of libqmx: group-wise affine quantized matrix-vector and
 * small-M matrix multiply, and the Q8_0 / Q4_K block matvecs, for AMD MI355X
 * (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument except those named "host" is a DEVICE pointer
 *   owned by the caller.  The library never allocates, frees or copies
 *   caller memory and never synchronises: work is enqueued on `stream`
 *   (a hipStream_t; NULL means the default stream) and the call returns as
 *   soon as it is enqueued.  Outputs are valid once the stream reaches them.
 * - Arrays are dense and row-major.  `out` must not overlap any input.
 * - All arguments are validated on the host before anything is enqueued; a
 *   negative qmx_status is returned and nothing is launched when a check
 *   fails.  QMX_ERR_LAUNCH reports a launch error returned by the HIP
 *   runtime.  Empty problems (M == 0 or N == 0) return QMX_OK and launch
 *   nothing; K == 0 writes zeros.
 * - Results are bit-reproducible run to run for the same build, device,
 *   arguments and split count: no atomics, fixed reduction orders.
 * - Accumulation is float32 throughout; the output is rounded once, to
 *   nearest even.
 * - The library keeps no state between calls apart from a per-device cache
 *   of the compute-unit count; calls may come from several host threads.
 *
 * The affine format (page "metaltile-std src/mlx/quantized.rs", qmv kernel
 * header, layouts comment of the int8 kernel; page "mlx PR 4682", transposed
 * quantized_matmul):
 *   w_packed : uint32 [N, K*bits/32]; row n is a little-endian bit stream,
 *              code q[n,k] is the unsigned field at stream bits
 *              [k*bits, (k+1)*bits) (4-bit: 8 codes per word, low nibble
 *              first; 8-bit: byte j of a word is code 4*word+j; 3-, 5- and
 *              6-bit fields may straddle two words).
 *   scales, biases : [N, K/group_size] in `dtype`.
 *   x        : [M, K] in `dtype`.     out : [M, N] in `dtype`.
 *   out[m,n] = sum_g ( scales[n,g] * sum_{k in g} q[n,k] * x[m,k]
 *                    + biases[n,g] * sum_{k in g} x[m,k] )
 *            = sum_k x[m,k] * (scales[n,k/gs] * q[n,k] + biases[n,k/gs]).
 * Supported: bits in {1, 2, 3, 4, 5, 6, 8} (the widths of the staged loader
 * of page "mlx PR 4682"); group_size in {32, 64, 128}; K % group_size == 0.
 */
#ifndef QMX_H
#define QMX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMX_API_VERSION 1

typedef enum qmx_dtype {
    QMX_F32 = 0,   /* IEEE binary32 */
    QMX_F16 = 1,   /* IEEE binary16 */
    QMX_BF16 = 2   /* bfloat16 (upper half of a binary32) */
} qmx_dtype;

typedef enum qmx_status {
    QMX_OK = 0,
    QMX_ERR_NULL = -1,       /* a required pointer is NULL                        */
    QMX_ERR_SHAPE = -2,      /* negative size, or a size the route cannot take     */
    QMX_ERR_BITS = -3,       /* bits not in {1, 2, 3, 4, 5, 6, 8}                  */
    QMX_ERR_GROUP = -4,      /* group_size not in {32, 64, 128} or K % gs != 0     */
    QMX_ERR_DTYPE = -5,      /* unknown dtype, or a dtype the route does not take  */
    QMX_ERR_ALIGN = -6,      /* a pointer lacks the alignment the route needs      */
    QMX_ERR_WORKSPACE = -7,  /* split-K workspace NULL or too small                */
    QMX_ERR_SPLITS = -8,     /* split count out of range for this K                */
    QMX_ERR_LAUNCH = -9,     /* the HIP runtime rejected a launch                  */
    QMX_ERR_DEVICE = -10,    /* no usable HIP device                               */
    QMX_ERR_SCRATCH = -11    /* partials larger than qmx_qmm_t_splitk_noalloc holds */
} qmx_status;

typedef enum qmx_route {
    QMX_ROUTE_QMV = 0,          /* qmx_qmv                      */
    QMX_ROUTE_QMM_T = 1,        /* qmx_qmm_t (unsplit)          */
    QMX_ROUTE_QMM_T_SPLITK = 2  /* qmx_qmm_t_splitk + accumulate */
} qmx_route;

/* Largest split count qmx_qmm_t_splitk accepts. */
#define QMX_MAX_SPLITS 16

/* qmx_qmv -- affine quantized matvec for small M (built for M = 1..7).
 * Computes the affine definition above with float32 accumulation on the
 * vector ALUs: weight codes are streamed once in chunks of 16 bytes (2-, 4-
 * and 8-bit) or of `bits` words = 32 codes (1, 3, 5, 6 bits), the sum
 * of x is formed once per group (bias hoist), lanes are reduced with a
 * fixed-order cross-lane tree (page "metaltile-std src/mlx/quantized.rs",
 * qmv kernel: bias hoist, x reuse across rows, simd_sum and lane-0 store).
 * dtype: QMX_F32, QMX_F16 or QMX_BF16 for x, scales, biases and out.
 * Any M >= 0 is accepted (rows of x are processed in tiles of up to 4).
 * Extra requirements: rows of w_packed are whole chunks ((K*bits) % 128 == 0
 * for 2, 4 and 8 bits; K % 32 == 0, always true, for the others), w_packed
 * 16-byte aligned, x aligned to its element size.
 */
int qmx_qmv(const uint32_t* w_packed, const void* scales, const void* biases,
            const void* x, void* out, int M, int N, int K, int bits, int group_size,
            int dtype, void* stream);

/* qmx_qmm_t -- affine quantized x * W^T on the matrix cores (any M; built
 * for M >= 8, and what qmx_plan picks at M = 2..7 for large weights)
 * (page "mlx PR 4682": staged transposed qmm that fetches the next K step
 * while the current one is consumed from threadgroup memory, with one
 * barrier per K step).  Here the packed codes and x of the next K blocks are
 * copied from HBM straight into a ring of LDS stages (global-to-LDS loads,
 * no register staging) while the matrix cores consume the current stage;
 * scales and biases are staged once per work-group in 16-byte chunks when
 * aligned, else with each stage.  Codes are expanded to exact 16-bit values
 * right before bf16/f16 MFMA, and scale and bias are applied per group in
 * float32, so the only rounding besides float32 accumulation is the final
 * one.
 * dtype: QMX_F16 or QMX_BF16 only (QMX_ERR_DTYPE for QMX_F32).
 * Extra requirements: K % 128 == 0; w_packed, x 16-byte aligned.
 */
int qmx_qmm_t(const uint32_t* w_packed, const void* scales, const void* biases,
              const void* x, void* out, int M, int N, int K, int bits, int group_size,
              int dtype, void* stream);

/* qmx_qmm_t_splitk -- qmx_qmm_t with K split into `splits` partitions
 * (page "mlx PR 4682": split-K kernel writing float32 partials that a
 * separate accumulate kernel sums, rounding once).  K is cut into segments
 * of 256 columns (of 128 columns when K is not a multiple of 256), and
 * partition p covers segments [floor(p*nseg/splits), floor((p+1)*nseg/splits))
 * with nseg = K/segment; each partition must hold at least 256 columns, so
 * 2 <= splits <= min(QMX_MAX_SPLITS, K/256).  The first kernel writes
 * workspace[p][m][n] (float32); the second sums p = 0..splits-1 in that
 * order and rounds once to `dtype`.  workspace: device memory of at least
 * qmx_splitk_workspace_bytes(M, N, splits) bytes, 16-byte aligned, owned by
 * the caller, overwritten by the call (its contents on entry do not
 * matter); calls that share one workspace must be ordered on one stream.
 * Other requirements as qmx_qmm_t.
 */
int qmx_qmm_t_splitk(const uint32_t* w_packed, const void* scales, const void* biases,
                     const void* x, void* out, int M, int N, int K, int bits, int group_size,
                     int dtype, int splits, void* workspace, size_t workspace_bytes,
                     void* stream);

/* qmx_qmm_t_partials -- the first kernel of qmx_qmm_t_splitk on its own:
 * writes partition p's float32 sums into workspace[p][m][n] for
 * p = 0..splits-1 (the split-K partial kernel of page "mlx PR 4682") and
 * touches nothing else.  Arguments, partitions and requirements are those
 * of qmx_qmm_t_splitk without `out`; a NULL or short workspace is
 * QMX_ERR_WORKSPACE. */
int qmx_qmm_t_partials(const uint32_t* w_packed, const void* scales, const void* biases,
                       const void* x, int M, int N, int K, int bits, int group_size,
                       int dtype, int splits, void* workspace, size_t workspace_bytes,
                       void* stream);

/* qmx_splitk_accumulate -- the second kernel of qmx_qmm_t_splitk on its own
 * (the separate accumulate kernel of page "mlx PR 4682"):
 * out[m][n] = round(sum over p = 0..splits-1, in that order, of
 * workspace[p][m][n]), float32 sums rounded once to `dtype` (QMX_F16 or
 * QMX_BF16).  workspace: splits*M*N float32, 16-byte aligned; out: M*N
 * elements.  2 <= splits <= QMX_MAX_SPLITS. */
int qmx_splitk_accumulate(const void* workspace, void* out, int M, int N, int splits, int dtype,
                          void* stream);

/* Bytes of float32 partials qmx_qmm_t_splitk needs: splits * M * N * 4
 * (0 for negative arguments). */
size_t qmx_splitk_workspace_bytes(int M, int N, int splits);

/* Size of the per-device scratch array of qmx_qmm_t_splitk_noalloc. */
#define QMX_NOALLOC_SCRATCH_BYTES (16u << 20)

/* qmx_qmm_t_splitk_noalloc -- qmx_qmm_t_splitk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, partitions, results and
 * errors as qmx_qmm_t_splitk without the workspace: the float32 partials go
 * into a scratch array of QMX_NOALLOC_SCRATCH_BYTES that this library holds
 * on each device it runs on until the process ends (16 MiB covers every
 * split qmx_plan picks on a 256-CU device: splits * tiles <= CUs, a tile at
 * most 128 x 128 floats).  QMX_ERR_SCRATCH when splits * M * N * 4 exceeds
 * it.  Nothing is allocated or freed: the array's device address is looked
 * up once per device (QMX_ERR_DEVICE if that fails).  Every call on one
 * device shares that device's array and nothing in it needs clearing; calls
 * that overlap on one device (e.g. on two streams) race on it and must be
 * ordered by the caller. */
int qmx_qmm_t_splitk_noalloc(const uint32_t* w_packed, const void* scales, const void* biases,
                             const void* x, void* out, int M, int N, int K, int bits, int group_size,
                             int dtype, int splits, void* stream);

/* qmx_matvec_q8_0 -- Q8_0 block matvec, M = 1 (page "hanzo-kernel
 * src/quant.rs": Q8_0 matvec and its packed layout).
 * w_blocks: uint32 [N, K/32*9]; each 32-weight block is 9 words, the f16
 * scale d in the low 16 bits of word 0 and 32 signed int8 quants in words
 * 1..8 (quant i at byte i%4 of word 1+i/4).  x: float32 [K]; out: float32
 * [N];  out[n] = sum_blocks d * sum_i q_i * x[32*block+i].
 * Requirements: K % 32 == 0; w_blocks and x 16-byte aligned.
 */
int qmx_matvec_q8_0(const uint32_t* w_blocks, const float* x, float* out, int N, int K,
                    void* stream);

/* qmx_matvec_q4_k -- Q4_K super-block matvec, M = 1 (page "hanzo-kernel
 * src/quant.rs": Q4_K block comment, scale/min unpack and kernel).
 * w_blocks: uint32 [N, K/256*36]; each 144-byte super-block holds f16 d
 * (bytes 0-1), f16 dmin (bytes 2-3), 12 bytes of packed 6-bit scales and
 * mins (bytes 4-15) and 128 bytes of 4-bit quants (bytes 16-143).  Quant
 * byte 32g+i gives element 64g+i (low nibble, sub-block 2g) and element
 * 64g+32+i (high nibble, sub-block 2g+1); the weight of code q in sub-block
 * j is d*sc_j*q - dmin*m_j.  x: float32 [K]; out: float32 [N].
 * Requirements: K % 256 == 0; w_blocks and x 16-byte aligned.
 */
int qmx_matvec_q4_k(const uint32_t* w_blocks, const float* x, float* out, int N, int K,
                    void* stream);

/* qmx_matvec_q8_i8 -- integer-activation matvec (page "hanzo-kernel
 * src/quant.rs", packed-int8 dp4a matvec and its block-per-row form):
 *   out[n] = sum_b wd[n*K/32 + b] * sum_{i in block b} wq[n][i] * xq[i]
 * wq: int8 weights [N][K] packed four to a uint32 (element i at byte i % 4,
 * two's complement); xq: int8 activations [K] packed the same way; wd:
 * float32 [N][K/32], one scale per 32-element block of a row; out: float32
 * [N].  Each block's integer sum is exact (4-way integer dot instructions);
 * the scaled blocks are summed in float32.  Requirements: K % 32 == 0
 * (QMX_ERR_GROUP), wq and xq 16-byte aligned, wd and out 4-byte aligned
 * (QMX_ERR_ALIGN); K = 0 writes zeros.  Device pointers, caller-owned,
 * asynchronous on `stream`.
 */
int qmx_matvec_q8_i8(const uint32_t* wq, const uint32_t* xq, const float* wd, float* out,
                     int N, int K, void* stream);

/* qmx_plan -- the dispatch policy as a pure host function (page "mlx PR
 * 4682", dispatch table and split rule; page "metaltile-std
 * src/mlx/quantized.rs", M-based kernel selector).  Writes the route
 * (qmx_route) and split count (1 when unsplit) that qmx_qmm would use for
 * this problem on a device with `num_cus` compute units (num_cus <= 0:
 * 256).  Routes: float32 activations, K % 128 != 0 and M = 1 take qmx_qmv;
 * M = 2..7 takes qmx_qmv unless a cost estimate (qmv's vector work grows
 * with M, the matrix route with the weight bytes) favours the matrix cores;
 * otherwise qmx_qmm_t, split along K when its tiles leave compute units idle
 * (tiles of 128 columns by up to 64 rows of x; above M = 192 by up to 128
 * rows when those fill the device or launch more work-groups after the
 * split; for 2-, 4- and 8-bit codes split tiles of 64 columns at half the
 * partitions where they fit one round of the device, and unsplit tiles of
 * 16 or 32 columns for M <= 32 where few columns would leave compute units
 * idle).  Performs no HIP call.  Returns QMX_OK or a validation status.
 * route/splits: host pointers.
 */
int qmx_plan(int M, int N, int K, int bits, int group_size, int dtype, int num_cus,
             int* route, int* splits);

/* Workspace bytes qmx_qmm needs for this problem (0 unless the plan picks
 * split-K) on the current device.  Host function; may query the device's
 * compute-unit count once. */
size_t qmx_qmm_workspace_bytes(int M, int N, int K, int bits, int group_size, int dtype);

/* qmx_qmm -- the policy-dispatched entry: runs qmx_qmv, qmx_qmm_t or
 * qmx_qmm_t_splitk as qmx_plan decides for the current device.  workspace
 * may be NULL when qmx_qmm_workspace_bytes() is 0; otherwise it must be at
 * least that large (QMX_ERR_WORKSPACE if not). */
int qmx_qmm(const uint32_t* w_packed, const void* scales, const void* biases,
            const void* x, void* out, int M, int N, int K, int bits, int group_size,
            int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* qmx_strerror(int status);

/* QMX_API_VERSION of the built library. */
int qmx_api_version(void);

/* qmx_qmm_batched -- qmx_qmm over a batch of independent problems of one
 * shape: 3-D (batched) quantized weights, strided activations and
 * activations at any element offset (page "mlx PR 4682": the batched
 * transposed qmm, its test of 3-D quantized weights with strided and
 * odd-offset activations, and activations that are not suitably aligned
 * being copied first).
 *   out[i][m][n] = sum_k x_i[m][k] * (s_i[n,k/gs] * q_i[n,k] + b_i[n,k/gs])
 * for i < batch, where
 *   weights i  : w_packed + i*w_batch_stride words (0 shares one matrix;
 *                a multiple of 4, so every matrix is 16-byte aligned),
 *   scales/biases i : + i*sb_batch_stride elements (0 shares them),
 *   x_i rows   : x + i*x_batch_stride + m*x_row_stride elements
 *                (x_row_stride >= K; any element offset),
 *   out        : contiguous [batch][M][N] in `dtype`.
 * Each matrix has the layout of the unbatched calls.  Routes and splits
 * follow qmx_plan_batched (one launch for the whole batch; split-K partials
 * are [S][batch][M][N]).  When x, x_batch_stride or x_row_stride is not
 * 16-byte aligned, x is first copied into the workspace as a contiguous
 * [batch][M][K] array.  workspace: at least
 * qmx_qmm_batched_workspace_bytes(...) bytes, 256-byte aligned, may be NULL
 * when that is 0; contents on entry do not matter; calls sharing one
 * workspace must be ordered on one stream.
 * Errors: as qmx_qmm; QMX_ERR_SHAPE for batch outside [0, 65535], a
 * negative stride or x_row_stride < K; QMX_ERR_ALIGN for a weight stride
 * that is not a multiple of 4 words.
 */
int qmx_qmm_batched(const uint32_t* w_packed, const void* scales, const void* biases,
                    const void* x, void* out, int batch, int M, int N, int K,
                    long long w_batch_stride, long long sb_batch_stride,
                    long long x_batch_stride, long long x_row_stride, int bits,
                    int group_size, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Workspace bytes qmx_qmm_batched needs (split-K partials as planned on the
 * current device, plus the copy of x when x or its strides are not 16-byte
 * aligned; x is only inspected, never dereferenced).  0 on invalid input. */
size_t qmx_qmm_batched_workspace_bytes(int batch, int M, int N, int K, int bits, int group_size,
                                       int dtype, const void* x, long long x_batch_stride,
                                       long long x_row_stride);

/* qmx_qmm_gather -- qmx_qmm_batched where problem i takes weight matrix
 * w_index[i] (of num_w) and activation matrix x_index[i] (of num_x) instead
 * of matrix i (page "mlx PR 4682": gathered qmm, the batched route with
 * per-problem weight selection, as mixture-of-experts layers use it).
 *   out[i] = x_{x_index[i]} * dequant(W_{w_index[i]})^T,  i < batch
 * w_index, x_index: device arrays of `batch` int32, 4-byte aligned, owned by
 * the caller and read by the kernels (so not checked on the host): a value
 * outside [0, count - 1] is clamped to that range.  Either may be NULL for
 * the identity (then that operand has `batch` matrices).  Strides, layouts,
 * routes, workspace (qmx_qmm_gather_workspace_bytes; a misaligned x is
 * copied as num_x matrices) and errors as qmx_qmm_batched; QMX_ERR_SHAPE
 * also for num_w or num_x < 1 with a non-empty batch.
 */
int qmx_qmm_gather(const uint32_t* w_packed, const void* scales, const void* biases,
                   const void* x, void* out, const int32_t* w_index, const int32_t* x_index,
                   int num_w, int num_x, int batch, int M, int N, int K,
                   long long w_batch_stride, long long sb_batch_stride,
                   long long x_batch_stride, long long x_row_stride, int bits, int group_size,
                   int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes qmx_qmm_gather needs (num_x: the activation matrices, or
 * `batch` when x_index is NULL). */
size_t qmx_qmm_gather_workspace_bytes(int batch, int num_x, int M, int N, int K, int bits,
                                      int group_size, int dtype, const void* x,
                                      long long x_batch_stride, long long x_row_stride);

/* qmx_qmm_gather_sorted -- qmx_qmm_gather for a w_index that holds runs of
 * equal values, as a mixture-of-experts router's output does once the
 * problems are ordered by expert (the gathered qmm of page "mlx PR 4682";
 * the grouping below is this library's).  Arguments, workspace
 * (qmx_qmm_gather_workspace_bytes), results within the same tolerance, and
 * errors as qmx_qmm_gather, for any index arrays: sortedness only decides
 * how much work is shared, never what is computed.
 * At M = 1 on the vector route, one work-group serves up to g consecutive
 * problems whose clamped w_index values are equal, as the x rows of one tile,
 * so a run of problems on one weight matrix streams those weights once
 * rather than once per problem.  g = 1, 2 or 4 is the run length that
 * batch / num_w suggests (rounded up; 4 from 3 on).  Runs are cut at
 * multiples of g.  Other shapes, and x matrices spanning 2 GiB or more, run
 * as qmx_qmm_gather.  Reruns with the same inputs are bit-identical; the
 * float32 summation order can differ from qmx_qmm_gather's.
 */
int qmx_qmm_gather_sorted(const uint32_t* w_packed, const void* scales, const void* biases,
                          const void* x, void* out, const int32_t* w_index,
                          const int32_t* x_index, int num_w, int num_x, int batch, int M, int N,
                          int K, long long w_batch_stride, long long sb_batch_stride,
                          long long x_batch_stride, long long x_row_stride, int bits,
                          int group_size, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* qmx_plan for a batch: the tiles of all problems share the device, so a
 * batch needs fewer K partitions.  Pure host function. */
int qmx_plan_batched(int batch, int M, int N, int K, int bits, int group_size, int dtype,
                     int num_cus, int* route, int* splits);

#ifdef __cplusplus
}
#endif

#endif /* QMX_H */
