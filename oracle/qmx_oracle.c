/*
 * qmx_oracle.c -- plain, slow, float64 CPU reference for the quantized
 * matvec / small-M matmul family.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this file.  It shares no
 * code, header, table or constant with the HIP library; it decodes every
 * stored value itself, from the IEEE-754 definitions and the layouts the
 * pages state.
 *
 * Every result is the plain definition written out, summed serially in index
 * order in float64.  Rows are spread over OpenMP threads, but each output is
 * summed by one thread in one fixed order, so the result does not depend on
 * the thread count.
 *
 * Storage dtype codes: 0 = float32, 1 = float16 (IEEE binary16), 2 = bfloat16.
 *
 * Parity pins: every entry point below is pinned by the CPU tests (exact
 * rational brute force on tiny inputs, one-hot probes against the stated
 * layouts, a dense numpy dequantise-then-matmul, closed forms and special
 * cases).  No function here is "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);              /* zero and subnormals */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);          /* (1024+f) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32. */
static double dec_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double value_at(const void* p, int dt, size_t i) {
    if (dt == OR_F32) return (double)((const float*)p)[i];
    uint16_t h = ((const uint16_t*)p)[i];
    return dt == OR_F16 ? dec_f16(h) : dec_bf16(h);
}

static int dtype_ok(int dt) { return dt == OR_F32 || dt == OR_F16 || dt == OR_BF16; }

/* Unsigned code k of a row whose codes form one little-endian bit stream:
 * bits [k*bits, (k+1)*bits) of the stream, word 0 holding stream bits 0..31.
 * A field may straddle two words (odd widths). */
static unsigned code_at(const uint32_t* row, long k, int bits) {
    long bit = k * (long)bits;
    long wi = bit >> 5;
    int sh = (int)(bit & 31);
    uint64_t window = row[wi];
    if (sh + bits > 32) window |= (uint64_t)row[wi + 1] << 32;
    return (unsigned)((window >> sh) & ((1u << bits) - 1u));
}

static int affine_args_ok(int M, int N, int K, int bits, int gs, int sb_dt, int x_dt) {
    if (M < 0 || N < 0 || K < 0) return 0;
    if (bits < 1 || bits > 8 || gs <= 0 || K % gs) return 0;
    if (((long)K * bits) % 32) return 0;
    return dtype_ok(sb_dt) && dtype_ok(x_dt);
}

/* out[m, c] = sum_{k in [g0*gs, g1*gs)} x[m,k] * (s[n,k/gs]*q[n,k] + b[n,k/gs]),
 * n = cols ? cols[c] : c.  This is the group-wise affine definition (pages:
 * "metaltile-std quantized.rs", qmv kernel header "Math" comment; "mlx PR 4682",
 * transposed quantized_matmul), with the sum restricted to a range of groups so
 * that the split-K partitions can be checked one by one.  out is [M, ncols]. */
int oracle_affine_groups(const uint32_t* w, const void* s, const void* b, int sb_dt,
                         const void* x, int x_dt, int M, int N, int K, int bits, int gs,
                         int g0, int g1, const int32_t* cols, int ncols, double* out) {
    if (!affine_args_ok(M, N, K, bits, gs, sb_dt, x_dt)) return -1;
    int G = gs ? K / gs : 0;
    if (g0 < 0 || g1 > G || g0 > g1) return -1;
    int nc = cols ? ncols : N;
    long words_per_row = (long)K * bits / 32;
    long total = (long)M * nc;
#pragma omp parallel for schedule(dynamic, 16)
    for (long idx = 0; idx < total; ++idx) {
        int m = (int)(idx / nc), c = (int)(idx % nc);
        int n = cols ? cols[c] : c;
        const uint32_t* row = w + (long)n * words_per_row;
        double acc = 0.0;
        for (long k = (long)g0 * gs; k < (long)g1 * gs; ++k) {
            long g = k / gs;
            double wk = value_at(s, sb_dt, (size_t)n * G + g) * (double)code_at(row, k, bits)
                      + value_at(b, sb_dt, (size_t)n * G + g);
            acc += value_at(x, x_dt, (size_t)m * K + k) * wk;
        }
        out[idx] = acc;
    }
    return 0;
}

/* The full contraction over all K: the dequantise-then-dot definition. */
int oracle_affine(const uint32_t* w, const void* s, const void* b, int sb_dt,
                  const void* x, int x_dt, int M, int N, int K, int bits, int gs,
                  const int32_t* cols, int ncols, double* out) {
    if (!affine_args_ok(M, N, K, bits, gs, sb_dt, x_dt)) return -1;
    return oracle_affine_groups(w, s, b, sb_dt, x, x_dt, M, N, K, bits, gs,
                                0, K / gs, cols, ncols, out);
}

/* The same quantity in the bias-hoisted form the pages use:
 * out[m,n] = sum_g ( s[n,g] * sum_{i in g} q[n,i] x[m,i] + b[n,g] * sum_{i in g} x[m,i] )
 * (page "metaltile-std quantized.rs", qmv header "Math" and the bias hoist). */
int oracle_affine_hoisted(const uint32_t* w, const void* s, const void* b, int sb_dt,
                          const void* x, int x_dt, int M, int N, int K, int bits, int gs,
                          double* out) {
    if (!affine_args_ok(M, N, K, bits, gs, sb_dt, x_dt)) return -1;
    int G = K / gs;
    long words_per_row = (long)K * bits / 32;
    long total = (long)M * N;
#pragma omp parallel for schedule(dynamic, 16)
    for (long idx = 0; idx < total; ++idx) {
        int m = (int)(idx / N), n = (int)(idx % N);
        const uint32_t* row = w + (long)n * words_per_row;
        double acc = 0.0;
        for (int g = 0; g < G; ++g) {
            double qx = 0.0, xs = 0.0;
            for (int i = 0; i < gs; ++i) {
                long k = (long)g * gs + i;
                double xv = value_at(x, x_dt, (size_t)m * K + k);
                qx += (double)code_at(row, k, bits) * xv;
                xs += xv;
            }
            acc += value_at(s, sb_dt, (size_t)n * G + g) * qx
                 + value_at(b, sb_dt, (size_t)n * G + g) * xs;
        }
        out[idx] = acc;
    }
    return 0;
}

/* Q8_0 block matvec (page "hanzo-kernel quant.rs", Q8_0 matvec and the packed
 * Q8_0 layout): each 32-weight block is 9 words; the f16 scale d is the low
 * half of word 0, quant i is the signed byte i%4 of word 1+i/4, and
 * out[n] = sum_blocks d * sum_i q_i * x[32*blk + i]. */
int oracle_q8_0(const uint32_t* blocks, const float* x, int N, int K,
                const int32_t* rows, int nrows, double* out) {
    if (N < 0 || K < 0 || K % 32) return -1;
    int nb = K / 32;
    int nr = rows ? nrows : N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int r = 0; r < nr; ++r) {
        int n = rows ? rows[r] : r;
        const uint32_t* rw = blocks + (long)n * nb * 9;
        double acc = 0.0;
        for (int j = 0; j < nb; ++j) {
            const uint32_t* blk = rw + (long)j * 9;
            double d = dec_f16((uint16_t)(blk[0] & 0xFFFFu));
            double bs = 0.0;
            for (int i = 0; i < 32; ++i) {
                uint32_t byte = (blk[1 + i / 4] >> (8 * (i % 4))) & 0xFFu;
                int q = byte >= 128 ? (int)byte - 256 : (int)byte;
                bs += (double)q * (double)x[32 * j + i];
            }
            acc += d * bs;
        }
        out[r] = acc;
    }
    return 0;
}

/* Integer-activation matvec (page "hanzo-kernel src/quant.rs", packed-int8
 * dp4a matvec and its block-per-row form): int8 weights wq[N][K] and int8
 * activations xq[K], both packed four to a word (element i at byte i % 4 of
 * word i / 4, two's complement), one float32 scale wd[n][b] per 32-element
 * block:  out[n] = sum_b wd[n][b] * sum_{i in block b} wq[n][i] * xq[i].
 * Each block's integer sum is exact in an int64; the scaled blocks are
 * summed in float64. */
static int sbyte(const uint32_t* wds, long i) {
    unsigned v = (wds[i / 4] >> (8 * (i % 4))) & 0xFFu;
    return v >= 128 ? (int)v - 256 : (int)v;
}

int oracle_q8_i8(const uint32_t* wq, const uint32_t* xq, const float* wd, int N, int K,
                 const int32_t* rows, int nrows, double* out) {
    if (N < 0 || K < 0 || K % 32) return -1;
    int nb = K / 32;
    int nr = rows ? nrows : N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int r = 0; r < nr; ++r) {
        int n = rows ? rows[r] : r;
        const uint32_t* rw = wq + (long)n * (K / 4);
        double acc = 0.0;
        for (int b = 0; b < nb; ++b) {
            long long dot = 0;
            for (int i = 32 * b; i < 32 * b + 32; ++i) dot += (long long)sbyte(rw, i) * sbyte(xq, i);
            acc += (double)wd[(long)n * nb + b] * (double)dot;
        }
        out[r] = acc;
    }
    return 0;
}

/* Byte i of a little-endian sequence of words. */
static unsigned byte_of(const uint32_t* wds, int i) {
    return (wds[i / 4] >> (8 * (i % 4))) & 0xFFu;
}

/* 6-bit scale (want_min = 0) or min (want_min = 1) of sub-block j (0..7) from
 * the 12 packed bytes s[0..11] (page "hanzo-kernel quant.rs", the Q4_K scale
 * and min unpack): for j < 4 the scale is s[j] & 63 and the min s[j+4] & 63;
 * for j >= 4 the scale is (s[j+4] & 15) | ((s[j-4] >> 6) << 4) and the min is
 * (s[j+4] >> 4) | ((s[j] >> 6) << 4). */
static unsigned q4k_field(const uint32_t* scale_words, int j, int want_min) {
    if (j < 4)
        return byte_of(scale_words, want_min ? j + 4 : j) & 63u;
    if (!want_min)
        return (byte_of(scale_words, j + 4) & 15u) | ((byte_of(scale_words, j - 4) >> 6) << 4);
    return (byte_of(scale_words, j + 4) >> 4) | ((byte_of(scale_words, j) >> 6) << 4);
}

/* Q4_K super-block matvec (page "hanzo-kernel quant.rs", Q4_K block layout,
 * kernel and CPU reference): a 144-byte block holds f16 d, f16 dmin, 12 scale
 * bytes and 128 quant bytes.  For g in 0..3 and i in 0..31, quant byte 32g+i
 * gives element 64g+i through its low nibble (sub-block 2g) and element
 * 64g+32+i through its high nibble (sub-block 2g+1); the weight of a code q in
 * sub-block j is d*sc_j*q - dmin*m_j. */
int oracle_q4_k(const uint32_t* blocks, const float* x, int N, int K,
                const int32_t* rows, int nrows, double* out) {
    if (N < 0 || K < 0 || K % 256) return -1;
    int nb = K / 256;
    int nr = rows ? nrows : N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int r = 0; r < nr; ++r) {
        int n = rows ? rows[r] : r;
        const uint32_t* rw = blocks + (long)n * nb * 36;
        double acc = 0.0;
        for (int blk = 0; blk < nb; ++blk) {
            const uint32_t* bw = rw + (long)blk * 36;
            double d = dec_f16((uint16_t)(bw[0] & 0xFFFFu));
            double dmin = dec_f16((uint16_t)(bw[0] >> 16));
            const uint32_t* sw = bw + 1;   /* bytes 4..15  */
            const uint32_t* qw = bw + 4;   /* bytes 16..143 */
            const float* xb = x + (long)blk * 256;
            for (int g = 0; g < 4; ++g) {
                double d1 = d * q4k_field(sw, 2 * g, 0), m1 = dmin * q4k_field(sw, 2 * g, 1);
                double d2 = d * q4k_field(sw, 2 * g + 1, 0), m2 = dmin * q4k_field(sw, 2 * g + 1, 1);
                for (int i = 0; i < 32; ++i) {
                    unsigned qb = byte_of(qw, 32 * g + i);
                    acc += (d1 * (double)(qb & 15u) - m1) * (double)xb[64 * g + i];
                    acc += (d2 * (double)(qb >> 4) - m2) * (double)xb[64 * g + 32 + i];
                }
            }
        }
        out[r] = acc;
    }
    return 0;
}

/* Round to the nearest value with p significant bits, ties to even, with
 * gradual underflow below 2^emin and overflow to infinity above maxv. */
static double round_sig(double v, int p, int emin, double maxv) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    (void)frexp(v, &e);          /* v = f * 2^e, 0.5 <= |f| < 1 */
    int ex = e - 1;              /* v = m * 2^ex, 1 <= |m| < 2  */
    if (ex < emin) ex = emin;
    double ulp = ldexp(1.0, ex - (p - 1));
    double r = nearbyint(v / ulp) * ulp;   /* default rounding mode: to nearest, ties to even */
    if (fabs(r) > maxv) r = copysign(INFINITY, v);
    return r;
}

/* Round float64 values to a storage dtype (round-to-nearest-even, directly
 * from float64, no double rounding); the results are returned as float64. */
int oracle_round(const double* in, long n, int dt, double* out) {
    if (!dtype_ok(dt)) return -1;
    for (long i = 0; i < n; ++i) {
        double v = in[i];
        if (dt == OR_F32) out[i] = round_sig(v, 24, -126, 3.4028234663852886e38);
        else if (dt == OR_F16) out[i] = round_sig(v, 11, -14, 65504.0);
        else out[i] = round_sig(v, 8, -126, 3.3895313892515355e38);
    }
    return 0;
}

/* Decode storage values (float32, f16 or bf16 bits) to float64. */
int oracle_decode(const void* in, long n, int dt, double* out) {
    if (!dtype_ok(dt)) return -1;
    for (long i = 0; i < n; ++i) out[i] = value_at(in, dt, (size_t)i);
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
