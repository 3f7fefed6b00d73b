// blocks.hip -- llama.cpp-style Q8_0 and Q4_K block matvecs (M = 1) on gfx950.
//
// Formats and arithmetic follow page "hanzo-kernel src/quant.rs" (Q8_0
// packed layout: 9 words per 32 weights; Q4_K: 144-byte super-blocks with
// 6-bit sub-block scales and mins).  Both kernels are weight-bandwidth
// bound.  Rows of up to 6144 (Q8_0) or 8192 (Q4_K) values take a deep form: a
// work-group of 4 waves stages the whole row of float32 x in LDS once, and
// every wave issues the loads of all its rounds before consuming the first,
// as straight-line code (2 rows per wave for Q8_0, 5 for Q4_K).  Longer rows
// take the looped form: 8 rows per wave for Q8_0 and 5 for Q4_K (both at 3
// waves per SIMD), walking K in rounds of 2048 values whose x is loaded once
// per work-group (two 16-byte loads per thread) and shared through LDS, with
// the next round's weights requested while the current one is consumed.
// Accumulation is float32 and each row ends with a fixed-order wave reduction.
#include "qmx_device.h"
#include "qmx_internal.h"

namespace qmx {

constexpr int Q8_ROWS = 8;                          // output rows per wave: Q8_0
constexpr int Q4K_ROWS = 5;                         // and Q4_K
constexpr int BLK_WAVES = 4;                        // waves per work-group
constexpr int BLK_THREADS = 64 * BLK_WAVES;
constexpr int BLK_ROUND = 2048;                     // x values per round (8 KB)
constexpr int BLK_XPT = BLK_ROUND / 4 / BLK_THREADS;   // 16-byte x pieces per thread per round
static_assert(BLK_XPT >= 1 && BLK_XPT * BLK_THREADS * 4 == BLK_ROUND, "x round split");

// The round's x as 512 16-byte pieces.  Piece u (x values 4u..4u+3 of the
// round) is stored at slot u ^ ((u >> 4) & 15), which spreads the pieces the
// lanes of a wave read together over distinct banks.
__device__ __forceinline__ int x_slot(int u) { return u ^ ((u >> 4) & 15); }

// Load the round starting at x value k0 (clamped into [0, K)): thread t takes
// pieces BLK_XPT*t .. BLK_XPT*t + BLK_XPT - 1.
__device__ __forceinline__ void x_round_load(const float* __restrict__ x, int K, int k0, int tid,
                                             u32x4 (&v)[BLK_XPT]) {
#pragma unroll
    for (int j = 0; j < BLK_XPT; ++j) {
        const int e = min(k0 + 4 * (BLK_XPT * tid + j), K - 4);
        v[j] = *reinterpret_cast<const u32x4*>(x + e);
    }
}

__device__ __forceinline__ void x_round_store(u32x4* buf, int tid, const u32x4 (&v)[BLK_XPT]) {
#pragma unroll
    for (int j = 0; j < BLK_XPT; ++j) buf[x_slot(BLK_XPT * tid + j)] = v[j];
}

__device__ __forceinline__ void x_piece(const u32x4* buf, int u, float* dst) {
    const u32x4 d = buf[x_slot(u)];
    dst[0] = __uint_as_float(d.x);
    dst[1] = __uint_as_float(d.y);
    dst[2] = __uint_as_float(d.z);
    dst[3] = __uint_as_float(d.w);
}

// Per-round skeleton shared by both formats: while round r is consumed, the
// weights of round r + 1 are already requested into the other register set and
// its x is loaded, then staged into the other LDS buffer; one barrier per round.
template <typename WStage, typename Load, typename Consume>
__device__ __forceinline__ void blk_rounds(const float* __restrict__ x, int K, int rounds, int tid,
                                           u32x4 (*xl)[BLK_ROUND / 4], Load&& load, Consume&& consume) {
    u32x4 v[BLK_XPT];
    WStage a, b;
    load(0, a);
    x_round_load(x, K, 0, tid, v);
    x_round_store(xl[0], tid, v);
    __syncthreads();
    // past the last round the loads repeat the last round and are never used
    auto step = [&](int rd, const WStage& cur, WStage& nxt) {
        const int rn = min(rd + 1, rounds - 1);
        load(rn, nxt);
        x_round_load(x, K, rn * BLK_ROUND, tid, v);
        consume(xl[rd & 1], rd, cur);
        x_round_store(xl[(rd + 1) & 1], tid, v);
        __syncthreads();
    };
    // two rounds per trip, alternating the register sets, so no set is copied
    for (int rd = 0; rd < rounds; rd += 2) {
        step(rd, a, b);
        if (rd + 1 < rounds) step(rd + 1, b, a);
    }
}

template <int ROWS>
__device__ __forceinline__ void blk_store(float (&acc)[ROWS], int lane, int n0, int N, float* __restrict__ out) {
    // the same fixed butterfly as wave_sum, step-major so the rows' exchanges of a
    // step share one wait
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) acc[r] += __shfl_xor(acc[r], off, 64);
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        if (lane == r) mine = acc[r];
    if (lane < ROWS && n0 + lane < N) out[n0 + lane] = mine;
}

// ---------------------------------------------------------------- Q8_0
// In round rd, lane l takes block 64*rd + l of its rows (x values 32l..32l+31
// of the round).  A signed byte q is read as the unsigned byte q ^ 0x80 =
// q + 128, and the 128 * sum(x) it adds is taken off once per block:
// sum_i q_i x_i = sum_i (q_i + 128) x_i - 128 sum_i x_i.
// One round of a wave's Q8_0 rows: lane l's block of each row against the
// round's x (buf: its 512 pieces, swizzled by x_slot); act is false for a lane
// whose block lies past the row.
template <int ROWS>
__device__ __forceinline__ void q8_0_round(const u32x4* buf, bool act, const uint32_t (&w)[ROWS][9], int lane,
                                           float (&acc)[ROWS]) {
    float xv[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) x_piece(buf, 8 * lane + i, xv + 4 * i);
    float xs = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) xs += xv[i];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const float d = f16_bits_to_f32(w[r][0] & 0xffffu);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t wd = w[r][1 + j] ^ 0x80808080u;
#pragma unroll
            for (int i = 0; i < 4; ++i) s = fmaf((float)((wd >> (8 * i)) & 0xffu), xv[4 * j + i], s);
        }
        const float add = d * fmaf(-128.f, xs, s);
        acc[r] += act ? add : 0.f;
    }
}

__global__ __launch_bounds__(BLK_THREADS) void q8_0_kernel(const uint32_t* __restrict__ wb,
                                                           const float* __restrict__ x,
                                                           float* __restrict__ out, int N, int K) {
    __shared__ u32x4 xl[2][BLK_ROUND / 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = (blockIdx.x * BLK_WAVES + wave) * Q8_ROWS;
    const int nb = K / 32;
    float acc[Q8_ROWS] = {};

    struct WS { uint32_t w[Q8_ROWS][9]; };
    if (nb > 0) {
        auto load = [&](int rd, WS& st) {
            const int b = min(64 * rd + lane, nb - 1);
#pragma unroll
            for (int r = 0; r < Q8_ROWS; ++r) {
                const uint32_t* blk = wb + ((size_t)min(n0 + r, N - 1) * nb + b) * 9;
#pragma unroll
                for (int j = 0; j < 9; ++j) st.w[r][j] = blk[j];
            }
        };
        blk_rounds<WS>(x, K, (nb + 63) / 64, tid, xl, load, [&](const u32x4* buf, int rd, const WS& st) {
            q8_0_round<Q8_ROWS>(buf, 64 * rd + lane < nb, st.w, lane, acc);
        });
    }
    blk_store(acc, lane, n0, N, out);
}

// Short rows (at most NR rounds of 64 blocks) with Q8_DEEP_ROWS rows per wave:
// the whole row of x is staged in LDS once and every wave issues the loads of
// all its rounds before consuming the first (as the deep Q4_K form below).
// Measured against the looped kernel over N = 4096..27648, K = 2048..6144: 1.1-
// 1.6x faster at 2 rows per wave (14336 x 5120: 20.2 -> 17.9 us); 1, 3, 4 and
// 6 rows were up to 9% slower than 2.
constexpr int Q8_DEEP_ROWS = 2;
constexpr int Q8_DEEP_MAX_ROUNDS = 3;

template <int NR>
__global__ __launch_bounds__(BLK_THREADS) void q8_0_deep_kernel(const uint32_t* __restrict__ wb,
                                                                const float* __restrict__ x,
                                                                float* __restrict__ out, int N, int K) {
    constexpr int R = Q8_DEEP_ROWS;
    constexpr int XPIECES = NR * BLK_ROUND / 4;
    constexpr int XPT = XPIECES / BLK_THREADS;
    static_assert(XPT * BLK_THREADS == XPIECES && XPT + 9 * NR * R < 64 * 4, "x pieces");
    __shared__ u32x4 xl[XPIECES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = (blockIdx.x * BLK_WAVES + wave) * R;
    const int nb = K / 32, xp = K / 4;

    u32x4 xv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j)
        xv[j] = *reinterpret_cast<const u32x4*>(x + 4 * min(j * BLK_THREADS + tid, xp - 1));
    __builtin_amdgcn_sched_barrier(0);
    uint32_t w[NR][R][9];
#pragma unroll
    for (int rd = 0; rd < NR; ++rd) {
        const int b = min(64 * rd + lane, nb - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t* blk = wb + ((size_t)min(n0 + r, N - 1) * nb + b) * 9;
#pragma unroll
            for (int j = 0; j < 9; ++j) w[rd][r][j] = blk[j];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < XPT; ++j) xl[x_slot(j * BLK_THREADS + tid)] = xv[j];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float acc[R] = {};
#pragma unroll
    for (int rd = 0; rd < NR; ++rd) q8_0_round<R>(xl + rd * (BLK_ROUND / 4), 64 * rd + lane < nb, w[rd], lane, acc);
    blk_store(acc, lane, n0, N, out);
}

// ---------------------------------------------------------------- Q4_K
// In round rd, eight lanes share super-block 8*rd + l/8: lane part j (0..7)
// reads quant bytes [16j, 16j+16), i.e. g = j/2 and i in [16(j%2), 16(j%2)+16):
// low nibbles are elements 64g+i of sub-block 2g, high nibbles elements
// 64g+32+i of sub-block 2g+1.  Per sub-block part the sum of q*x and the sum
// of x are formed once; the weight d*sc*q - dmin*m is applied as
// d*sc*sum(q x) - dmin*m*sum(x).
// The 6-bit scale and min of sub-block j from the scale words s0, s1, s2
// (bytes 0-3, 4-7, 8-11).  Both are a 4-bit field plus a 2-bit field above it:
// j < 4: sc = s0 bits [8j, 8j+4) | s0 bits [8j+4, 8j+6) << 4,
//        mn = s1 bits [8j, 8j+4) | s1 bits [8j+4, 8j+6) << 4;
// j >= 4 (jj = j - 4): sc = s2 bits [8jj, 8jj+4) | s0 bits [8jj+6, 8jj+8) << 4,
//        mn = s2 bits [8jj+4, 8jj+8) | s1 bits [8jj+6, 8jj+8) << 4.
// The word and bit positions depend only on j, so a lane forms them once.
struct Q4kFields {
    bool hi;               // j >= 4: the low 4 bits come from s2
    uint32_t sc_lo, mn_lo;  // positions of the 4-bit fields
    uint32_t sc_up, mn_up;  // positions of the 2-bit fields (in s0 and s1)
};

__device__ __forceinline__ Q4kFields q4k_fields(int j) {
    const uint32_t jj = (uint32_t)(j & 3);
    if (j < 4) return {false, 8 * jj, 8 * jj, 8 * jj + 4, 8 * jj + 4};
    return {true, 8 * jj, 8 * jj + 4, 8 * jj + 6, 8 * jj + 6};
}

__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, const Q4kFields& f,
                                              uint32_t& sc, uint32_t& mn) {
    const uint32_t a = f.hi ? s2 : s0, c = f.hi ? s2 : s1;
    sc = __builtin_amdgcn_ubfe(a, f.sc_lo, 4) | (__builtin_amdgcn_ubfe(s0, f.sc_up, 2) << 4);
    mn = __builtin_amdgcn_ubfe(c, f.mn_lo, 4) | (__builtin_amdgcn_ubfe(s1, f.mn_up, 2) << 4);
}

// One round of a wave's Q4_K rows: the lanes' super-block parts against the
// round's x (buf: its 512 pieces, swizzled by x_slot); act is false for a lane
// whose super-block lies past the row.
__device__ __forceinline__ void q4k_round(const u32x4* buf, bool act, const u32x4 (&hdr)[Q4K_ROWS],
                                          const u32x4 (&qw)[Q4K_ROWS], int slot, int g, int t0,
                                          const Q4kFields& f_lo, const Q4kFields& f_hi, float (&acc)[Q4K_ROWS]) {
    float xlo[16], xhi[16];
    const int u0 = (256 * slot + 64 * g + t0) / 4;   // first piece of the low half
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x_piece(buf, u0 + i, xlo + 4 * i);
        x_piece(buf, u0 + 8 + i, xhi + 4 * i);
    }
    float xsl = 0.f, xsh = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { xsl += xlo[i]; xsh += xhi[i]; }
#pragma unroll
    for (int r = 0; r < Q4K_ROWS; ++r) {
        const float d = f16_bits_to_f32(hdr[r].x & 0xffffu);
        const float dmin = f16_bits_to_f32(hdr[r].x >> 16);
        uint32_t sc_lo, mn_lo, sc_hi, mn_hi;
        q4k_scale_min(hdr[r].y, hdr[r].z, hdr[r].w, f_lo, sc_lo, mn_lo);
        q4k_scale_min(hdr[r].y, hdr[r].z, hdr[r].w, f_hi, sc_hi, mn_hi);
        float sl = 0.f, sh = 0.f;
        const uint32_t qws[4] = {qw[r].x, qw[r].y, qw[r].z, qw[r].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t lo = qws[k] & 0x0f0f0f0fu, hi = (qws[k] >> 4) & 0x0f0f0f0fu;
            // keep the masked words whole so each code converts with one
            // byte-select v_cvt_f32_ubyte<i> instead of a field extract plus a convert
            asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sl = fmaf((float)((lo >> (8 * i)) & 0xffu), xlo[4 * k + i], sl);
                sh = fmaf((float)((hi >> (8 * i)) & 0xffu), xhi[4 * k + i], sh);
            }
        }
        const float qpart = fmaf((float)sc_lo, sl, (float)sc_hi * sh);
        const float mpart = fmaf((float)mn_lo, xsl, (float)mn_hi * xsh);
        const float add = fmaf(d, qpart, -dmin * mpart);
        acc[r] += act ? add : 0.f;
    }
}

__global__ __launch_bounds__(BLK_THREADS) void q4_k_kernel(const uint32_t* __restrict__ wb,
                                                           const float* __restrict__ x,
                                                           float* __restrict__ out, int N, int K) {
    __shared__ u32x4 xl[2][BLK_ROUND / 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = lane >> 3, part = lane & 7;
    const int g = part >> 1, t0 = (part & 1) * 16;
    const int n0 = (blockIdx.x * BLK_WAVES + wave) * Q4K_ROWS;
    const int nb = K / 256;
    const Q4kFields f_lo = q4k_fields(2 * g), f_hi = q4k_fields(2 * g + 1);
    float acc[Q4K_ROWS] = {};

    struct WS { u32x4 hdr[Q4K_ROWS], qw[Q4K_ROWS]; };
    if (nb > 0) {
        auto load = [&](int rd, WS& st) {
            const int b = min(8 * rd + slot, nb - 1);
#pragma unroll
            for (int r = 0; r < Q4K_ROWS; ++r) {
                const uint32_t* blk = wb + ((size_t)min(n0 + r, N - 1) * nb + b) * 36;
                st.hdr[r] = *reinterpret_cast<const u32x4*>(blk);
                st.qw[r] = *reinterpret_cast<const u32x4*>(blk + 4 + 4 * part);
            }
        };
        blk_rounds<WS>(x, K, (nb + 7) / 8, tid, xl, load, [&](const u32x4* buf, int rd, const WS& st) {
            q4k_round(buf, 8 * rd + slot < nb, st.hdr, st.qw, slot, g, t0, f_lo, f_hi, acc);
        });
    }
    blk_store(acc, lane, n0, N, out);
}

// Short rows (at most NR rounds of 8 super-blocks): the whole row of x is staged
// in LDS once, and every wave issues the header and quant loads of all its
// rounds before consuming the first, as straight-line code (NR is a template
// parameter), so no round waits on another's loads.
constexpr int Q4K_DEEP_MAX_ROUNDS = 4;

template <int NR>
__global__ __launch_bounds__(BLK_THREADS) void q4_k_deep_kernel(const uint32_t* __restrict__ wb,
                                                                const float* __restrict__ x,
                                                                float* __restrict__ out, int N, int K) {
    constexpr int XPIECES = NR * BLK_ROUND / 4;           // 16-byte x pieces of the longest row
    constexpr int XPT = XPIECES / BLK_THREADS;
    static_assert(XPT * BLK_THREADS == XPIECES && XPT + 2 * NR * Q4K_ROWS < 64, "x pieces; memory counter range");
    __shared__ u32x4 xl[XPIECES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = lane >> 3, part = lane & 7;
    const int g = part >> 1, t0 = (part & 1) * 16;
    const int n0 = (blockIdx.x * BLK_WAVES + wave) * Q4K_ROWS;
    const int nb = K / 256, xp = K / 4;
    const Q4kFields f_lo = q4k_fields(2 * g), f_hi = q4k_fields(2 * g + 1);

    // 1. x pieces into registers (pieces past the row repeat its last one)
    u32x4 xv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j)
        xv[j] = *reinterpret_cast<const u32x4*>(x + 4 * min(j * BLK_THREADS + tid, xp - 1));
    // keep the x loads ahead of the weight loads (loads complete in order, so the
    // wait before the LDS store then leaves every weight load in flight)
    __builtin_amdgcn_sched_barrier(0);
    // 2. every round's headers and quants (blocks past the row repeat its last one)
    u32x4 hdr[NR][Q4K_ROWS], qw[NR][Q4K_ROWS];
#pragma unroll
    for (int rd = 0; rd < NR; ++rd) {
        const int b = min(8 * rd + slot, nb - 1);
#pragma unroll
        for (int r = 0; r < Q4K_ROWS; ++r) {
            const uint32_t* blk = wb + ((size_t)min(n0 + r, N - 1) * nb + b) * 36;
            hdr[rd][r] = *reinterpret_cast<const u32x4*>(blk);
            qw[rd][r] = *reinterpret_cast<const u32x4*>(blk + 4 + 4 * part);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. x to LDS (the compiler waits for the x loads only), one barrier
#pragma unroll
    for (int j = 0; j < XPT; ++j) xl[x_slot(j * BLK_THREADS + tid)] = xv[j];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // 4. the rounds in order (round rd's x starts at piece 512 rd; the swizzle
    //    repeats every 256 pieces, so x_slot addresses it relative to that start)
    float acc[Q4K_ROWS] = {};
#pragma unroll
    for (int rd = 0; rd < NR; ++rd)
        q4k_round(xl + rd * (BLK_ROUND / 4), 8 * rd + slot < nb, hdr[rd], qw[rd], slot, g, t0, f_lo, f_hi, acc);
    blk_store(acc, lane, n0, N, out);
}

hipError_t launch_q8_0(const uint32_t* w, const float* x, float* out, int N, int K, hipStream_t st) {
    const int rounds = (K / 32 + 63) / 64;
    if (K >= 32 && rounds <= Q8_DEEP_MAX_ROUNDS) {
        const dim3 grid((N + BLK_WAVES * Q8_DEEP_ROWS - 1) / (BLK_WAVES * Q8_DEEP_ROWS));
        switch (rounds) {
            case 1: hipLaunchKernelGGL(q8_0_deep_kernel<1>, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K); break;
            case 2: hipLaunchKernelGGL(q8_0_deep_kernel<2>, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K); break;
            default: hipLaunchKernelGGL(q8_0_deep_kernel<3>, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K); break;
        }
        return hipGetLastError();
    }
    const dim3 grid((N + BLK_WAVES * Q8_ROWS - 1) / (BLK_WAVES * Q8_ROWS));
    hipLaunchKernelGGL(q8_0_kernel, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K);
    return hipGetLastError();
}

hipError_t launch_q4_k(const uint32_t* w, const float* x, float* out, int N, int K, hipStream_t st) {
    const dim3 grid((N + BLK_WAVES * Q4K_ROWS - 1) / (BLK_WAVES * Q4K_ROWS));
    // Measured against the looped kernel (N = 4096..27648, K = 2048..8192): the
    // deep form is 1-13% faster, except at three rounds (176 registers, 2 waves
    // per SIMD) on grids beyond three work-groups per CU (27648 x 5120: 5% slower).
    const int rounds = (K / 256 + 7) / 8;
    const bool deep = K >= 256 && rounds <= Q4K_DEEP_MAX_ROUNDS && (rounds != 3 || (long long)grid.x <= 3LL * device_cu_count());
    if (deep) {
        switch (rounds) {
            case 1: hipLaunchKernelGGL(q4_k_deep_kernel<1>, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K); break;
            case 2: hipLaunchKernelGGL(q4_k_deep_kernel<2>, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K); break;
            case 3: hipLaunchKernelGGL(q4_k_deep_kernel<3>, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K); break;
            default: hipLaunchKernelGGL(q4_k_deep_kernel<4>, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K); break;
        }
    } else {
        hipLaunchKernelGGL(q4_k_kernel, grid, dim3(BLK_THREADS), 0, st, w, x, out, N, K);
    }
    return hipGetLastError();
}

}  // namespace qmx
