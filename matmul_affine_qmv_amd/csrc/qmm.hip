// qmm.hip -- tile-size choice for the staged qmm_t kernel, its launcher, and
// the split-K accumulate kernel.
#include "qmm_impl.h"

namespace qmx {

// 16-row x fragments per tile: the smallest of 1, 2, 3, 4, 6, 8 that covers
// M in one tile, else tiles of at most 8 fragments spread evenly over M.
int qmm_mt_for(int M) {
    static const int choices[] = {1, 2, 3, 4, 6, 8};
    const int tiles = qmm_mtiles_for(M);
    const int rows = (M + tiles - 1) / tiles;
    const int frags = (rows + 15) / 16;
    for (int c : choices)
        if (c >= frags) return c;
    return 8;
}

int qmm_mtiles_for(int M) { return M <= 128 ? 1 : (M + 127) / 128; }

hipError_t launch_qmm_t(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                        float* ws, int M, int N, int K, int bits, int gs, int dt, int splits,
                        hipStream_t st) {
    switch (bits) {
        case 2: return qmm_launch_b2(w, s, b, x, out, ws, M, N, K, gs, dt, splits, st);
        case 4: return qmm_launch_b4(w, s, b, x, out, ws, M, N, K, gs, dt, splits, st);
        default: return qmm_launch_b8(w, s, b, x, out, ws, M, N, K, gs, dt, splits, st);
    }
}

// out[i] = round(sum_{p=0}^{S-1} ws[p*MN + i]), summed in ascending p in float32
// and rounded once (page "mlx PR 4682": separate accumulate kernel, one rounding).
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void splitk_accum_kernel(const float* __restrict__ ws, void* __restrict__ out,
                                                           int S, size_t MN) {
    const size_t i0 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i0 >= MN) return;
    if (VEC && i0 + 4 <= MN) {
        f32x4 acc = *reinterpret_cast<const f32x4*>(ws + i0);
        for (int p = 1; p < S; ++p) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(ws + (size_t)p * MN + i0);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        store_elem<DT>(out, i0 + 0, acc.x);
        store_elem<DT>(out, i0 + 1, acc.y);
        store_elem<DT>(out, i0 + 2, acc.z);
        store_elem<DT>(out, i0 + 3, acc.w);
    } else {
        const size_t iend = i0 + 4 < MN ? i0 + 4 : MN;
        for (size_t i = i0; i < iend; ++i) {
            float acc = ws[i];
            for (int p = 1; p < S; ++p) acc += ws[(size_t)p * MN + i];
            store_elem<DT>(out, i, acc);
        }
    }
}

hipError_t launch_splitk_accum(const float* ws, void* out, int splits, size_t MN, int dt, hipStream_t st) {
    const size_t threads = (MN + 3) / 4;
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    const bool vec = (MN % 4) == 0;
    if (dt == DT_F16) {
        if (vec) hipLaunchKernelGGL((splitk_accum_kernel<DT_F16, true>), grid, block, 0, st, ws, out, splits, MN);
        else hipLaunchKernelGGL((splitk_accum_kernel<DT_F16, false>), grid, block, 0, st, ws, out, splits, MN);
    } else {
        if (vec) hipLaunchKernelGGL((splitk_accum_kernel<DT_BF16, true>), grid, block, 0, st, ws, out, splits, MN);
        else hipLaunchKernelGGL((splitk_accum_kernel<DT_BF16, false>), grid, block, 0, st, ws, out, splits, MN);
    }
    return hipGetLastError();
}

}  // namespace qmx
