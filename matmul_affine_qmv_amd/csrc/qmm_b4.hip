// qmm_b4.hip -- 4-bit instances of the staged qmm_t kernel (kept apart so the
// code widths compile in parallel).
#include "qmm_impl.h"

namespace qmx {

hipError_t qmm_launch_b4(const uint32_t* w, const void* s, const void* b, const void* x, void* out,
                         float* ws, int batch, QmxStrides sd, int M, int N, int K, int gs, int dt, int splits,
                         hipStream_t st) {
    return qmm_launch_bits<4>(w, s, b, x, out, ws, batch, sd, M, N, K, gs, dt, splits, st);
}

}  // namespace qmx
