// noalloc.hip -- qmx_qmm_t_splitk_noalloc: split-K without a caller
// workspace, for callers that cannot allocate.  The float32 partials live in a
// file-scope device array; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name in host
// code is a host-side stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "qmx.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QMX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;

// The device address of `scratch` on the current device, looked up once per
// device with that device current; nullptr if it cannot be had.
void* scratch_here() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" int qmx_qmm_t_splitk_noalloc(const uint32_t* w_packed, const void* scales, const void* biases,
                                        const void* x, void* out, int M, int N, int K, int bits, int group_size,
                                        int dtype, int splits, void* stream) {
    if (M >= 0 && N >= 0 && splits >= 2 && qmx_splitk_workspace_bytes(M, N, splits) > QMX_NOALLOC_SCRATCH_BYTES)
        return QMX_ERR_SCRATCH;
    // argument errors and empty problems need no device address
    const int rc = qmx_qmm_t_splitk(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype, splits,
                                    nullptr, 0, stream);
    if (rc != QMX_ERR_WORKSPACE) return rc;
    void* ws = scratch_here();
    if (!ws) return QMX_ERR_DEVICE;
    return qmx_qmm_t_splitk(w_packed, scales, biases, x, out, M, N, K, bits, group_size, dtype, splits, ws,
                            QMX_NOALLOC_SCRATCH_BYTES, stream);
}
