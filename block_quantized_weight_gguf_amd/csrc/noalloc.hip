// qmm_gemm without a workspace argument and without allocating: for callers that
// cannot call hipMalloc or take memory from a pool at all (code under graph capture
// that owns no buffers, tight serving loops, harnesses that forbid allocation).
//
// The split-K partials that qmm_gemm keeps in the caller's workspace live here in a
// fixed file-scope device array, `scratch`.  Each GPU the library runs on holds its own
// copy for the life of the process.  In host code the array's name is a host-side
// stand-in, not a device address, so the entry point looks up the device address of
// the current device's copy with hipGetSymbolAddress, once per device, and passes that
// pointer to the kernels.  Every call on a GPU shares that GPU's array: calls that
// overlap on one GPU (concurrent streams, threads) race on it.  Nothing in it needs to
// start at zero (each split writes all of its partials before the reduce reads them).
#include <mutex>

#include "../../include/qmm.h"
#include "qmm_internal.hpp"

// qmm_gemm's partials take nsplit x T x M x 4 bytes, and its plan splits K only while
// the output tiles number fewer than 192, into at most 256 / tiles splits of tiles of at
// most 256 x 256 outputs: at most 256 x 256 x 256 x 4 bytes = 64 MiB.
static __device__ __align__(256) uint8_t scratch[QMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch` (nullptr on failure).
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

bool is_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" int qmm_gemm_noalloc(int fmt, const void* W, const void* X, float* Y, int64_t M, int64_t K, int64_t T,
                                void* stream) {
    // Argument checks and the workspace size as qmm_gemm computes them.
    const int64_t need = qmm_workspace_size(QMM_OP_GEMM, fmt, M, K, T, QMM_VARIANT_AUTO);
    if (need < 0) return static_cast<int>(need);
    if (!W || !X || !Y) return QMM_ERR_NULL;
    if (!is_aligned(W, 16) || !is_aligned(X, 16) || !is_aligned(Y, 4)) return QMM_ERR_ALIGN;
    if (need > QMM_NOALLOC_SCRATCH_BYTES) return QMM_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_ptr();
        if (!ws) return QMM_ERR_HIP;
    }
    const hipError_t e = qmm::launch_gemm_mfma(fmt, W, nullptr, X, nullptr, Y, M, K, T, static_cast<float*>(ws),
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}
