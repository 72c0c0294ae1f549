// Register-staged streaming decode GEMV: the dispatcher over the block formats (the
// kernel and its launch helpers are in gemv_stream.hpp, instantiated per format in
// gemv_stream_<format>.hip).
#include <mutex>
#include <set>
#include <utility>

#include "gemv_stream.hpp"

namespace qmm {

// Raise a kernel's dynamic LDS limit once per (kernel, device): the attribute belongs
// to the current device, and launches may come from several host threads.
void allow_dynamic_lds(const void* kern, int bytes) {
    static std::mutex mu;
    static std::set<std::pair<const void*, int>> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (done.emplace(kern, dev).second) {
        if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
            (void)hipGetLastError();  // the launch below then reports the failure
    }
}

int64_t launch_gemv_stream(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                           int NT, int ep, const DecodeEpi& epi, hipStream_t s) {
    switch (fmt) {
        case 8: return gemv_stream_fmt<8>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 2: return gemv_stream_fmt<2>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 3: return gemv_stream_fmt<3>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 6: return gemv_stream_fmt<6>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 7: return gemv_stream_fmt<7>(W, Wu, x, y, M, K, NT, ep, epi, s);
        default: return 0;
    }
}

}  // namespace qmm
