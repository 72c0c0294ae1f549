// Streaming-read reference: the HBM read rate that a plain kernel reaches on this GPU,
// measured beside the decode GEMVs so that their weight streams can be compared with
// what the memory system delivers to a kernel, not only with the nominal peak.
//
// It reads a buffer with the loads of the single-token decode stream (16 bytes per
// lane, non-temporal) and does the least work that keeps every load: each workgroup
// folds its range with XOR and stores one word.  Workgroup b covers the 16-byte units
// [b * per, min((b + 1) * per, n)), per = ceil(n / QMM_STREAM_READ_BLOCKS); each lane
// keeps 8 loads in flight.
#include "qmm.h"
#include "qmm_common.hpp"

namespace qmm {

constexpr int SR_THREADS = 256;
constexpr int SR_UNROLL = 8;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const uint4* __restrict__ p, int64_t n,
                                                                 uint32_t* __restrict__ sink) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t b = per * blockIdx.x, e = min(b + per, n);
    uint32_t acc = 0;
    for (int64_t i = b + threadIdx.x; i < e; i += int64_t{SR_THREADS} * SR_UNROLL) {
        uint4 v[SR_UNROLL];
#pragma unroll
        for (int u = 0; u < SR_UNROLL; ++u) {
            const int64_t j = i + int64_t{SR_THREADS} * u;
            v[u] = j < e ? load16_nt(p + j) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ uint32_t part[SR_THREADS / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace qmm

extern "C" int qmm_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return QMM_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0) return QMM_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return QMM_ERR_ALIGN;
    hipLaunchKernelGGL(qmm::stream_read_kernel, dim3(QMM_STREAM_READ_BLOCKS), dim3(qmm::SR_THREADS), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}
