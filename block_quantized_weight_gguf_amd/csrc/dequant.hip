// Whole-matrix decode to fp32 ("EdgeRunner Core Architecture", section 3.4 Weight
// Dequantization Strategy, Tier 2: GPU decode kernels writing a float buffer).
//
// One thread per 32-weight block: the block's bytes are read with 2-byte loads
// (blocks are only 2-byte aligned), decoded in registers, and written as eight
// 16-byte stores.  Each decoded value is the float64 definition rounded once to
// fp32 (exact for the unbiased formats: an 11-bit scale times a code of at most 8
// bits; fma(d, u, m) for the biased ones).
#include "block_decode.hpp"
#include "qmm_internal.hpp"

namespace qmm {

// Thread per chunk of 4 weights (one 16-byte fp32 store).
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ W, float* __restrict__ out,
                                                      int64_t nchunks) {
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < nchunks;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float w[4];
        decode_chunk_f32<FMT, 4>(W + (e >> 3) * Fmt<FMT>::BB, static_cast<int>(e & 7), w);
        *reinterpret_cast<float4*>(out + e * 4) = make_float4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_dequant(int fmt, const void* W, float* out, int64_t M, int64_t K, hipStream_t s) {
    const int64_t nchunks = M * (K / 32) * 8;
    const int64_t grid = std::min<int64_t>((nchunks + 255) / 256, 1 << 20);
    const auto* w = static_cast<const uint8_t*>(W);
    switch (fmt) {
        case 8: hipLaunchKernelGGL(dequant_kernel<8>, dim3(grid), dim3(256), 0, s, w, out, nchunks); break;
        case 2: hipLaunchKernelGGL(dequant_kernel<2>, dim3(grid), dim3(256), 0, s, w, out, nchunks); break;
        case 3: hipLaunchKernelGGL(dequant_kernel<3>, dim3(grid), dim3(256), 0, s, w, out, nchunks); break;
        case 6: hipLaunchKernelGGL(dequant_kernel<6>, dim3(grid), dim3(256), 0, s, w, out, nchunks); break;
        case 7: hipLaunchKernelGGL(dequant_kernel<7>, dim3(grid), dim3(256), 0, s, w, out, nchunks); break;
        default: hipLaunchKernelGGL(dequant_kernel<1>, dim3(grid), dim3(256), 0, s, w, out, nchunks); break;
    }
    return hipGetLastError();
}

}  // namespace qmm
