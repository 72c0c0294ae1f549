// Whole-matrix decode to fp32 ("EdgeRunner Core Architecture", section 3.4 Weight
// Dequantization Strategy, Tier 2: GPU decode kernels writing a float buffer).
//
// One thread per 32-weight block: the block's bytes are read with 2-byte loads
// (blocks are only 2-byte aligned), decoded in registers, and written as eight
// 16-byte stores.  Each decoded value is exact in fp32 (an 11-bit scale times a
// code of at most 8 bits), so the output equals the float64 definition.
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ W, float* __restrict__ out,
                                                      int64_t nblocks) {
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; b < nblocks;
         b += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float w[32];
    if constexpr (FMT == 1) {
        const uint4* p = reinterpret_cast<const uint4*>(W + b * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = p[i];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w[8 * i + 2 * j] = half_bits_to_float(d[j]);
                w[8 * i + 2 * j + 1] = half_bits_to_float(d[j] >> 16);
            }
        }
    } else {
        constexpr int BB = Fmt<FMT>::BB;
        const uint16_t* p = reinterpret_cast<const uint16_t*>(W + b * BB);
        const float d = half_bits_to_float(p[0]);
        if constexpr (FMT == 8) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t h = p[1 + i];
                w[2 * i] = d * sbyte_to_float(h, 0);
                w[2 * i + 1] = d * sbyte_to_float(h, 1);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t h = p[1 + i];
                w[2 * i] = d * static_cast<float>(static_cast<int>(h & 15u) - 8);
                w[2 * i + 1] = d * static_cast<float>(static_cast<int>((h >> 8) & 15u) - 8);
                w[2 * i + 16] = d * static_cast<float>(static_cast<int>((h >> 4) & 15u) - 8);
                w[2 * i + 17] = d * static_cast<float>(static_cast<int>((h >> 12) & 15u) - 8);
            }
        }
    }
    float4* o = reinterpret_cast<float4*>(out + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    }
}

hipError_t launch_dequant(int fmt, const void* W, float* out, int64_t M, int64_t K, hipStream_t s) {
    const int64_t nblocks = M * (K / 32);
    const int64_t grid = std::min<int64_t>((nblocks + 255) / 256, 1 << 20);
    const auto* w = static_cast<const uint8_t*>(W);
    switch (fmt) {
        case 8: hipLaunchKernelGGL(dequant_kernel<8>, dim3(grid), dim3(256), 0, s, w, out, nblocks); break;
        case 2: hipLaunchKernelGGL(dequant_kernel<2>, dim3(grid), dim3(256), 0, s, w, out, nblocks); break;
        default: hipLaunchKernelGGL(dequant_kernel<1>, dim3(grid), dim3(256), 0, s, w, out, nblocks); break;
    }
    return hipGetLastError();
}

}  // namespace qmm
