// fp32 tokens -> per-token scaled fp16, the operand form of the tiled GEMM when it
// serves fp32-token products (more than 32 tokens, F16 weights, K % 256 != 0; the
// weight-streaming MFMA GEMV converts its tokens itself, stage by stage).
//
// The MFMA products multiply fp16 operands ("alpaca.swift", Design: half-precision
// activations on the matrix hardware).  Decode activations arrive as fp32, whose
// range fp16 cannot hold ("alpaca.swift", Limitations: activations are not
// quantised), so each token row t is scaled by the power of two 2^s_t that brings its
// largest magnitude into [2^14, 2^15) before the one rounding to fp16: nothing
// overflows, and every element keeps a relative error <= 2^-11 unless it lies more
// than about 2^28 below its token's largest.  The GEMM multiplies token t's sums by
// inv[t] = 2^-s_t, an exact power of two.
//
// One workgroup per token row: a pass over the row for its largest |x| (waves reduce
// with shuffles, then the workgroup in LDS), then a pass that converts 8 values per
// thread and step with one 16-byte store (the row is read twice; the second read
// comes from the caches).
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int ST_THREADS = 256;

__device__ __forceinline__ uint32_t half2_bits(float a, float b) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(a))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(b))) << 16);
}

__global__ __launch_bounds__(ST_THREADS) void scale_tokens_kernel(const float* __restrict__ x,
                                                                   _Float16* __restrict__ x16,
                                                                   float* __restrict__ inv, int64_t K) {
    const int64_t t = blockIdx.x;
    const float4* row = reinterpret_cast<const float4*>(x + t * K);
    uint4* out = reinterpret_cast<uint4*>(x16 + t * K);
    const int64_t n8 = K / 8;
    float m = 0.0f;
    for (int64_t c = threadIdx.x; c < n8; c += ST_THREADS) {
        const float4 a = row[2 * c], b = row[2 * c + 1];
        m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                           fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w)))));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float wmax[ST_THREADS / 64];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu) - 127;  // floor(log2 m); -127 for 0
    const int se = min(126, 14 - e);                                            // >= -114 (m <= inf)
    const float sc = __uint_as_float(static_cast<uint32_t>(se + 127) << 23);
    if (threadIdx.x == 0) inv[t] = __uint_as_float(static_cast<uint32_t>(127 - se) << 23);
    for (int64_t c = threadIdx.x; c < n8; c += ST_THREADS) {
        const float4 a = row[2 * c], b = row[2 * c + 1];
        out[c] = make_uint4(half2_bits(a.x * sc, a.y * sc), half2_bits(a.z * sc, a.w * sc),
                            half2_bits(b.x * sc, b.y * sc), half2_bits(b.z * sc, b.w * sc));
    }
}

hipError_t launch_scale_tokens(const float* x, void* x16, float* inv, int64_t N, int64_t K, hipStream_t s) {
    hipLaunchKernelGGL(scale_tokens_kernel, dim3(static_cast<unsigned>(N)), dim3(ST_THREADS), 0, s, x,
                       static_cast<_Float16*>(x16), inv, K);
    return hipGetLastError();
}

}  // namespace qmm
