// Element-wise weight kernels beside the products:
//   * row gather (embedding lookup): out[i] = W[ids[i]] decoded to fp32.
//     ("llama.cpp Metal ...", section 3.2 "Input embd": token ids -> get_rows on the
//     token-embedding matrix; P8: GET_ROWS dispatches per-format get_rows kernels.
//     "EdgeRunner Core Architecture", section 3.4 Tier 3: embedding lookups decode
//     straight into the destination.)
//   * fp16 expansion: out = fp16(W) rounded to nearest even, the input of the
//     expand-then-GEMM prefill variant ("alpaca.swift", Design: quantised weights are
//     expanded one matrix at a time into a scratch buffer for the tensor-op GEMMs;
//     "EdgeRunner Core Architecture", section 3.4 Tier 2: GPU decode to float16).
// A thread per chunk of 4 (fp32) or 8 (fp16) weights.  The fp16 expansion rounds
// each exact weight once (which is the value the fused GEMM feeds its MFMAs): the
// unbiased formats decode exactly in fp32 first, the biased ones use an fp16 fma.
#include "block_decode.hpp"
#include "qmm_internal.hpp"

namespace qmm {

// Workgroups tile one output row along x (a thread per chunk of 4 weights, one
// 16-byte store) and stride over the rows along y.  ids are device data: an id
// outside [0, M) turns its output row into NaN instead of reading outside W.
template <int FMT>
__global__ __launch_bounds__(256) void get_rows_kernel(const uint8_t* __restrict__ W, const int32_t* __restrict__ ids,
                                                       float* __restrict__ out, int64_t M, int64_t nb, int64_t n) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // chunk within a row
    if (e >= nb * 8) return;
    const int64_t rb = nb * Fmt<FMT>::BB;
    for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
        const int64_t id = ids[i];
        float w[4];
        if (id >= 0 && id < M) {
            decode_chunk_f32<FMT, 4>(W + id * rb + (e >> 3) * Fmt<FMT>::BB, static_cast<int>(e & 7), w);
        } else {
            w[0] = w[1] = w[2] = w[3] = __builtin_nanf("");
        }
        *reinterpret_cast<float4*>(out + i * nb * 32 + e * 4) = make_float4(w[0], w[1], w[2], w[3]);
    }
}

// Thread per chunk of 8 weights (one 16-byte fp16 store).
template <int FMT>
__global__ __launch_bounds__(256) void expand_f16_kernel(const uint8_t* __restrict__ W, _Float16* __restrict__ out,
                                                         int64_t nchunks) {
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < nchunks;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        uint4* dst = reinterpret_cast<uint4*>(out + e * 8);
        if constexpr (FMT == 1) {  // already half precision: a copy, bit for bit
            *dst = *reinterpret_cast<const uint4*>(W + e * 16);
        } else if constexpr (Nib<FMT>::BIAS) {
            _Float16 w[8];
            decode_chunk_f16_biased<FMT, 8>(W + (e >> 2) * Fmt<FMT>::BB, static_cast<int>(e & 3), w);
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                h[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, w[2 * j])) |
                       (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, w[2 * j + 1])) << 16);
            *dst = make_uint4(h[0], h[1], h[2], h[3]);
        } else {
            float w[8];
            decode_chunk_f32<FMT, 8>(W + (e >> 2) * Fmt<FMT>::BB, static_cast<int>(e & 3), w);
            // Keep the exact fp32 product and the fp16 conversion apart: fused into an
            // fma(d, q, +0) with an fp16 result, a -0 weight would come out as +0.
#pragma unroll
            for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(w[j]));
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const _Float16 lo = static_cast<_Float16>(w[2 * j]);
                const _Float16 hi = static_cast<_Float16>(w[2 * j + 1]);
                h[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                       (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
            }
            *dst = make_uint4(h[0], h[1], h[2], h[3]);
        }
    }
}

hipError_t launch_get_rows(int fmt, const void* W, const int32_t* ids, float* out, int64_t M, int64_t K, int64_t n,
                           hipStream_t s) {
    const int64_t nb = K / 32;
    const dim3 grid(static_cast<unsigned>((nb * 8 + 255) / 256), static_cast<unsigned>(std::min<int64_t>(n, 65535)));
    const auto* w = static_cast<const uint8_t*>(W);
    switch (fmt) {
        case 8: hipLaunchKernelGGL(get_rows_kernel<8>, grid, dim3(256), 0, s, w, ids, out, M, nb, n); break;
        case 2: hipLaunchKernelGGL(get_rows_kernel<2>, grid, dim3(256), 0, s, w, ids, out, M, nb, n); break;
        case 3: hipLaunchKernelGGL(get_rows_kernel<3>, grid, dim3(256), 0, s, w, ids, out, M, nb, n); break;
        case 6: hipLaunchKernelGGL(get_rows_kernel<6>, grid, dim3(256), 0, s, w, ids, out, M, nb, n); break;
        case 7: hipLaunchKernelGGL(get_rows_kernel<7>, grid, dim3(256), 0, s, w, ids, out, M, nb, n); break;
        default: hipLaunchKernelGGL(get_rows_kernel<1>, grid, dim3(256), 0, s, w, ids, out, M, nb, n); break;
    }
    return hipGetLastError();
}

hipError_t launch_expand_f16(int fmt, const void* W, void* out, int64_t M, int64_t K, hipStream_t s) {
    const int64_t nchunks = M * (K / 32) * 4;
    const int64_t grid = std::min<int64_t>((nchunks + 255) / 256, 1 << 20);
    const auto* w = static_cast<const uint8_t*>(W);
    auto* o = static_cast<_Float16*>(out);
    switch (fmt) {
        case 8: hipLaunchKernelGGL(expand_f16_kernel<8>, dim3(grid), dim3(256), 0, s, w, o, nchunks); break;
        case 2: hipLaunchKernelGGL(expand_f16_kernel<2>, dim3(grid), dim3(256), 0, s, w, o, nchunks); break;
        case 3: hipLaunchKernelGGL(expand_f16_kernel<3>, dim3(grid), dim3(256), 0, s, w, o, nchunks); break;
        case 6: hipLaunchKernelGGL(expand_f16_kernel<6>, dim3(grid), dim3(256), 0, s, w, o, nchunks); break;
        case 7: hipLaunchKernelGGL(expand_f16_kernel<7>, dim3(grid), dim3(256), 0, s, w, o, nchunks); break;
        default: hipLaunchKernelGGL(expand_f16_kernel<1>, dim3(grid), dim3(256), 0, s, w, o, nchunks); break;
    }
    return hipGetLastError();
}

}  // namespace qmm
