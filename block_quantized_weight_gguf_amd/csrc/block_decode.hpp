// Decode of one chunk of C consecutive weights (C = 4 or 8) of a 32-weight block to
// fp32, for the element-wise kernels (dequant, row gather, fp16 expansion).  A lane
// per chunk keeps every output store a whole 16-byte piece with consecutive lanes
// on consecutive addresses.  ("EdgeRunner Core Architecture", sections 1.3, 3.1 and
// 3.2: Q8_0 = fp16 d + 32 int8 codes, w = d * q; Q4_0 = fp16 d + 16 bytes, byte j
// holding weight j in its low nibble and weight j + 16 in its high nibble,
// w = d * (n - 8); Q4_1, Q5_0, Q5_1 as laid out in qmm_common.hpp.)  Quantised blocks
// are only 2-byte aligned, so their bytes are read with 2-byte loads; F16 chunks are
// 8- or 16-byte aligned.  The unbiased formats decode exactly in fp32 (an 11-bit
// scale times a code of at most 8 bits); the biased ones as fma(d, u, m), the exact
// d * u + m rounded once.
#pragma once

#include "qmm_common.hpp"

namespace qmm {

// Weights [C*c, C*c + C) of block blk.
template <int FMT, int C>
__device__ __forceinline__ void decode_chunk_f32(const uint8_t* blk, int c, float (&w)[C]) {
    static_assert(C == 4 || C == 8, "chunk of 4 or 8 weights");
    if constexpr (FMT == 1) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(blk + 2 * C * c);
        uint32_t v[C / 2];
        if constexpr (C == 8) {
            const uint4 t = *reinterpret_cast<const uint4*>(p);
            v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
        } else {
            const uint2 t = *reinterpret_cast<const uint2*>(p);
            v[0] = t.x; v[1] = t.y;
        }
#pragma unroll
        for (int j = 0; j < C / 2; ++j) {
            w[2 * j] = half_bits_to_float(v[j]);
            w[2 * j + 1] = half_bits_to_float(v[j] >> 16);
        }
    } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(blk);
        const float d = half_bits_to_float(p[0]);
        if constexpr (FMT == 8) {
            const uint16_t* q = p + 1 + (C / 2) * c;
#pragma unroll
            for (int j = 0; j < C / 2; ++j) {
                const uint32_t h = q[j];
                w[2 * j] = d * sbyte_to_float(h, 0);
                w[2 * j + 1] = d * sbyte_to_float(h, 1);
            }
        } else {
            using T = Nib<FMT>;
            const int first = C * c;                 // first weight of the chunk
            const uint16_t* q = p + T::QS / 2 + (first & 15) / 2;
            const int sh = first >= 16 ? 4 : 0;      // high nibbles hold weights 16..31
            uint32_t hb = 0;                         // fifth bits of the chunk, from bit 0
            if constexpr (T::FIVE) hb = (p[T::QH / 2] | (static_cast<uint32_t>(p[T::QH / 2 + 1]) << 16)) >> first;
            const float m = T::BIAS ? half_bits_to_float(p[1]) : 0.0f;
#pragma unroll
            for (int j = 0; j < C / 2; ++j) {
                const uint32_t h = static_cast<uint32_t>(q[j]) >> sh;
                const int u0 = static_cast<int>((h & 15u) | (((hb >> (2 * j)) & 1u) << 4));
                const int u1 = static_cast<int>(((h >> 8) & 15u) | (((hb >> (2 * j + 1)) & 1u) << 4));
                if constexpr (T::BIAS) {
                    w[2 * j] = fmaf(d, static_cast<float>(u0), m);
                    w[2 * j + 1] = fmaf(d, static_cast<float>(u1), m);
                } else {
                    w[2 * j] = d * static_cast<float>(u0 - T::OFF);
                    w[2 * j + 1] = d * static_cast<float>(u1 - T::OFF);
                }
            }
        }
    }
}

// The biased formats (Q4_1, Q5_1) to fp16: fp16 fma(d, u, m) rounds the exact
// d * u + m once (u <= 31 is exact in fp16), which a round to fp32 and then to fp16
// would not always do.
template <int FMT, int C>
__device__ __forceinline__ void decode_chunk_f16_biased(const uint8_t* blk, int c, _Float16 (&w)[C]) {
    using T = Nib<FMT>;
    static_assert(T::BIAS, "biased formats only");
    const uint16_t* p = reinterpret_cast<const uint16_t*>(blk);
    const _Float16 d = __builtin_bit_cast(_Float16, p[0]);
    const _Float16 m = __builtin_bit_cast(_Float16, p[1]);
    const int first = C * c;
    const uint16_t* q = p + T::QS / 2 + (first & 15) / 2;
    const int sh = first >= 16 ? 4 : 0;
    uint32_t hb = 0;
    if constexpr (T::FIVE) hb = (p[T::QH / 2] | (static_cast<uint32_t>(p[T::QH / 2 + 1]) << 16)) >> first;
#pragma unroll
    for (int j = 0; j < C / 2; ++j) {
        const uint32_t h = static_cast<uint32_t>(q[j]) >> sh;
        const uint32_t u0 = (h & 15u) | (((hb >> (2 * j)) & 1u) << 4);
        const uint32_t u1 = ((h >> 8) & 15u) | (((hb >> (2 * j + 1)) & 1u) << 4);
        w[2 * j] = __builtin_fmaf16(d, static_cast<_Float16>(static_cast<int>(u0)), m);
        w[2 * j + 1] = __builtin_fmaf16(d, static_cast<_Float16>(static_cast<int>(u1)), m);
    }
}

}  // namespace qmm
