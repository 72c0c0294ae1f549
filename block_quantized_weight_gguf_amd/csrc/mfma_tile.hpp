// Shared pieces of the MFMA kernels (prefill GEMM and small-batch GEMV) for gfx950:
// fp16-domain decode of GGUF blocks into MFMA operands (the buffer->LDS DMA and
// wait helpers are in dma.hpp).
//
// Decode ("EdgeRunner Core Architecture", sections 3.1 and 3.2: w = d * q for Q8_0,
// d * (n - 8) for Q4_0, byte j of a Q4_0 block holding weights j and j + 16): a code
// byte c becomes the half 1024 + c via v_perm with 0x64 bytes, v_pk_add_f16 removes
// the offset exactly and v_pk_mul_f16 by the fp16 scale gives fp16(d * q) with a
// single rounding.  Q5_0 does the same with its 5-bit code u and offset 16; Q4_1 and
// Q5_1 remove 1024 and finish with v_pk_fma_f16(u, d, m): fp16(d * u + m), again a
// single rounding of the exact weight.
#pragma once

#include "dma.hpp"
#include "qmm_common.hpp"

namespace qmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t h2_bits(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2_t bits_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// Two bytes (selected by `sel`) of `c` as halves 1024 + byte, i.e. bits 0x64bb.
__device__ __forceinline__ half2_t bytes_to_h2(uint32_t c, uint32_t sel) {
    return bits_h2(__builtin_amdgcn_perm(0x64646464u, c, sel));
}
constexpr uint32_t kSelLo = 0x05010400u;  // bytes 0, 1
constexpr uint32_t kSelHi = 0x05030402u;  // bytes 2, 3

// 4 Q8_0 codes (one dword) -> 4 fp16 weights fp16(d * q) in 2 dwords.
__device__ __forceinline__ void q8_4(uint32_t codes, half2_t d2, uint32_t& o0, uint32_t& o1) {
    const uint32_t c = codes ^ 0x80808080u;  // q + 128 as unsigned bytes
    const half2_t off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
    o0 = h2_bits((bytes_to_h2(c, kSelLo) + off) * d2);
    o1 = h2_bits((bytes_to_h2(c, kSelHi) + off) * d2);
}

// 4 Q4_0 nibbles (one per byte, already masked) -> 4 fp16 weights fp16(d * (n - 8)).
__device__ __forceinline__ void q4_4(uint32_t nib, half2_t d2, uint32_t& o0, uint32_t& o1) {
    const half2_t off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
    o0 = h2_bits((bytes_to_h2(nib, kSelLo) + off) * d2);
    o1 = h2_bits((bytes_to_h2(nib, kSelHi) + off) * d2);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return h2_bits(half2_t{static_cast<_Float16>(a), static_cast<_Float16>(b)});
}

// Weight stage geometry: K steps per stage, 16-byte chunks per row window, and
// the bytes of the per-row segment one stage covers.
template <int FMT>
struct WStage;
template <>
struct WStage<8> {  // Q8_0: 4 blocks = 136 bytes, in 9 chunks
    static constexpr int KPS = 2, WCH = 9;
};
template <>
struct WStage<2> {  // Q4_0: 4 blocks = 72 bytes, in 5 chunks
    static constexpr int KPS = 2, WCH = 5;
};
template <>
struct WStage<3> {  // Q4_1: 4 blocks = 80 bytes, in 5 chunks (always at offset 0)
    static constexpr int KPS = 2, WCH = 5;
};
template <>
struct WStage<6> {  // Q5_0: 4 blocks = 88 bytes at offset 0 or 8, in 6 chunks
    static constexpr int KPS = 2, WCH = 6;
};
template <>
struct WStage<7> {  // Q5_1: 4 blocks = 96 bytes, in 6 chunks (always at offset 0)
    static constexpr int KPS = 2, WCH = 6;
};
template <>
struct WStage<1> {  // F16: 64 halfs = 128 bytes
    static constexpr int KPS = 1, WCH = 8;
};

// Byte offset of a block-format weight stage inside its 16-byte aligned window: the
// four-block segment of stage st starts st * 4 * BB bytes into the (16-byte aligned)
// row, i.e. 0 or 8 bytes into its window, 8 only for odd stages of formats whose
// segment is not a multiple of 16 bytes (Q8_0, Q4_0, Q5_0).
template <int FMT>
constexpr int stage_shift(int parity) {
    return (FMT == 1 || (4 * Fmt<FMT>::BB) % 16 == 0) ? 0 : 8 * parity;
}

// A fragment of v_mfma_f32_16x16x32_f16 decoded from a raw block-format row window in
// LDS: the 8 weights 8 q4 .. 8 q4 + 7 (lane l: q4 = l / 16) of the block that starts
// `o` bytes into the row (o even; blocks are 2-byte aligned).  Q4_0 fragments 0, 1
// take the low nibbles of code bytes 0..7 / 8..15, fragments 2, 3 the high nibbles.
// The LDS words frag_decode needs: the scale dword and the (unaligned) code dwords
// (Q4_1 / Q5_0 / Q5_1: d = the dword holding the scale, h = the next one, which
// holds the bias or the fifth bits).
struct RawA {
    uint32_t d, w0, w1, w2, h;
};

// Q4_1 / Q5_0 / Q5_1 fragments: lane l needs the scale, the bias (biased formats), the
// fifth bits of its 8 weights (byte q4 of qh) and 8 nibble bytes at QS + 8 (q4 & 1),
// low nibbles for q4 < 2, high ones otherwise.  Q4_1 and Q5_1 blocks (20 and 24
// bytes, stage offset 0) start on a dword; Q5_0 blocks (22 bytes) on a dword or
// halfword.
template <int FMT>
__device__ __forceinline__ RawA frag_load_nib(const QMM_L3 uint32_t* dw, int o, int q4) {
    using T = Nib<FMT>;
    constexpr bool A4 = Fmt<FMT>::BB % 4 == 0;
    RawA r;
    const int o4 = o >> 2;
    r.d = dw[o4];
    r.h = T::FIVE ? dw[o4 + 1] : 0u;
    const int p = o + T::QS + 8 * (q4 & 1);  // first code byte of the fragment
    r.w0 = dw[p >> 2];
    r.w1 = dw[(p >> 2) + 1];
    r.w2 = A4 ? 0u : dw[(p >> 2) + 2];
    return r;
}

template <int FMT>
__device__ __forceinline__ half8_t frag_decode_nib(const RawA& r, int o, int q4) {
    using T = Nib<FMT>;
    constexpr bool A4 = Fmt<FMT>::BB % 4 == 0;
    const bool lo_half = A4 || (o & 3) == 0;  // the scale in the low half of r.d
    const uint32_t d = lo_half ? (r.d & 0xFFFFu) : (r.d >> 16);
    uint32_t qh = 0;
    if constexpr (T::FIVE) qh = (A4 || !lo_half) ? r.h : align_bytes(r.h, r.d, 2);
    const int p = o + T::QS + 8 * (q4 & 1);
    uint32_t c0 = r.w0, c1 = r.w1;
    if (!A4 && (p & 3) != 0) {
        c0 = align_bytes(r.w1, r.w0, 2);
        c1 = align_bytes(r.w2, r.w1, 2);
    }
    const uint32_t s4 = 4 * (q4 >> 1);
    uint32_t n0 = (c0 >> s4) & 0x0F0F0F0Fu, n1 = (c1 >> s4) & 0x0F0F0F0Fu;
    if constexpr (T::FIVE) {
        const uint32_t hb = qh >> (8 * q4);
        n0 |= spread4(hb) << 4;
        n1 |= spread4(hb >> 4) << 4;
    }
    const half2_t d2 = bits_h2(d | (d << 16));
    uint32_t o4[4];
    if constexpr (T::BIAS) {
        const uint32_t m = r.d >> 16;  // biased blocks start on a dword: m is the high half
        const half2_t m2 = bits_h2(m | (m << 16));
        const half2_t off = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};
        o4[0] = h2_bits(__builtin_elementwise_fma(bytes_to_h2(n0, kSelLo) + off, d2, m2));
        o4[1] = h2_bits(__builtin_elementwise_fma(bytes_to_h2(n0, kSelHi) + off, d2, m2));
        o4[2] = h2_bits(__builtin_elementwise_fma(bytes_to_h2(n1, kSelLo) + off, d2, m2));
        o4[3] = h2_bits(__builtin_elementwise_fma(bytes_to_h2(n1, kSelHi) + off, d2, m2));
    } else {
        const half2_t off = {static_cast<_Float16>(-1040.0f), static_cast<_Float16>(-1040.0f)};
        o4[0] = h2_bits((bytes_to_h2(n0, kSelLo) + off) * d2);
        o4[1] = h2_bits((bytes_to_h2(n0, kSelHi) + off) * d2);
        o4[2] = h2_bits((bytes_to_h2(n1, kSelLo) + off) * d2);
        o4[3] = h2_bits((bytes_to_h2(n1, kSelHi) + off) * d2);
    }
    return __builtin_bit_cast(half8_t, u32x4_t{o4[0], o4[1], o4[2], o4[3]});
}

template <int FMT>
__device__ __forceinline__ RawA frag_load(const QMM_L3 uint8_t* row, int o, int q4) {
    static_assert(FMT != 1, "block formats only");
    const QMM_L3 uint32_t* dw = reinterpret_cast<const QMM_L3 uint32_t*>(row);
    if constexpr (FMT != 8 && FMT != 2) return frag_load_nib<FMT>(dw, o, q4);
    const int cb = (FMT == 8) ? 8 * q4 : 8 * (q4 & 1);  // code byte offset in the block
    RawA r{};
    if ((o & 3) == 0) {
        r.d = dw[o >> 2];
        const int base = (o + cb) >> 2;  // codes start 2 bytes into dword `base`
        r.w0 = dw[base];
        r.w1 = dw[base + 1];
        r.w2 = dw[base + 2];
    } else {
        r.d = dw[(o - 2) >> 2];
        const int base = (o + 2 + cb) >> 2;
        r.w0 = dw[base];
        r.w1 = dw[base + 1];
        r.w2 = 0;
    }
    return r;
}

template <int FMT>
__device__ __forceinline__ half8_t frag_decode(const RawA& r, int o, int q4) {
    if constexpr (FMT != 8 && FMT != 2) return frag_decode_nib<FMT>(r, o, q4);
    uint32_t d, c0, c1;
    if ((o & 3) == 0) {
        d = r.d & 0xFFFFu;
        c0 = align_bytes(r.w1, r.w0, 2);
        c1 = align_bytes(r.w2, r.w1, 2);
    } else {
        d = r.d >> 16;
        c0 = r.w0;
        c1 = r.w1;
    }
    const half2_t d2 = bits_h2(d | (d << 16));
    uint32_t r0, r1, r2, r3;
    if constexpr (FMT == 8) {
        q8_4(c0, d2, r0, r1);
        q8_4(c1, d2, r2, r3);
    } else {
        const uint32_t s4 = 4 * (q4 >> 1);  // fragments 2, 3 take the high nibbles
        q4_4((c0 >> s4) & 0x0F0F0F0Fu, d2, r0, r1);
        q4_4((c1 >> s4) & 0x0F0F0F0Fu, d2, r2, r3);
    }
    return __builtin_bit_cast(half8_t, u32x4_t{r0, r1, r2, r3});
}

template <int FMT>
__device__ __forceinline__ half8_t frag_raw(const QMM_L3 uint8_t* row, int o, int q4) {
    return frag_decode<FMT>(frag_load<FMT>(row, o, q4), o, q4);
}

}  // namespace qmm
