// Per-block decode + FMA used by the GEMV kernels.
//
// One lane handles one 32-weight block of up to RU row units at once, reading the
// raw block bytes from LDS at any 2-byte aligned address (Q4_1 and Q5_1 blocks, whose
// fields all lie on 4 bytes, at 4-byte aligned ones) and the matching 32 activations
// per token from LDS (block stride XS_STRIDE floats).  The activations
// are read once and reused for all row units.
//   Q8_0: 32 codes -> one signed-byte-to-float op each (SDWA sext) -> one FMA each;
//         the block partial is scaled by d once.
//   Q4_0: xor 0x88 maps each nibble n to n ^ 8; moved into the high half of a byte
//         it reads as the signed byte 16 * (n - 8), so the same one-op convert gives
//         the exact code; the scale is d / 16 (exact).
//   Q5_0: the same with the fifth bit: (u ^ 16) << 3 reads as the signed byte
//         8 * (u - 16); the scale is d / 8.
//   Q4_1, Q5_1: the unsigned code u as an unsigned byte, each weight formed as
//         fma(d, u, m) (the exact d * u + m rounded once) before its product with x.
#pragma once

#include "block_decode.hpp"
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int XS_STRIDE = 36;  // floats per block in the LDS copy of x (32 + 4 padding)

// The fields of a Q4_1 / Q5_0 / Q5_1 block from LDS: scale, bias (biased formats),
// the fifth-bit word (5-bit formats) and the four dwords of nibbles.  Q4_1 and Q5_1
// blocks (20 and 24 bytes, every field on 4 bytes) lie on 4 bytes wherever they are
// staged, since W is 16-byte aligned and rows and blocks are multiples of 4 bytes
// long, so their dwords are read as they lie; Q5_0 blocks (22 bytes) are realigned.
template <int FMT>
__device__ __forceinline__ void read_nib_block(const uint8_t* buf, int off, float& d, float& m, uint32_t& qh,
                                               uint32_t (&cw)[4]) {
    using T = Nib<FMT>;
    if constexpr (T::BIAS) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(buf + off);
        const uint32_t dm = w[0];
        d = half_bits_to_float(static_cast<uint16_t>(dm));
        m = half_bits_to_float(static_cast<uint16_t>(dm >> 16));
        qh = T::FIVE ? w[1] : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = w[(T::FIVE ? 2 : 1) + i];
        return;
    }
    d = half_bits_to_float(lds_read_u16(buf, off));
    m = 0.0f;
    if constexpr (T::FIVE) {
        uint32_t w[5];  // qh is followed directly by the nibbles
        lds_read_dwords<5>(buf, off + T::QH, w);
        qh = w[0];
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = w[i + 1];
    } else {
        qh = 0;
        lds_read_dwords<4>(buf, off + T::QS, cw);
    }
}

// Code bytes of weights 4i..4i+3 (lo) and 16+4i..16+4i+3 (hi) of a nibble-format
// block, from nibble dword cw = dword i and the fifth-bit word qh:
//   Q5_0: signed bytes 8 (u - 16); Q4_1 / Q5_1: unsigned bytes u.
template <int FMT>
__device__ __forceinline__ void nib_code_bytes(uint32_t cw, uint32_t qh, int i, uint32_t& lo, uint32_t& hi) {
    using T = Nib<FMT>;
    lo = cw & 0x0F0F0F0Fu;
    hi = (cw >> 4) & 0x0F0F0F0Fu;
    if constexpr (T::FIVE) {
        lo |= spread4(qh >> (4 * i)) << 4;
        hi |= spread4(qh >> (16 + 4 * i)) << 4;
    }
    if constexpr (FMT == 6) {
        lo = (lo ^ 0x10101010u) << 3;
        hi = (hi ^ 0x10101010u) << 3;
    }
}

// block_fma for Q4_1, Q5_0, Q5_1 (see the header comment for the code bytes).  The
// biased formats form each weight w = fma(d, u, m), the exact d u + m rounded once,
// before its product with x: factoring the bias out (d sum u x + m sum x) would round
// two sums that can cancel far below sum |w x|.
template <int FMT, int RU, int NT>
__device__ __forceinline__ void block_fma_nib(const uint8_t* const (&buf)[RU], const int (&off)[RU],
                                              const float* const (&xb)[NT], float (&acc)[RU][NT]) {
    constexpr bool BIAS = Nib<FMT>::BIAS;
    float bacc[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) bacc[u][n] = 0.0f;
    float d[RU], m[RU];
    uint32_t qh[RU], cw[RU][4];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        read_nib_block<FMT>(buf[u], off[u], d[u], m[u], qh[u], cw[u]);
        if constexpr (FMT == 6) d[u] *= 0.125f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 xl[NT], xh[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            xl[n] = *reinterpret_cast<const float4*>(xb[n] + 4 * i);
            xh[n] = *reinterpret_cast<const float4*>(xb[n] + 16 + 4 * i);
        }
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            uint32_t lo, hi;
            nib_code_bytes<FMT>(cw[u][i], qh[u], i, lo, hi);
            float c[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = (FMT == 6) ? sbyte_to_float(lo, j) : ubyte_to_float(lo, j);
                c[4 + j] = (FMT == 6) ? sbyte_to_float(hi, j) : ubyte_to_float(hi, j);
            }
            if constexpr (BIAS) {
#pragma unroll
                for (int j = 0; j < 8; ++j) c[j] = fmaf(d[u], c[j], m[u]);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                float a = bacc[u][n];
                a = fmaf(c[0], xl[n].x, a);
                a = fmaf(c[1], xl[n].y, a);
                a = fmaf(c[2], xl[n].z, a);
                a = fmaf(c[3], xl[n].w, a);
                a = fmaf(c[4], xh[n].x, a);
                a = fmaf(c[5], xh[n].y, a);
                a = fmaf(c[6], xh[n].z, a);
                a = fmaf(c[7], xh[n].w, a);
                bacc[u][n] = a;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if constexpr (BIAS) acc[u][n] += bacc[u][n];
            else acc[u][n] = fmaf(d[u], bacc[u][n], acc[u][n]);
        }
}

// buf[u]: 16-byte aligned LDS buffer of row unit u; off[u]: byte offset of the block in it.
template <int FMT, int RU, int NT>
__device__ __forceinline__ void block_fma(const uint8_t* const (&buf)[RU], const int (&off)[RU],
                                          const float* const (&xb)[NT], float (&acc)[RU][NT]) {
    float bacc[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) bacc[u][n] = 0.0f;
    float d[RU];
    if constexpr (FMT == 8) {
        uint32_t qw[RU][8];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            d[u] = half_bits_to_float(lds_read_u16(buf[u], off[u]));
            lds_read_dwords<8>(buf[u], off[u] + 2, qw[u]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 xv[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) xv[n] = *reinterpret_cast<const float4*>(xb[n] + 4 * i);
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const float w0 = sbyte_to_float(qw[u][i], 0);
                const float w1 = sbyte_to_float(qw[u][i], 1);
                const float w2 = sbyte_to_float(qw[u][i], 2);
                const float w3 = sbyte_to_float(qw[u][i], 3);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    float a = bacc[u][n];
                    a = fmaf(w0, xv[n].x, a);
                    a = fmaf(w1, xv[n].y, a);
                    a = fmaf(w2, xv[n].z, a);
                    a = fmaf(w3, xv[n].w, a);
                    bacc[u][n] = a;
                }
            }
        }
    } else if constexpr (FMT != 2) {
        block_fma_nib<FMT, RU, NT>(buf, off, xb, acc);
        return;
    } else {
        uint32_t cw[RU][4];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            d[u] = half_bits_to_float(lds_read_u16(buf[u], off[u])) * 0.0625f;
            lds_read_dwords<4>(buf[u], off[u] + 2, cw[u]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 xl[NT], xh[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                xl[n] = *reinterpret_cast<const float4*>(xb[n] + 4 * i);
                xh[n] = *reinterpret_cast<const float4*>(xb[n] + 16 + 4 * i);
            }
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const uint32_t t = cw[u][i] ^ 0x88888888u;
                const uint32_t lo = (t << 4) & 0xF0F0F0F0u;
                const uint32_t hi = t & 0xF0F0F0F0u;
                const float l0 = sbyte_to_float(lo, 0), l1 = sbyte_to_float(lo, 1);
                const float l2 = sbyte_to_float(lo, 2), l3 = sbyte_to_float(lo, 3);
                const float h0 = sbyte_to_float(hi, 0), h1 = sbyte_to_float(hi, 1);
                const float h2 = sbyte_to_float(hi, 2), h3 = sbyte_to_float(hi, 3);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    float a = bacc[u][n];
                    a = fmaf(l0, xl[n].x, a);
                    a = fmaf(l1, xl[n].y, a);
                    a = fmaf(l2, xl[n].z, a);
                    a = fmaf(l3, xl[n].w, a);
                    a = fmaf(h0, xh[n].x, a);
                    a = fmaf(h1, xh[n].y, a);
                    a = fmaf(h2, xh[n].z, a);
                    a = fmaf(h3, xh[n].w, a);
                    bacc[u][n] = a;
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[u][n] = fmaf(d[u], bacc[u][n], acc[u][n]);
}

// ---- fp16-pair activations with packed dot products (streaming kernels) ----
//
// The streaming kernels keep x in LDS as block floating point: each 32-value block of
// a token is scaled by a power of two 2^s that brings its largest magnitude into
// [2^14, 2^15), then rounded to fp16 (x~ = fp16(2^s x)).  Nothing overflows, and every
// element keeps a relative error <= 2^-11 as long as it is zero or 2^s |x| is a normal
// fp16 (>= 2^-14).  A block holding a nonzero element below that range (more than
// about 2^28 under the block's largest) is "wide": staging reports it, and a workgroup
// that sees one takes the exact fp32 path (gemv_rows_exact) for all its rows instead.
//
// Codes enter v_dot2_f32_f16 as exact fp16 numbers.  One v_perm or v_and_or against a
// constant high byte builds a normal half v = v0 + code * unit, and one packed fp16 add
// (or fma) removes the offset v0; the difference is representable, so it is exact:
//   Q8_0: q: the code byte xor 0x80 under 0x64 is v = 1024 + (q + 128); v - 1152;
//   Q4_0: n - 8: low nibbles under 0x6400 are v = 1024 + n, high ones (in place, bits
//         4..7) v = 1024 + 16 n; v - 1032, resp. fma(v, 1/16, -72);
//   Q4_1: n - c, the same with the block's centre c (below) in place of 8;
//   Q5_0: (u - 16) / 64: the nibble in mantissa bits 4..7 under 0x3C, the fifth bit h
//         in bit 0 of the high byte 0x3C | h, v = 1 + u/64; v - 1.25;
//   Q5_1: (u - c) / 64.
// Every product code * x~ is exact in fp32 (at most 8 + 11 significant bits, and no
// underflow: |x~| >= 2^-14 and |code| >= 2^-6), so the 16 dot2 steps of a block, each
// within an fp32 ulp of its exact value (measured), round only terms of sum |w x|: a
// code equal to the offset contributes exactly zero, and there is no large offset sum
// to cancel.  A block adds (d F p) 2^-s to the lane's sum, p = sum code * x~ (F = 64
// for the 5-bit formats, else 1).
// Biased formats: w = d u + m = d (u - c) + r with r = m + c d (exact) and the integer
// centre c of block_centre.  Then |r| <= |d| / 2 when -m / d lies in [-1/2, 31 + 1/2];
// for -m / d in (31 + 1/2, 62] (c = 31) and below -1/2 (c = 0) r has the sign of
// d (u - c) for every code; above 62 (c = 0, r = m) |w| >= |m| - 31 |d| > (|m| +
// 31 |d|) / 3.  So |d| |u - c| + |r| <= 3 |d (u - c) + r| = 3 |w| always.  The block adds
// (d F p + r X) 2^-s with X = sum x~ (a dot2 chain formed at staging), whose rounding
// is therefore within 3 times that of sum |w x~|.  (Factoring out m alone,
// d sum u x + m sum x, cancels without bound when d u + m is small against m.)
// Bound: a term passes through at most 16 dot2 steps, 2 roundings into the lane's sum,
// K / 2048 later block additions of that lane, 6 butterfly levels and 1 epilogue
// product, so with u = 2^-23 per step
//     |y - y_exact| <= (2^-11 + 3 (25 + K / 2048) 2^-23) (1 + 2^-11) sum_k |w_k x_k|,
// i.e. below 1.3e-3 sum |w x| for every K up to 2^22 (5.0e-4 at K = 14336).
// Per block the LDS copy holds 16 dwords of fp16 pairs in the order the codes are
// unpacked (see stage_x16), then X (biased formats) and 2^-s, padded to XS16 dwords so
// that the lanes' 16-byte reads at a stride of XS16 dwords hit distinct banks.
constexpr int XS16 = 20;

typedef _Float16 h2x_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2x_t as_h2x(uint32_t u) { return __builtin_bit_cast(h2x_t, u); }
__device__ __forceinline__ uint32_t h2x_bits(h2x_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2x(a), as_h2x(b), c, false);
}
// Packed fp16 a + b and a * b + c on bit patterns (exact wherever used here).
__device__ __forceinline__ uint32_t add_h2(uint32_t a, uint32_t b) { return h2x_bits(as_h2x(a) + as_h2x(b)); }
__device__ __forceinline__ uint32_t fma_h2(uint32_t a, uint32_t b, uint32_t c) {
    return h2x_bits(__builtin_elementwise_fma(as_h2x(a), as_h2x(b), as_h2x(c)));
}
// A constant held in a vector register, opaque to the optimiser: (a & m) | vconst(k)
// then selects one v_and_or_b32 (a gfx9 VOP3 instruction reads at most one scalar
// or literal operand; with both constants as literals the compiler emits v_and plus
// v_or).  Pure (a register move, no side effects), so it is hoisted out of loops.
__device__ __forceinline__ uint32_t vconst(uint32_t k) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(k));
    return r;
}
// Code pairs: bytes 0 and 2 (sel02) or 1 and 3 (sel13) of v as the low bytes of the
// two 16-bit halves, under the high byte of k (v_perm_b32 of {k, v}).
__device__ __forceinline__ uint32_t sel02(uint32_t v, uint32_t k) { return __builtin_amdgcn_perm(k, v, 0x07020400u); }
__device__ __forceinline__ uint32_t sel13(uint32_t v, uint32_t k) { return __builtin_amdgcn_perm(k, v, 0x07030401u); }

template <int FMT>
struct DotCode {
    static constexpr bool NIB4 = FMT == 2 || FMT == 3;                  // v_and_or construction
    static constexpr bool BIAS = FMT == 3 || FMT == 7;
    static constexpr uint32_t K = FMT == 8 ? 0x64646464u : 0x3C3C3C3Cu;  // v_perm high bytes
    // -v0 as an fp16 pair: -1152 (Q8_0), -1032 (Q4_0 low nibbles), -1.25 (Q5_0).
    static constexpr uint32_t NEG = FMT == 8 ? 0xE480E480u : FMT == 2 ? 0xE408E408u : 0xBD00BD00u;
    static constexpr uint32_t NEG_HI = 0xD480D480u;                     // -72 (Q4_0 high nibbles)
    static constexpr uint32_t SIXTEENTH = 0x2C002C00u;                 // 1/16
    static constexpr float F = (FMT == 6 || FMT == 7) ? 64.0f : 1.0f;
};

// The integer centre c of a biased block: round(-m / d) clamped to [0, 31] while
// -m / d <= 62, else 0 (also for a NaN quotient: d = m = 0, or both infinite).  With
// this choice r = m + c d is exact in fp32 (c = 0: r = m; otherwise |m| <= 62 |d| and
// m is no finer than half d's last place, so r spans at most 19 bits).
__device__ __forceinline__ int block_centre(float d, float m) {
    const float t = -m * __builtin_amdgcn_rcpf(d);
    const float c = fminf(fmaxf(t + 0.5f, 0.0f), 31.0f);
    return t <= 62.0f ? static_cast<int>(c) : 0;
}

// v from another lane of the row, as selected by the DPP control CTRL (all lanes of
// the 8-lane groups using it are active).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(lo))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(hi))) << 16);
}

// Unsigned key of |v| that orders nonzero magnitudes and sends +-0 above them all:
// 2 * bits(|v|) - 2 (the sign bit shifted out).
__device__ __forceinline__ uint32_t mag_key(float v) { return (__float_as_uint(v) << 1) - 2u; }

// The scale exponent se of a block with largest magnitude m (2^se m in [2^14, 2^15)),
// 2^se, 2^-se, and the key of 2^(-14 - se): a nonzero element whose key lies below it
// would not be a normal fp16 once scaled.
struct BlockScale {
    float sc, inv;
    uint32_t wide_key;
};
__device__ __forceinline__ BlockScale block_scale(float m) {
    const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu) - 127;  // floor(log2 m); -127 for 0
    const int se = min(126, 14 - e);                                            // >= -114 (m <= inf)
    BlockScale b;
    b.sc = __uint_as_float(static_cast<uint32_t>(se + 127) << 23);   // 2^se
    b.inv = __uint_as_float(static_cast<uint32_t>(127 - se) << 23);  // 2^-se
    b.wide_key = mag_key(ldexpf(1.0f, -14 - se));                    // 2^-140 .. 2^100, exact
    return b;
}

// Stage chunk c (0..7: values 4c..4c+3) of one block of one token.  Called by 8
// consecutive lanes per block, all active, lane c of the group holding chunk c.
// They agree on the block's scale with three DPP exchanges; stage_chain fills in X
// (biased formats) once every block is written.  Pair order matches the unpacking in
// block_dot:
//   Q8_0: dword 2c holds (x[4c], x[4c+2]), dword 2c+1 holds (x[4c+1], x[4c+3]) --
//         the lanes of sel02 / sel13 applied to code dword c;
//   nibble formats: code dword i holds weights 4i..4i+3 (low nibbles) and
//         16+4i..16+4i+3 (high nibbles); dwords 4i, 4i+1 pair the low ones, 4i+2,
//         4i+3 the high.
// Returns true when one of the lane's four values makes the block wide.
template <int FMT>
__device__ __forceinline__ bool stage_x16(float4 v, int c, uint32_t* blk) {
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    // Max over the 8 lanes with DPP moves: swap neighbours, swap pairs (quad_perm),
    // then mirror the two quads of the 8-lane half row.
    m = fmaxf(m, dpp_f32<0xB1>(m));   // quad_perm [1, 0, 3, 2]
    m = fmaxf(m, dpp_f32<0x4E>(m));   // quad_perm [2, 3, 0, 1]
    m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
    const BlockScale s = block_scale(m);
    const uint32_t w0 = pack_h2(v.x * s.sc, v.z * s.sc), w1 = pack_h2(v.y * s.sc, v.w * s.sc);
    const int slot = (FMT == 8) ? 2 * c : 4 * (c & 3) + ((c >> 2) << 1);
    *reinterpret_cast<uint2*>(blk + slot) = make_uint2(w0, w1);
    if (c == 0) blk[17] = __float_as_uint(s.inv);
    const uint32_t k = min(min(mag_key(v.x), mag_key(v.y)), min(mag_key(v.z), mag_key(v.w)));
    return k < s.wide_key;
}

// Rotated code order (Q8_0 and Q4_0, whose 34- and 18-byte blocks put the codes of
// every other block at an offset of 2 mod 4 in a 16-byte aligned slice): such a
// block's code dwords come from lds_read_rotated, so code dword i holds code bytes
// rot_byte(i, p), p = 0..3 (ND code dwords in all).  Aligned blocks keep 4i + p.
__host__ __device__ constexpr int rot_byte(int nd, int i, int p, bool rot) {
    return !rot ? 4 * i + p : i > 0 ? 4 * i - 2 + p : p < 2 ? p : 4 * nd - 4 + p;
}
// The value index of half h (0 = low) of staged dword j for Q8_0 / Q4_0 in either
// code order: Q8_0 pairs bytes (0, 2) and (1, 3) of code dword j / 2 (sel02, sel13);
// Q4_0 dword 4i + k pairs the low (k < 2) or high nibbles of bytes (k & 1) and
// (k & 1) + 2 of code dword i, the high nibble of byte c being value 16 + c.
template <int FMT>
__host__ __device__ constexpr int staged_value(int j, int h, bool rot) {
    return FMT == 8 ? rot_byte(8, j >> 1, (j & 1) + 2 * h, rot)
                    : ((j & 3) >= 2 ? 16 : 0) + rot_byte(4, j >> 2, (j & 1) + 2 * h, rot);
}
__device__ __forceinline__ float value_at(const float4 (&v)[8], int k) {
    const float4 t = v[k >> 2];
    return (k & 3) == 0 ? t.x : (k & 3) == 1 ? t.y : (k & 3) == 2 ? t.z : t.w;
}

// One whole block of one token staged by one lane: v holds its 32 values (chunk c =
// values 4c..4c+3).  The same block floating point and pair order as stage_x16, and
// X (biased formats: stage_chain's dot2 steps, so it is bit-identical) formed from
// the lane's own registers; the block's 20 dwords go out as five 16-byte LDS writes.
// ROT (Q8_0 / Q4_0 only) stages the pairs in the rotated code order instead.
// Returns true when the block is wide.
template <int FMT>
__device__ __forceinline__ bool stage_block(const float4 (&v)[8], uint32_t* blk, bool rot = false) {
    float m = 0.0f;
    uint32_t k = 0xFFFFFFFFu;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[c].x), fabsf(v[c].y)), fmaxf(fabsf(v[c].z), fabsf(v[c].w))));
        k = min(k, min(min(mag_key(v[c].x), mag_key(v[c].y)), min(mag_key(v[c].z), mag_key(v[c].w))));
    }
    const BlockScale s = block_scale(m);
    uint32_t w[16];
    if constexpr (FMT == 8 || FMT == 2) {
        if (rot) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                w[j] = pack_h2(value_at(v, staged_value<FMT>(j, 0, true)) * s.sc,
                               value_at(v, staged_value<FMT>(j, 1, true)) * s.sc);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                w[j] = pack_h2(value_at(v, staged_value<FMT>(j, 0, false)) * s.sc,
                               value_at(v, staged_value<FMT>(j, 1, false)) * s.sc);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int slot = 4 * (c & 3) + ((c >> 2) << 1);
            w[slot] = pack_h2(v[c].x * s.sc, v[c].z * s.sc);
            w[slot + 1] = pack_h2(v[c].y * s.sc, v[c].w * s.sc);
        }
    }
    float chain = 0.0f;
    if constexpr (DotCode<FMT>::BIAS) {
#pragma unroll
        for (int i = 0; i < 16; ++i) chain = dot2(0x3C003C00u, w[i], chain);
    }
    uint4* o = reinterpret_cast<uint4*>(blk);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    o[4] = make_uint4(__float_as_uint(chain), __float_as_uint(s.inv), 0u, 0u);
    return k < s.wide_key;
}

// Biased formats, after the staged pairs are visible: X of one block, the dot2 chain
// of its 16 dwords against (1, 1) in slot order.
template <int FMT>
__device__ __forceinline__ void stage_chain(uint32_t* blk) {
    float chain = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 w = *reinterpret_cast<const uint4*>(blk + 4 * i);
        chain = dot2(0x3C003C00u, w.x, chain);
        chain = dot2(0x3C003C00u, w.y, chain);
        chain = dot2(0x3C003C00u, w.z, chain);
        chain = dot2(0x3C003C00u, w.w, chain);
    }
    blk[16] = __float_as_uint(chain);
}

// One lane's block for RU row units and NT tokens with packed fp16 dot products
// (xb[n]: the token's staged block, XS16 dwords).  ROT (Q8_0 / Q4_0): the codes are
// read in the rotated order (lds_read_rotated), one v_perm per block in place of a
// realignment per dword, against x staged in the matching order (stage_block's rot
// for blocks whose codes start at 2 mod 4).
template <int FMT, int RU, int NT, bool ROT = false>
__device__ __forceinline__ void block_dot(const uint8_t* const (&buf)[RU], const int (&off)[RU],
                                          const uint32_t* const (&xb)[NT], float (&acc)[RU][NT]) {
    using DC = DotCode<FMT>;
    constexpr int NDW = FMT == 8 ? 8 : 4;
    constexpr uint32_t KB = DC::K;
    constexpr bool BIAS = DC::BIAS;
    constexpr bool FIVE = FMT == 6 || FMT == 7;
    float p[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) p[u][n] = 0.0f;
    float d[RU], r[RU];
    uint32_t cw[RU][NDW], qh[RU], nlo[RU], nhi[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        nlo[u] = DC::NEG;
        nhi[u] = DC::NEG_HI;
        r[u] = 0.0f;
        if constexpr (FMT == 8 || FMT == 2) {
            d[u] = half_bits_to_float(lds_read_u16(buf[u], off[u]));
            if constexpr (ROT) lds_read_rotated<NDW>(buf[u], off[u] + 2, cw[u]);
            else lds_read_dwords<NDW>(buf[u], off[u] + 2, cw[u]);
            qh[u] = 0;
        } else {
            float m;
            read_nib_block<FMT>(buf[u], off[u], d[u], m, qh[u], cw[u]);
            if constexpr (BIAS) {
                const int c = block_centre(d[u], m);
                const uint32_t cu = static_cast<uint32_t>(c);
                r[u] = fmaf(static_cast<float>(c), d[u], m);
                if constexpr (FMT == 3) {
                    nlo[u] = (0xE400u | cu) * 0x10001u;         // -(1024 + c)
                    nhi[u] = (0xD400u | (cu << 4)) * 0x10001u;  // -(64 + c)
                } else {
                    nlo[u] = (0xBC00u | (cu << 4)) * 0x10001u;  // -(1 + c / 64)
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 xv[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) xv[n] = *reinterpret_cast<const uint4*>(xb[n] + 4 * i);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            uint32_t a0, a1, a2, a3;
            if constexpr (FMT == 8) {
                const uint32_t t0 = cw[u][2 * i] ^ 0x80808080u, t1 = cw[u][2 * i + 1] ^ 0x80808080u;
                a0 = add_h2(sel02(t0, KB), nlo[u]);
                a1 = add_h2(sel13(t0, KB), nlo[u]);
                a2 = add_h2(sel02(t1, KB), nlo[u]);
                a3 = add_h2(sel13(t1, KB), nlo[u]);
            } else if constexpr (DC::NIB4) {
                // (w4i, w4i+2), (w4i+1, w4i+3) from the low nibbles of bytes 0, 2 and 1, 3;
                // (w16+4i, w16+4i+2), (w16+4i+1, w16+4i+3) from the high nibbles.
                const uint32_t w = cw[u][i], t = w >> 8, hb = vconst(0x64006400u);
                a0 = add_h2((w & 0x000F000Fu) | hb, nlo[u]);
                a1 = add_h2((t & 0x000F000Fu) | hb, nlo[u]);
                a2 = fma_h2((w & 0x00F000F0u) | hb, DC::SIXTEENTH, nhi[u]);
                a3 = fma_h2((t & 0x00F000F0u) | hb, DC::SIXTEENTH, nhi[u]);
            } else {
                static_assert(FIVE, "5-bit formats");
                // Nibbles in bits 4..7 of the low byte; the high byte of weight j's half is
                // 0x3C | h_j, one word per four weights, and the byte selectors pair byte j
                // with byte j.
                const uint32_t lo = (cw[u][i] << 4) & 0xF0F0F0F0u, hi = cw[u][i] & 0xF0F0F0F0u;
                const uint32_t hl = spread4(qh[u] >> (4 * i)) | KB, hh = spread4(qh[u] >> (16 + 4 * i)) | KB;
                a0 = add_h2(__builtin_amdgcn_perm(hl, lo, 0x06020400u), nlo[u]);
                a1 = add_h2(__builtin_amdgcn_perm(hl, lo, 0x07030501u), nlo[u]);
                a2 = add_h2(__builtin_amdgcn_perm(hh, hi, 0x06020400u), nlo[u]);
                a3 = add_h2(__builtin_amdgcn_perm(hh, hi, 0x07030501u), nlo[u]);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                float a = p[u][n];
                a = dot2(a0, xv[n].x, a);
                a = dot2(a1, xv[n].y, a);
                a = dot2(a2, xv[n].z, a);
                a = dot2(a3, xv[n].w, a);
                p[u][n] = a;
            }
        }
    }
    float xs[NT], inv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const uint2 t = *reinterpret_cast<const uint2*>(xb[n] + 16);
        xs[n] = __uint_as_float(t.x);
        inv[n] = __uint_as_float(t.y);
    }
    // (p d F) * 2^-s: each factor stays within the block's own contribution, so
    // nothing overflows unless that contribution does.
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const float dF = d[u] * DC::F;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if constexpr (BIAS) acc[u][n] = fmaf(fmaf(r[u], xs[n], p[u][n] * dF), inv[n], acc[u][n]);
            else acc[u][n] = fmaf(p[u][n] * dF, inv[n], acc[u][n]);
        }
    }
}

// ---- end of fp16-pair helpers ----

// Per-token partial sums of squares of a workgroup -> LDS.  Each wave reduces its
// lanes' values; lane 0 writes red[wave * NT + n].  A barrier must separate this
// from norm_scales.
template <int NT>
__device__ __forceinline__ void norm_partials(float (&ss)[NT], float* red, int wave, int lane) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        float v = ss[n];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[wave * NT + n] = v;
    }
}

// The token whose sums lane `lane` holds after reduce_store's transposing reduction.
template <int RU, int NT>
__device__ __forceinline__ int reduced_token(int lane) {
    constexpr int NTP = (NT == 3) ? 4 : NT;
    constexpr int LPI = kWave / (RU * NTP);
    return min((lane / LPI) % NTP, NT - 1);
}

// Inverse RMS of token n from the waves' partials, summed in wave order.
template <int NT>
__device__ __forceinline__ float norm_scale(const float* red, int waves, int n, int K, float eps) {
    float t = 0.0f;
    for (int w = 0; w < waves; ++w) t += red[w * NT + n];
    return 1.0f / sqrtf(t / static_cast<float>(K) + eps);
}

// Reduce the RU x NT per-lane partial sums of a wave and store them:
// rows row0 + (u % R) for u < R go to y (or, gated, h = silu(gate) * up with the
// up partials in u >= R), with the EP step applied (scale: the norm scale of the
// lane's reduced token, reduced_token<RU, NT>(lane)).
template <int R, int RU, int NT, bool GATED, int EP = EP_NONE>
__device__ __forceinline__ void reduce_store(float (&acc)[RU][NT], int lane, int row0, int M, float* y,
                                             int64_t ldy, float scale, const float* res) {
    constexpr int NTP = (NT == 3) ? 4 : NT;
    constexpr int V = RU * NTP;
    float v[V];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NTP; ++n) v[u * NTP + n] = (n < NT) ? acc[u][n < NT ? n : 0] : 0.0f;
    wave_reduce_transpose<V>(v, lane);
    constexpr int LPI = kWave / V;  // lanes per reduced index
    const int idx = lane / LPI;
    const bool holder = (lane % LPI) == 0;
    const int u = idx / NTP;
    const int n = idx - u * NTP;
    const int r = row0 + u;
    if constexpr (!GATED) {
        if (holder && n < NT && r < M) {
            float val = v[0];
            if constexpr (EP == EP_NORM) val *= scale;
            if constexpr (EP == EP_RES) val += res[n * ldy + r];
            y[n * ldy + r] = val;
        }
    } else {
        // The up sums sit 32 lanes above the gate sums (R * NTP * LPI == 32).
        static_assert(R * NTP * LPI == 32, "up rows reduce into the upper half");
        float upv = wave_partner<32>(v[0]);
        float gv = v[0];
        if constexpr (EP == EP_NORM) {
            gv *= scale;
            upv *= scale;
        }
        if (holder && u < R && n < NT && r < M) y[n * ldy + r] = silu(gv) * upv;
    }
}

// The exact fp32 form of the streaming kernels' product for one wave's row groups
// (groups first_group + gi * group_stride, gi < my_groups), taken by a whole workgroup
// when a block of x is wide: weights decoded exactly (the biased ones rounded once, as
// by qmm_dequant) straight from the weight buffer, fp32 x (EP_NORM: times gamma) from
// global memory, fp32 FMAs (each block's 32 products summed first, then added to the
// lane's total).  It keeps the error bound for inputs whose block floating point would
// not; no workload of interest takes it.
template <int FMT, int NT, int R, bool GATED, int EP>
__device__ inline void gemv_rows_exact(const uint8_t* Wg, const uint8_t* Wu, const float* x, float* y, int M,
                                             int K, int64_t ldx, int64_t ldy, DecodeEpi epi, float scale,
                                             int first_group, int group_stride, int my_groups, int lane) {
    constexpr int RU = GATED ? 2 * R : R;
    constexpr int BB = Fmt<FMT>::BB;
    const int nb = K / kQK;
    const int64_t rb = static_cast<int64_t>(nb) * BB;
    for (int gi = 0; gi < my_groups; ++gi) {
        const int g = first_group + gi * group_stride;
        float acc[RU][NT];
#pragma unroll
        for (int u = 0; u < RU; ++u)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[u][n] = 0.0f;
        for (int b = lane; b < nb; b += kWave) {
            float bacc[RU][NT];
#pragma unroll
            for (int u = 0; u < RU; ++u)
#pragma unroll
                for (int n = 0; n < NT; ++n) bacc[u][n] = 0.0f;
            for (int c = 0; c < 4; ++c) {
                float xv[NT][8];
                const int64_t k0 = 32 * static_cast<int64_t>(b) + 8 * c;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const float4 lo = *reinterpret_cast<const float4*>(x + n * ldx + k0);
                    const float4 hi = *reinterpret_cast<const float4*>(x + n * ldx + k0 + 4);
                    xv[n][0] = lo.x, xv[n][1] = lo.y, xv[n][2] = lo.z, xv[n][3] = lo.w;
                    xv[n][4] = hi.x, xv[n][5] = hi.y, xv[n][6] = hi.z, xv[n][7] = hi.w;
                    if constexpr (EP == EP_NORM) {
                        const float4 gl = *reinterpret_cast<const float4*>(epi.gamma + k0);
                        const float4 gh = *reinterpret_cast<const float4*>(epi.gamma + k0 + 4);
                        xv[n][0] *= gl.x, xv[n][1] *= gl.y, xv[n][2] *= gl.z, xv[n][3] *= gl.w;
                        xv[n][4] *= gh.x, xv[n][5] *= gh.y, xv[n][6] *= gh.z, xv[n][7] *= gh.w;
                    }
                }
#pragma unroll
                for (int u = 0; u < RU; ++u) {
                    const int64_t row = min(g * R + (u % R), M - 1);  // rows past M are never stored
                    const uint8_t* wb = (GATED && u >= R) ? Wu : Wg;
                    float w[8];
                    decode_chunk_f32<FMT, 8>(wb + row * rb + static_cast<int64_t>(b) * BB, c, w);
#pragma unroll
                    for (int n = 0; n < NT; ++n)
#pragma unroll
                        for (int j = 0; j < 8; ++j) bacc[u][n] = fmaf(w[j], xv[n][j], bacc[u][n]);
                }
            }
#pragma unroll
            for (int u = 0; u < RU; ++u)
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[u][n] += bacc[u][n];
        }
        reduce_store<R, RU, NT, GATED, EP>(acc, lane, g * R, M, y, ldy, scale, epi.res);
    }
}

// Whether any wave of the workgroup staged a wide block: each wave's lane 0 writes its
// ballot to flags[wave] before a workgroup barrier; read after it.  Uniform.
__device__ __forceinline__ void publish_wide(bool wide, uint32_t* flags, int wave, int lane) {
    const unsigned long long b = __ballot(wide);
    if (lane == 0) flags[wave] = b != 0ull ? 1u : 0u;
}
template <int WAVES>
__device__ __forceinline__ bool any_wide(const uint32_t* flags) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) a |= flags[w];
    return __builtin_amdgcn_readfirstlane(a) != 0;
}

}  // namespace qmm
