// Per-block decode + FMA used by the GEMV kernels.
//
// One lane handles one 32-weight block of up to RU row units at once, reading the
// raw block bytes from LDS at any 2-byte aligned address and the matching 32
// activations per token from LDS (block stride XS_STRIDE floats).  The activations
// are read once and reused for all row units.
//   Q8_0: 32 codes -> one signed-byte-to-float op each (SDWA sext) -> one FMA each;
//         the block partial is scaled by d once.
//   Q4_0: xor 0x88 maps each nibble n to n ^ 8; moved into the high half of a byte
//         it reads as the signed byte 16 * (n - 8), so the same one-op convert gives
//         the exact code; the scale is d / 16 (exact).
//   Q5_0: the same with the fifth bit: (u ^ 16) << 3 reads as the signed byte
//         8 * (u - 16); the scale is d / 8.
//   Q4_1, Q5_1: the unsigned code u as an unsigned byte; per block and token the
//         lane sums u x and x, and adds d * sum(u x) + m * sum(x).
#pragma once

#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int XS_STRIDE = 36;  // floats per block in the LDS copy of x (32 + 4 padding)

// The fields of a Q4_1 / Q5_0 / Q5_1 block from LDS: scale, bias (biased formats),
// the fifth-bit word (5-bit formats) and the four dwords of nibbles.
template <int FMT>
__device__ __forceinline__ void read_nib_block(const uint8_t* buf, int off, float& d, float& m, uint32_t& qh,
                                               uint32_t (&cw)[4]) {
    using T = Nib<FMT>;
    d = half_bits_to_float(lds_read_u16(buf, off));
    m = T::BIAS ? half_bits_to_float(lds_read_u16(buf, off + 2)) : 0.0f;
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

// block_fma for Q4_1, Q5_0, Q5_1 (see the header comment for the code bytes).
template <int FMT, int RU, int NT>
__device__ __forceinline__ void block_fma_nib(const uint8_t* const (&buf)[RU], const int (&off)[RU],
                                              const float* const (&xb)[NT], float (&acc)[RU][NT]) {
    constexpr bool BIAS = Nib<FMT>::BIAS;
    float bacc[RU][NT], sx[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) sx[n] = 0.0f;
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
            if constexpr (BIAS) sx[n] += ((xl[n].x + xl[n].y) + (xl[n].z + xl[n].w)) +
                                         ((xh[n].x + xh[n].y) + (xh[n].z + xh[n].w));
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
            if constexpr (BIAS) acc[u][n] = fmaf(d[u], bacc[u][n], fmaf(m[u], sx[n], acc[u][n]));
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

// ---- fp16-pair activations with packed dot products (streaming kernel) ----
//
// The streaming kernel keeps x in LDS as block floating point: each 32-value block
// of a token is scaled by a power of two 2^s that brings its largest magnitude into
// [2^14, 2^15), then rounded to fp16 (x~ = fp16(2^s x)).  That cannot overflow or
// lose a block to underflow, and every element keeps a relative error <= 2^-11.
// Codes enter v_dot2_f32_f16 as normal fp16 numbers built with one v_perm against a
// constant byte (the instruction is accurate to about an fp32 ulp for normal
// operands; it loses precision on subnormal ones):
//   Q8_0: u = q + 128 (xor 0x80) as the low byte under 0x64: v = 1024 + u, and
//         w = d (v - 1152);
//   Q4_0: the nibble n in bits 4..7 under 0x3C: v = 1 + n/64, and
//         w = 64 d (v - 1.125);
//   Q5_0: the nibble as for Q4_0 and the fifth bit h in bit 0 of the high byte,
//         0x3C | h: v = 1 + h/4 + n/64 = 1 + u/64, and w = 64 d (v - 1.25);
//   Q4_1, Q5_1: v as for Q4_0 / Q5_0, with offset 1: w = 64 d (v - 1) + m.
// Both products v x~ are exact in fp32.  With
//     p = sum_j v_j x~_j   and   c = sum_j v0 x~_j   (v0 = 1152, 1.125, 1.25 or 1),
// accumulated by the same chain of dot2 steps in the same pair order, a block
// contributes (d F) (p - c) 2^-s with F = 1 or 64.  Codes all equal to the offset
// (q = 0, n = 8, u = 16) therefore give exactly zero, and the cancellation costs at most
// about 2^-24 * 16 * 2 * max(v0 / |v - v0|) ~ 3e-5 of sum |w x| (|v - v0| averages
// 64 resp. 4/64), so |y - y_exact| <= (2^-11 + 4e-5) sum |w x|, inside the 2e-3 bound.
// The biased formats add m c 2^-s (c = sum x~ there): the block's sum of x~ w.
// Per block the LDS copy holds 16 dwords of fp16 pairs in the order the codes are
// unpacked (see stage_x16), then c and 2^-s, padded to XS16 dwords so that the
// lanes' 16-byte reads at a stride of XS16 dwords hit distinct banks.
constexpr int XS16 = 20;

typedef _Float16 h2x_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2x_t as_h2x(uint32_t u) { return __builtin_bit_cast(h2x_t, u); }
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2x(a), as_h2x(b), c, false);
}
// Code pairs: bytes 0 and 2 (sel02) or 1 and 3 (sel13) of v as the low bytes of the
// two 16-bit halves, under the high byte of k (v_perm_b32 of {k, v}).
__device__ __forceinline__ uint32_t sel02(uint32_t v, uint32_t k) { return __builtin_amdgcn_perm(k, v, 0x07020400u); }
__device__ __forceinline__ uint32_t sel13(uint32_t v, uint32_t k) { return __builtin_amdgcn_perm(k, v, 0x07030401u); }

template <int FMT>
struct DotCode {
    static constexpr uint32_t K = FMT == 8 ? 0x64646464u : 0x3C3C3C3Cu;    // high bytes
    static constexpr uint32_t V0 = FMT == 8   ? 0x64806480u   // offset code pair
                                   : FMT == 2 ? 0x3C803C80u
                                   : FMT == 6 ? 0x3D003D00u
                                              : 0x3C003C00u;
    static constexpr float F = FMT == 8 ? 1.0f : 64.0f;
};

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

// Stage chunk c (0..7: values 4c..4c+3) of one block of one token.  Called by 8
// consecutive lanes per block, all active, lane c of the group holding chunk c.
// They agree on the block's scale with three DPP exchanges; stage_chain fills in
// c once every block is written.  Pair order matches
// the unpacking in block_dot:
//   Q8_0: dword 2c holds (x[4c], x[4c+2]), dword 2c+1 holds (x[4c+1], x[4c+3]) --
//         the lanes of sel02 / sel13 applied to code dword c;
//   Q4_0: code dword i holds weights 4i..4i+3 (low nibbles) and 16+4i..16+4i+3
//         (high nibbles); dwords 4i, 4i+1 pair the low ones, 4i+2, 4i+3 the high.
template <int FMT>
__device__ __forceinline__ void stage_x16(float4 v, int c, uint32_t* blk) {
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    // Max over the 8 lanes with DPP moves: swap neighbours, swap pairs (quad_perm),
    // then mirror the two quads of the 8-lane half row.
    m = fmaxf(m, dpp_f32<0xB1>(m));   // quad_perm [1, 0, 3, 2]
    m = fmaxf(m, dpp_f32<0x4E>(m));   // quad_perm [2, 3, 0, 1]
    m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
    const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu) - 127;  // floor(log2 m); -127 for 0
    const int se = min(126, 14 - e);                                            // >= -114 (m <= inf)
    const float sc = __uint_as_float(static_cast<uint32_t>(se + 127) << 23);     // 2^se
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - se) << 23);    // 2^-se
    const uint32_t w0 = pack_h2(v.x * sc, v.z * sc), w1 = pack_h2(v.y * sc, v.w * sc);
    const int slot = (FMT == 8) ? 2 * c : 4 * (c & 3) + ((c >> 2) << 1);
    *reinterpret_cast<uint2*>(blk + slot) = make_uint2(w0, w1);
    if (c == 0) blk[17] = __float_as_uint(inv);
}

// One whole block of one token staged by one lane: v holds its 32 values (chunk c =
// values 4c..4c+3).  The same block floating point and pair order as stage_x16,
// and the offset chain c (stage_chain's dot2 steps in block_dot's order, so c is
// bit-identical) formed from the lane's own registers; the block's 20 dwords go
// out as five 16-byte LDS writes.
template <int FMT>
__device__ __forceinline__ void stage_block(const float4 (&v)[8], uint32_t* blk) {
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[c].x), fabsf(v[c].y)), fmaxf(fabsf(v[c].z), fabsf(v[c].w))));
    const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu) - 127;  // floor(log2 m); -127 for 0
    const int se = min(126, 14 - e);
    const float sc = __uint_as_float(static_cast<uint32_t>(se + 127) << 23);   // 2^se
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - se) << 23);  // 2^-se
    uint32_t w[16];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int slot = (FMT == 8) ? 2 * c : 4 * (c & 3) + ((c >> 2) << 1);
        w[slot] = pack_h2(v[c].x * sc, v[c].z * sc);
        w[slot + 1] = pack_h2(v[c].y * sc, v[c].w * sc);
    }
    float chain = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) chain = dot2(DotCode<FMT>::V0, w[i], chain);
    uint4* o = reinterpret_cast<uint4*>(blk);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    o[4] = make_uint4(__float_as_uint(chain), __float_as_uint(inv), 0u, 0u);
}

// After the staged pairs are visible: c of one block, the dot2 chain over its 16
// dwords in slot order with every code equal to the offset code (block_dot's chain).
template <int FMT>
__device__ __forceinline__ void stage_chain(uint32_t* blk) {
    float chain = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 w = *reinterpret_cast<const uint4*>(blk + 4 * i);
        chain = dot2(DotCode<FMT>::V0, w.x, chain);
        chain = dot2(DotCode<FMT>::V0, w.y, chain);
        chain = dot2(DotCode<FMT>::V0, w.z, chain);
        chain = dot2(DotCode<FMT>::V0, w.w, chain);
    }
    blk[16] = __float_as_uint(chain);
}

// One lane's block for RU row units and NT tokens with packed fp16 dot products
// (xb[n]: the token's staged block, XS16 dwords).
template <int FMT, int RU, int NT>
__device__ __forceinline__ void block_dot(const uint8_t* const (&buf)[RU], const int (&off)[RU],
                                          const uint32_t* const (&xb)[NT], float (&acc)[RU][NT]) {
    constexpr int NDW = FMT == 8 ? 8 : 4;
    constexpr uint32_t KB = DotCode<FMT>::K;
    constexpr bool BIAS = FMT != 8 && Nib<FMT>::BIAS;
    constexpr bool FIVE = FMT != 8 && Nib<FMT>::FIVE;
    float p[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) p[u][n] = 0.0f;
    float d[RU], mb[RU];
    uint32_t cw[RU][NDW], qh[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        if constexpr (FMT == 8 || FMT == 2) {
            d[u] = half_bits_to_float(lds_read_u16(buf[u], off[u]));
            lds_read_dwords<NDW>(buf[u], off[u] + 2, cw[u]);
            mb[u] = 0.0f;
            qh[u] = 0;
        } else {
            read_nib_block<FMT>(buf[u], off[u], d[u], mb[u], qh[u], cw[u]);
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
                a0 = sel02(t0, KB), a1 = sel13(t0, KB), a2 = sel02(t1, KB), a3 = sel13(t1, KB);
            } else if constexpr (FIVE) {
                // Nibbles as for Q4_0; the high byte of weight j's half is 0x3C | h_j, one
                // word per four weights, and the byte selectors pair byte j with byte j.
                const uint32_t lo = (cw[u][i] << 4) & 0xF0F0F0F0u, hi = cw[u][i] & 0xF0F0F0F0u;
                const uint32_t hl = spread4(qh[u] >> (4 * i)) | KB, hh = spread4(qh[u] >> (16 + 4 * i)) | KB;
                a0 = __builtin_amdgcn_perm(hl, lo, 0x06020400u), a1 = __builtin_amdgcn_perm(hl, lo, 0x07030501u);
                a2 = __builtin_amdgcn_perm(hh, hi, 0x06020400u), a3 = __builtin_amdgcn_perm(hh, hi, 0x07030501u);
            } else {
                const uint32_t lo = (cw[u][i] << 4) & 0xF0F0F0F0u, hi = cw[u][i] & 0xF0F0F0F0u;
                a0 = sel02(lo, KB), a1 = sel13(lo, KB), a2 = sel02(hi, KB), a3 = sel13(hi, KB);
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
    float cs[NT], inv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const uint2 t = *reinterpret_cast<const uint2*>(xb[n] + 16);
        cs[n] = __uint_as_float(t.x);
        inv[n] = __uint_as_float(t.y);
    }
    // ((p - c) * d F) * 2^-s: each factor stays within the block's own contribution,
    // so nothing overflows unless that contribution does.
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const float dF = d[u] * DotCode<FMT>::F;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if constexpr (BIAS) acc[u][n] = fmaf(fmaf(mb[u], cs[n], (p[u][n] - cs[n]) * dF), inv[n], acc[u][n]);
            else acc[u][n] = fmaf((p[u][n] - cs[n]) * dF, inv[n], acc[u][n]);
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

}  // namespace qmm
