// Device-side helpers shared by the qmm kernels (gfx950 / CDNA4, wave64).
//
// Block formats ("EdgeRunner Core Architecture", sections 1.3, 3.1 and 3.2):
//   Q8_0: [fp16 d][32 x int8 q]           34 bytes, weight = d * q
//   Q4_0: [fp16 d][16 bytes of nibbles]   18 bytes, byte j: low nibble -> weight j,
//                                          high nibble -> weight j + 16; weight = d * (n - 8)
//   Q4_1: [fp16 d][fp16 m][16 bytes of nibbles]              20 bytes, weight = d * n + m
//   Q5_0: [fp16 d][u32 qh][16 bytes of nibbles]              22 bytes, weight = d * (u - 16)
//   Q5_1: [fp16 d][fp16 m][u32 qh][16 bytes of nibbles]      24 bytes, weight = d * u + m
//         (the pages give the type ids, byte counts and the bias / 5-bit nature; the
//         field order is GGUF's: nibbles in Q4_0's order, bit e of the little-endian
//         word qh is the fifth bit of element e, u = n + 16 * bit)
//   F16 : 32 halfs treated as a 64-byte "block" so every format shares the 32-wide K tiling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

constexpr int kWave = 64;
constexpr int kQK = 32;  // weights per block

template <int FMT>
struct Fmt;
template <>
struct Fmt<8> {  // Q8_0
    static constexpr int BB = 34;
};
template <>
struct Fmt<2> {  // Q4_0
    static constexpr int BB = 18;
};
template <>
struct Fmt<3> {  // Q4_1
    static constexpr int BB = 20;
};
template <>
struct Fmt<6> {  // Q5_0
    static constexpr int BB = 22;
};
template <>
struct Fmt<7> {  // Q5_1
    static constexpr int BB = 24;
};
template <>
struct Fmt<1> {  // F16
    static constexpr int BB = 64;
};

// Fields of the formats whose codes are (at least) nibbles in Q4_0's order.
template <int FMT>
struct Nib {
    static constexpr bool BIAS = FMT == 3 || FMT == 7;        // weight = d * u + m
    static constexpr bool FIVE = FMT == 6 || FMT == 7;        // fifth bits in qh
    static constexpr int QH = BIAS ? 4 : 2;                   // byte offset of qh
    static constexpr int QS = 2 + (BIAS ? 2 : 0) + (FIVE ? 4 : 0);  // byte offset of the nibbles
    static constexpr int OFF = FMT == 2 ? 8 : FMT == 6 ? 16 : 0;    // code offset of the unbiased ones
};

// Bits 0..3 of x moved to bit 0 of bytes 0..3: the four copies of x made by the
// multiply sit at bits 0, 7, 14 and 21 and do not overlap, so no carry crosses them.
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return ((x & 15u) * 0x00204081u) & 0x01010101u; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte global load marked non-temporal (streamed weights are read once).
__device__ __forceinline__ uint4 load16_nt(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}

// Signed byte j (0..3) of a dword, converted to float.
__device__ __forceinline__ float sbyte_to_float(uint32_t w, int j) {
    return static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(w >> (8 * j))));
}

// Unsigned byte j (0..3) of a dword, converted to float.
__device__ __forceinline__ float ubyte_to_float(uint32_t w, int j) {
    return static_cast<float>(static_cast<uint8_t>(w >> (8 * j)));
}

// ({hi, lo} >> 8*sh)[31:0] for sh in 0..3: realigns a byte stream read as dwords.
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t sh) {
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

// Address arithmetic in these helpers is done on integer byte offsets from the
// original (global or LDS) base pointers, never by casting a pointer to an
// integer: that keeps the loads in their own address space (global_load /
// ds_read) instead of flat loads, which would also stall every LDS wait.

// Copy the global bytes [base + off, base + off + n) to LDS such that byte
// base + off + i lands at dst + (off & 15) + i.  Whole 16-byte aligned chunks
// (base is 16-byte aligned) move with one 16-byte load each; nothing at or
// beyond base + end is read (a chunk crossing it is fetched in dword and
// halfword pieces; buffer sizes are multiples of 2).  Bytes before off inside
// the first chunk are read too and lie at or after base.  Work is spread over
// `nl` lanes.
__device__ __forceinline__ void stage_bytes(const uint8_t* base, int64_t off, int n, uint8_t* dst, int64_t end,
                                            int lane, int nl) {
    const int64_t a = off & ~int64_t(15);
    const int total = static_cast<int>(off + n - a);
    const int chunks = (total + 15) >> 4;
    for (int c = lane; c < chunks; c += nl) {
        const int64_t p = a + 16 * c;
        uint4 v;
        if (p + 16 <= end) {
            v = load16_nt(base + p);
        } else {
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t q = p + 4 * i;
                if (q + 4 <= end) w[i] = *reinterpret_cast<const uint32_t*>(base + q);
                else if (q + 2 <= end) w[i] = *reinterpret_cast<const uint16_t*>(base + q);
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        *reinterpret_cast<uint4*>(dst + 16 * c) = v;
    }
}

// Read `ND` dwords starting at LDS byte offset `off` (2-byte aligned) from the
// 4-byte aligned LDS buffer `buf`, realigned so that out[i] holds bytes
// off+4i .. off+4i+3.  Reads ND+1 dwords from the enclosing 4-byte aligned
// offset (the caller keeps 4 bytes of slack after the data).
template <int ND>
__device__ __forceinline__ void lds_read_dwords(const uint8_t* buf, int off, uint32_t (&out)[ND]) {
    const uint32_t* base = reinterpret_cast<const uint32_t*>(buf + (off & ~3));
    const uint32_t sh = static_cast<uint32_t>(off & 3);
    uint32_t d[ND + 1];
#pragma unroll
    for (int i = 0; i <= ND; ++i) d[i] = base[i];
#pragma unroll
    for (int i = 0; i < ND; ++i) out[i] = align_bytes(d[i + 1], d[i], sh);
}

// The same ND + 1 dwords read without realignment: with off = 4a + 2 (2-byte aligned
// codes), d[0] holds bytes off-2 .. off+1 and d[ND] bytes off+4ND-2 .. off+4ND+1, so
// out[0] = bytes off, off+1, off+4ND-2, off+4ND-1 (one v_perm) and out[i] = d[i]
// holds bytes off+4i-2 .. off+4i+1 for i >= 1; with off = 4a, out[i] = d[i] are the
// aligned dwords.  Every code byte appears once, in an order that depends only on
// off % 4, which the staged operand it meets is laid out for.
template <int ND>
__device__ __forceinline__ void lds_read_rotated(const uint8_t* buf, int off, uint32_t (&out)[ND]) {
    const uint32_t* base = reinterpret_cast<const uint32_t*>(buf + (off & ~3));
    const uint32_t sel = (off & 2) ? 0x05040302u : 0x03020100u;
    uint32_t d[ND + 1];
#pragma unroll
    for (int i = 0; i <= ND; ++i) d[i] = base[i];
    out[0] = __builtin_amdgcn_perm(d[ND], d[0], sel);
#pragma unroll
    for (int i = 1; i < ND; ++i) out[i] = d[i];
}

__device__ __forceinline__ uint32_t lds_read_u16(const uint8_t* buf, int off) {
    return *reinterpret_cast<const uint16_t*>(buf + off);
}

// silu(z) = z / (1 + e^-z)  ("EdgeRunner Core Architecture", section 8 SwiGLU FFN).
// expf is the ROCm device-library exponential.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// The value `send` of this lane's partner at butterfly distance OFF, in VALU
// instructions only (a ds_bpermute per step would make the reduction a chain of
// LDS round trips).  OFF = 32, 16: v_permlane32_swap / v_permlane16_swap exchange
// the two halves / the odd and even 16-lane rows; of the two registers they return,
// one keeps this lane's value and the other holds the partner's, so their xor with
// the lane's own value is the partner's, bit for bit.  OFF = 8, 4, 2, 1: DPP moves
// within a row, whose partners (row_mirror 15 - i, row_half_mirror 7 - i,
// quad_perm i ^ 2, i ^ 1) differ from the lane exactly in bit OFF and pair up
// disjoint sets of lanes at every step, like the xor partners.
template <int OFF>
__device__ __forceinline__ float wave_partner(float send) {
    if constexpr (OFF == 32 || OFF == 16) {
        const uint32_t s = __float_as_uint(send);
        const auto r = (OFF == 32) ? __builtin_amdgcn_permlane32_swap(s, s, false, false)
                                   : __builtin_amdgcn_permlane16_swap(s, s, false, false);
        return __uint_as_float(r[0] ^ r[1] ^ s);
    } else {
        constexpr int CTRL = OFF == 8 ? 0x140 : OFF == 4 ? 0x141 : OFF == 2 ? 0x4E : 0xB1;
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xF, 0xF, false));
    }
}

template <int CNT, int OFF, int V>
__device__ __forceinline__ void wave_reduce_step(float (&v)[V], int lane) {
    if constexpr (OFF >= 1) {
        if constexpr (CNT > 1) {
            const bool upper = (lane & OFF) != 0;
            constexpr int H = CNT / 2;
#pragma unroll
            for (int i = 0; i < H; ++i) {
                const float send = upper ? v[i] : v[i + H];
                const float keep = upper ? v[i + H] : v[i];
                v[i] = keep + wave_partner<OFF>(send);
            }
            wave_reduce_step<H, OFF / 2>(v, lane);
        } else {
            v[0] += wave_partner<OFF>(v[0]);
            wave_reduce_step<1, OFF / 2>(v, lane);
        }
    }
}

// Transposing butterfly reduction over a wave64 (all lanes active).  On entry every
// lane holds V partial sums v[0..V); on exit lane l holds, in v[0], the wave-wide sum
// of index l / (64 / V).  Cost: V - 1 + (6 - log2 V) exchanges instead of 6 V.
template <int V>
__device__ __forceinline__ void wave_reduce_transpose(float (&v)[V], int lane) {
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
    wave_reduce_step<V, 32>(v, lane);
}

}  // namespace qmm
