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
#pragma once

#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int XS_STRIDE = 36;  // floats per block in the LDS copy of x (32 + 4 padding)

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
        float upv = __shfl(v[0], (lane + R * NTP * LPI) & (kWave - 1), kWave);
        float gv = v[0];
        if constexpr (EP == EP_NORM) {
            gv *= scale;
            upv *= scale;
        }
        if (holder && u < R && n < NT && r < M) y[n * ldy + r] = silu(gv) * upv;
    }
}

}  // namespace qmm
