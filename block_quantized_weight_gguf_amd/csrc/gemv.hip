// Decode GEMV on VALU: y[n][m] = sum_k W[m][k] x[n][k] with the weights decoded in
// registers straight from their GGUF block bytes ("EdgeRunner Core Architecture",
// section 3.4 Tier 1 and section 2.1 fused Q8_0 dequant + GEMV; "llama.cpp Metal
// ...", section 3.2 and P9: one mat-vec kernel per format, plus a batched variant
// for a few tokens that reads each weight once).  The gated instance fuses the
// gate and up projections with the SwiGLU epilogue h = silu(g) * u
// ("EdgeRunner Core Architecture", section 8).
//
// Layout of the work (MI355X, wave64):
//   * A workgroup is 4 waves; each wave owns R output rows (2R row units when
//     gated: R gate rows and the same R up rows) for the whole K range, so no
//     partial sum ever leaves the wave until the final reduction.
//   * K is walked in slices of 64 blocks (2048 weights).  Lane l always handles
//     block l of the slice, for every row the wave owns: the activations of that
//     block are read once from LDS and reused for all row units.
//   * Q8_0 / Q4_0 blocks are 34 / 18 bytes, so a block is only 2-byte aligned.
//     Each row slice is therefore copied to LDS with whole, coalesced 16-byte
//     loads, and each lane then re-reads its own block from LDS at any byte
//     offset (dword reads realigned with v_alignbyte).  F16 rows are 16-byte
//     aligned and are read straight into registers instead.
//   * The slice of x (N <= 4 tokens per pass) is staged in LDS once per workgroup
//     and shared by the 4 waves; the per-block stride is padded to 36 floats so
//     that the lanes' 16-byte reads hit distinct banks.
//   * Q8_0: every code is converted with one signed-byte-to-float op and enters
//     one FMA; the block scale multiplies the block's partial sum once.
//     Q4_0: xor 0x88 turns each nibble n into n ^ 8, which shifted into the high
//     half of a byte reads as the signed byte 16 * (n - 8); the same one-op
//     signed-byte convert then gives the exact code and 1/16 joins the scale.
//   * At the end each lane holds RU * NT partial sums that a transposing
//     butterfly reduces across the wave with RU*NT - 1 + few exchanges.
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int GV_THREADS = 256;
constexpr int GV_WAVES = GV_THREADS / kWave;
constexpr int GV_SLICE = 64;    // blocks per K slice; lane l handles block l
constexpr int XS_STRIDE = 36;   // floats per block in the LDS copy of x (32 + 4 padding)

template <int FMT, int NT, int R, bool GATED>
struct GemvCfg {
    static constexpr int BB = Fmt<FMT>::BB;
    static constexpr int RU = GATED ? 2 * R : R;                       // row units per wave
    static constexpr int ROWBUF = (FMT == 1) ? 16 : GV_SLICE * BB + 32;  // staged bytes per row unit
    static constexpr int NTP = (NT == 3) ? 4 : NT;                      // padded for the reduction
    static constexpr int V = RU * NTP;
    static constexpr int XS = (FMT == 1) ? GV_SLICE * 32 : GV_SLICE * XS_STRIDE;  // floats per token
};

template <int FMT, int NT, int R, bool GATED>
__global__ __launch_bounds__(GV_THREADS) void gemv_valu_kernel(const uint8_t* __restrict__ Wg,
                                                                const uint8_t* __restrict__ Wu,
                                                                const float* __restrict__ x,
                                                                float* __restrict__ y, int M, int K,
                                                                int64_t ldx, int64_t ldy) {
    using C = GemvCfg<FMT, NT, R, GATED>;
    constexpr int BB = C::BB, RU = C::RU, NTP = C::NTP, V = C::V;
    __shared__ __align__(16) float xs[NT][C::XS];
    __shared__ __align__(16) uint8_t ws[(FMT == 1) ? 1 : GV_WAVES][(FMT == 1) ? 1 : RU][C::ROWBUF];

    x += static_cast<int64_t>(blockIdx.y) * NT * ldx;
    y += static_cast<int64_t>(blockIdx.y) * NT * ldy;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nb = K / kQK;
    const int64_t rb = static_cast<int64_t>(nb) * BB;
    const int row0 = blockIdx.x * (GV_WAVES * R) + wave * R;

    float acc[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[u][n] = 0.0f;

    for (int s0 = 0; s0 < nb; s0 += GV_SLICE) {
        const int sb = min(GV_SLICE, nb - s0);
        __syncthreads();  // the previous slice's readers are done with LDS

        // Stage this slice of x (NT tokens x sb*32 floats).
        const int nx4 = NT * sb * 8;
        for (int i = threadIdx.x; i < nx4; i += GV_THREADS) {
            const int n = i / (sb * 8);
            const int j = i - n * (sb * 8);  // float4 index inside the slice
            const float4 v = *reinterpret_cast<const float4*>(x + n * ldx + static_cast<int64_t>(s0) * kQK + 4 * j);
            const int dst = (FMT == 1) ? 4 * j : (j >> 3) * XS_STRIDE + 4 * (j & 7);
            *reinterpret_cast<float4*>(&xs[n][dst]) = v;
        }

        // Stage this wave's weight row slices (block formats only).
        if constexpr (FMT != 1) {
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = row0 + (u % R);
                if (r < M) {
                    const bool up = GATED && u >= R;
                    const uint8_t* base = up ? Wu : Wg;
                    stage_bytes(base + r * rb + static_cast<int64_t>(s0) * BB, sb * BB, ws[wave][u],
                                base + static_cast<int64_t>(M) * rb, lane, kWave);
                }
            }
        }
        __syncthreads();

        if constexpr (FMT == 8) {
            if (lane < sb) {
                uint32_t qw[RU][8];
                float d[RU];
#pragma unroll
                for (int u = 0; u < RU; ++u) {
                    const int r = row0 + (u % R);
                    if (r < M) {
                        const int sh = static_cast<int>((r * rb + static_cast<int64_t>(s0) * BB) & 15);
                        const uint8_t* p = ws[wave][u] + sh + lane * BB;
                        d[u] = half_bits_to_float(lds_read_u16(p));
                        lds_read_dwords<8>(p + 2, qw[u]);
                    } else {
                        d[u] = 0.0f;
#pragma unroll
                        for (int i = 0; i < 8; ++i) qw[u][i] = 0;
                    }
                }
                float bacc[RU][NT];
#pragma unroll
                for (int u = 0; u < RU; ++u)
#pragma unroll
                    for (int n = 0; n < NT; ++n) bacc[u][n] = 0.0f;
                const int xo = lane * XS_STRIDE;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float4 xv[NT];
#pragma unroll
                    for (int n = 0; n < NT; ++n) xv[n] = *reinterpret_cast<const float4*>(&xs[n][xo + 4 * i]);
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
#pragma unroll
                for (int u = 0; u < RU; ++u)
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[u][n] = fmaf(d[u], bacc[u][n], acc[u][n]);
            }
        } else if constexpr (FMT == 2) {
            if (lane < sb) {
                uint32_t cw[RU][4];
                float d[RU];
#pragma unroll
                for (int u = 0; u < RU; ++u) {
                    const int r = row0 + (u % R);
                    if (r < M) {
                        const int sh = static_cast<int>((r * rb + static_cast<int64_t>(s0) * BB) & 15);
                        const uint8_t* p = ws[wave][u] + sh + lane * BB;
                        d[u] = half_bits_to_float(lds_read_u16(p));
                        lds_read_dwords<4>(p + 2, cw[u]);
                    } else {
                        d[u] = 0.0f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) cw[u][i] = 0;
                    }
                }
                float bacc[RU][NT];
#pragma unroll
                for (int u = 0; u < RU; ++u)
#pragma unroll
                    for (int n = 0; n < NT; ++n) bacc[u][n] = 0.0f;
                const int xo = lane * XS_STRIDE;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float4 xl[NT], xh[NT];
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        xl[n] = *reinterpret_cast<const float4*>(&xs[n][xo + 4 * i]);
                        xh[n] = *reinterpret_cast<const float4*>(&xs[n][xo + 16 + 4 * i]);
                    }
#pragma unroll
                    for (int u = 0; u < RU; ++u) {
                        // n ^ 8 in the high half of a byte is the signed byte 16 * (n - 8).
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
                // The codes entered as 16 * (n - 8); 1/16 is folded into the scale (exact).
#pragma unroll
                for (int u = 0; u < RU; ++u)
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[u][n] = fmaf(d[u] * 0.0625f, bacc[u][n], acc[u][n]);
            }
        } else {  // F16: lane l reads 16-byte chunks l, l+64, l+128, l+192 of the row slice
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = lane + kWave * t;
                if (c < 4 * sb) {
                    float4 x0[NT], x1[NT];
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        x0[n] = *reinterpret_cast<const float4*>(&xs[n][8 * c]);
                        x1[n] = *reinterpret_cast<const float4*>(&xs[n][8 * c + 4]);
                    }
#pragma unroll
                    for (int u = 0; u < RU; ++u) {
                        const int r = row0 + (u % R);
                        if (r < M) {
                            const bool up = GATED && u >= R;
                            const uint8_t* base = up ? Wu : Wg;
                            const uint4 hv = load16_nt(
                                reinterpret_cast<const uint4*>(base + r * rb + static_cast<int64_t>(s0) * 64) + c);
                            const float w0 = half_bits_to_float(hv.x), w1 = half_bits_to_float(hv.x >> 16);
                            const float w2 = half_bits_to_float(hv.y), w3 = half_bits_to_float(hv.y >> 16);
                            const float w4 = half_bits_to_float(hv.z), w5 = half_bits_to_float(hv.z >> 16);
                            const float w6 = half_bits_to_float(hv.w), w7 = half_bits_to_float(hv.w >> 16);
#pragma unroll
                            for (int n = 0; n < NT; ++n) {
                                float a = acc[u][n];
                                a = fmaf(w0, x0[n].x, a);
                                a = fmaf(w1, x0[n].y, a);
                                a = fmaf(w2, x0[n].z, a);
                                a = fmaf(w3, x0[n].w, a);
                                a = fmaf(w4, x1[n].x, a);
                                a = fmaf(w5, x1[n].y, a);
                                a = fmaf(w6, x1[n].z, a);
                                a = fmaf(w7, x1[n].w, a);
                                acc[u][n] = a;
                            }
                        }
                    }
                }
            }
        }
    }

    // Reduce the RU x NT partial sums across the wave; lane l ends with index l / (64/V).
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
    if constexpr (!GATED) {
        const int r = row0 + u;
        if (holder && n < NT && r < M) y[n * ldy + r] = v[0];
    } else {
        const float upv = __shfl(v[0], (lane + R * NTP * LPI) & (kWave - 1), kWave);
        const int r = row0 + u;
        if (holder && u < R && n < NT && r < M) y[n * ldy + r] = silu(v[0]) * upv;
    }
}

template <int FMT, int NT, bool GATED>
static void launch_fmt_nt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                          int64_t chunks, hipStream_t s) {
    constexpr int R = (FMT == 1) ? 2 : 4;
    const dim3 grid(static_cast<unsigned>((M + GV_WAVES * R - 1) / (GV_WAVES * R)), static_cast<unsigned>(chunks));
    hipLaunchKernelGGL((gemv_valu_kernel<FMT, NT, R, GATED>), grid, dim3(GV_THREADS), 0, s,
                       static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Wu), x, y,
                       static_cast<int>(M), static_cast<int>(K), K, M);
}

template <int FMT, bool GATED>
static void launch_fmt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K, int NT,
                       int64_t chunks, hipStream_t s) {
    switch (NT) {
        case 1: launch_fmt_nt<FMT, 1, GATED>(W, Wu, x, y, M, K, chunks, s); break;
        case 2: launch_fmt_nt<FMT, 2, GATED>(W, Wu, x, y, M, K, chunks, s); break;
        case 3: launch_fmt_nt<FMT, 3, GATED>(W, Wu, x, y, M, K, chunks, s); break;
        default: launch_fmt_nt<FMT, 4, GATED>(W, Wu, x, y, M, K, chunks, s); break;
    }
}

static void launch_any(int fmt, bool gated, const void* W, const void* Wu, const float* x, float* y, int64_t M,
                       int64_t K, int NT, int64_t chunks, hipStream_t s) {
    if (gated) {
        if (fmt == 8) launch_fmt<8, true>(W, Wu, x, y, M, K, NT, chunks, s);
        else if (fmt == 2) launch_fmt<2, true>(W, Wu, x, y, M, K, NT, chunks, s);
        else launch_fmt<1, true>(W, Wu, x, y, M, K, NT, chunks, s);
    } else {
        if (fmt == 8) launch_fmt<8, false>(W, Wu, x, y, M, K, NT, chunks, s);
        else if (fmt == 2) launch_fmt<2, false>(W, Wu, x, y, M, K, NT, chunks, s);
        else launch_fmt<1, false>(W, Wu, x, y, M, K, NT, chunks, s);
    }
}

hipError_t launch_gemv_valu(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M,
                            int64_t K, int64_t N, hipStream_t s) {
    const bool gated = Wu != nullptr;
    // Tokens go 4 per pass (grid.y indexes the pass); a remainder pass takes N % 4.
    constexpr int64_t kMaxChunks = 65535;
    int64_t done = 0;
    while (N - done >= 4) {
        const int64_t chunks = std::min<int64_t>((N - done) / 4, kMaxChunks);
        launch_any(fmt, gated, W, Wu, x + done * K, y + done * M, M, K, 4, chunks, s);
        done += 4 * chunks;
    }
    if (N - done > 0) launch_any(fmt, gated, W, Wu, x + done * K, y + done * M, M, K, static_cast<int>(N - done), 1, s);
    return hipGetLastError();
}

}  // namespace qmm
