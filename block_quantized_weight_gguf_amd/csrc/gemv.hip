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
//   * Q8_0 / Q4_0 / Q5_0 blocks are 34 / 18 / 22 bytes, so a block is only 2-byte
//     aligned (Q4_1 / Q5_1: 20 / 24 bytes).
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
#include "gemv_block.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int GV_THREADS = 256;
constexpr int GV_WAVES = GV_THREADS / kWave;
constexpr int GV_SLICE = 64;    // blocks per K slice; lane l handles block l

template <int FMT, int NT, int R, bool GATED>
struct GemvCfg {
    static constexpr int BB = Fmt<FMT>::BB;
    static constexpr int RU = GATED ? 2 * R : R;                       // row units per wave
    static constexpr int ROWBUF = (FMT == 1) ? 16 : GV_SLICE * BB + 32;  // staged bytes per row unit
    static constexpr int NTP = (NT == 3) ? 4 : NT;                      // padded for the reduction
    static constexpr int V = RU * NTP;
    static constexpr int XS = (FMT == 1) ? GV_SLICE * 32 : GV_SLICE * XS_STRIDE;  // floats per token
};

template <int FMT, int NT, int R, bool GATED, int EP>
__global__ __launch_bounds__(GV_THREADS) void gemv_valu_kernel(const uint8_t* __restrict__ Wg,
                                                                const uint8_t* __restrict__ Wu,
                                                                const float* __restrict__ x,
                                                                float* __restrict__ y, int M, int K,
                                                                int64_t ldx, int64_t ldy, int row_begin,
                                                                DecodeEpi epi) {
    using C = GemvCfg<FMT, NT, R, GATED>;
    constexpr int BB = C::BB, RU = C::RU;
    __shared__ __align__(16) float xs[NT][C::XS];
    __shared__ __align__(16) uint8_t ws[(FMT == 1) ? 1 : GV_WAVES][(FMT == 1) ? 1 : RU][C::ROWBUF];
    __shared__ float red[(EP == EP_NORM) ? GV_WAVES * NT : 1];

    x += static_cast<int64_t>(blockIdx.y) * NT * ldx;
    y += static_cast<int64_t>(blockIdx.y) * NT * ldy;
    const float* res = (EP == EP_RES) ? epi.res + static_cast<int64_t>(blockIdx.y) * NT * ldy : nullptr;
    float ss[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) ss[n] = 0.0f;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nb = K / kQK;
    const int64_t rb = static_cast<int64_t>(nb) * BB;
    const int row0 = row_begin + blockIdx.x * (GV_WAVES * R) + wave * R;

    float acc[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[u][n] = 0.0f;

    for (int s0 = 0; s0 < nb; s0 += GV_SLICE) {
        const int sb = min(GV_SLICE, nb - s0);
        __syncthreads();  // the previous slice's readers are done with LDS

        // Stage this slice of x (NT tokens x sb*32 floats); EP_NORM: gamma .* x, with
        // the sum of squares of x gathered on the way.
        if constexpr (EP == EP_NORM) {
            for (int j = threadIdx.x; j < sb * 8; j += GV_THREADS) {  // float4 index inside the slice
                const int64_t k = static_cast<int64_t>(s0) * kQK + 4 * j;
                const int dst = (FMT == 1) ? 4 * j : (j >> 3) * XS_STRIDE + 4 * (j & 7);
                const float4 gm = *reinterpret_cast<const float4*>(epi.gamma + k);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    float4 v = *reinterpret_cast<const float4*>(x + n * ldx + k);
                    ss[n] = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss[n]))));
                    v.x *= gm.x, v.y *= gm.y, v.z *= gm.z, v.w *= gm.w;
                    *reinterpret_cast<float4*>(&xs[n][dst]) = v;
                }
            }
        } else {
            const int nx4 = NT * sb * 8;
            for (int i = threadIdx.x; i < nx4; i += GV_THREADS) {
                const int n = i / (sb * 8);
                const int j = i - n * (sb * 8);  // float4 index inside the slice
                const float4 v =
                    *reinterpret_cast<const float4*>(x + n * ldx + static_cast<int64_t>(s0) * kQK + 4 * j);
                const int dst = (FMT == 1) ? 4 * j : (j >> 3) * XS_STRIDE + 4 * (j & 7);
                *reinterpret_cast<float4*>(&xs[n][dst]) = v;
            }
        }

        // Stage this wave's weight row slices (block formats only).
        if constexpr (FMT != 1) {
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = row0 + (u % R);
                if (r < M) {
                    const bool up = GATED && u >= R;
                    stage_bytes(up ? Wu : Wg, r * rb + static_cast<int64_t>(s0) * BB, sb * BB, ws[wave][u],
                                static_cast<int64_t>(M) * rb, lane, kWave);
                }
            }
        }
        __syncthreads();

        if constexpr (FMT != 1) {
            if (lane < sb) {
                // Rows past the end decode stale LDS bytes; their sums are never stored.
                const uint8_t* buf[RU];
                int off[RU];
#pragma unroll
                for (int u = 0; u < RU; ++u) {
                    const int r = min(row0 + (u % R), M - 1);
                    buf[u] = ws[wave][u];
                    off[u] = static_cast<int>((r * rb + static_cast<int64_t>(s0) * BB) & 15) + lane * BB;
                }
                const float* xb[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) xb[n] = &xs[n][lane * XS_STRIDE];
                block_fma<FMT, RU, NT>(buf, off, xb, acc);
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

    float scale = 1.0f;
    if constexpr (EP == EP_NORM) {
        norm_partials<NT>(ss, red, wave, lane);
        __syncthreads();
        scale = norm_scale<NT>(red, GV_WAVES, reduced_token<RU, NT>(lane), K, epi.eps);
    }
    reduce_store<R, RU, NT, GATED, EP>(acc, lane, row0, M, y, ldy, scale, res);
}

template <int FMT, int NT, bool GATED, int EP>
static void launch_fmt_nt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                          int64_t chunks, int64_t row_begin, const DecodeEpi& epi, hipStream_t s) {
    constexpr int R = (FMT == 1) ? 2 : 4;
    const int64_t rows = M - row_begin;
    const dim3 grid(static_cast<unsigned>((rows + GV_WAVES * R - 1) / (GV_WAVES * R)), static_cast<unsigned>(chunks));
    hipLaunchKernelGGL((gemv_valu_kernel<FMT, NT, R, GATED, EP>), grid, dim3(GV_THREADS), 0, s,
                       static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Wu), x, y,
                       static_cast<int>(M), static_cast<int>(K), K, M, static_cast<int>(row_begin), epi);
}

template <int FMT, bool GATED, int EP>
static void launch_fmt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K, int NT,
                       int64_t chunks, int64_t row_begin, const DecodeEpi& epi, hipStream_t s) {
    switch (NT) {
        case 1: launch_fmt_nt<FMT, 1, GATED, EP>(W, Wu, x, y, M, K, chunks, row_begin, epi, s); break;
        case 2: launch_fmt_nt<FMT, 2, GATED, EP>(W, Wu, x, y, M, K, chunks, row_begin, epi, s); break;
        case 3: launch_fmt_nt<FMT, 3, GATED, EP>(W, Wu, x, y, M, K, chunks, row_begin, epi, s); break;
        default: launch_fmt_nt<FMT, 4, GATED, EP>(W, Wu, x, y, M, K, chunks, row_begin, epi, s); break;
    }
}

template <int FMT>
static void launch_fmt_any(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K, int NT,
                           int64_t chunks, int64_t row_begin, int ep, const DecodeEpi& epi, hipStream_t s) {
    if (Wu) {
        if (ep == EP_NORM) launch_fmt<FMT, true, EP_NORM>(W, Wu, x, y, M, K, NT, chunks, row_begin, epi, s);
        else launch_fmt<FMT, true, EP_NONE>(W, Wu, x, y, M, K, NT, chunks, row_begin, epi, s);
    } else if (ep == EP_NORM) {
        launch_fmt<FMT, false, EP_NORM>(W, Wu, x, y, M, K, NT, chunks, row_begin, epi, s);
    } else if (ep == EP_RES) {
        launch_fmt<FMT, false, EP_RES>(W, Wu, x, y, M, K, NT, chunks, row_begin, epi, s);
    } else {
        launch_fmt<FMT, false, EP_NONE>(W, Wu, x, y, M, K, NT, chunks, row_begin, epi, s);
    }
}

void launch_gemv_sliced(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                        int NT, int64_t chunks, int64_t row_begin, int ep, const DecodeEpi& epi, hipStream_t s) {
    if (fmt == 8) launch_fmt_any<8>(W, Wu, x, y, M, K, NT, chunks, row_begin, ep, epi, s);
    else if (fmt == 2) launch_fmt_any<2>(W, Wu, x, y, M, K, NT, chunks, row_begin, ep, epi, s);
    else if (fmt == 3) launch_fmt_any<3>(W, Wu, x, y, M, K, NT, chunks, row_begin, ep, epi, s);
    else if (fmt == 6) launch_fmt_any<6>(W, Wu, x, y, M, K, NT, chunks, row_begin, ep, epi, s);
    else if (fmt == 7) launch_fmt_any<7>(W, Wu, x, y, M, K, NT, chunks, row_begin, ep, epi, s);
    else launch_fmt_any<1>(W, Wu, x, y, M, K, NT, chunks, row_begin, ep, epi, s);
}

hipError_t launch_gemv_valu(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M,
                            int64_t K, int64_t N, hipStream_t s, int ep, const DecodeEpi& epi) {
    int64_t done = 0;
    // The residual of the pass that starts at token `done`.
    auto at = [&](int64_t d) {
        DecodeEpi e = epi;
        if (e.res) e.res += d * M;
        return e;
    };
    // Block formats: the DMA-fed streaming kernel (16-byte aligned rows, more than
    // 2 kSmallRows rows), else the register-staged one; up to 4 tokens per pass, as
    // many tokens per pass as its LDS copy of x allows; a final row it leaves is done
    // by the sliced kernel.
    while (done < N) {
        int nt = static_cast<int>(std::min<int64_t>(4, N - done));
        int64_t rows = 0;
        const DecodeEpi e = at(done);
        while (nt > 0) {
            rows = M <= 2 * kSmallRows ? 0 : launch_gemv_dma(fmt, W, Wu, x + done * K, y + done * M, M, K, nt, ep, e, s);
            if (rows == 0) rows = launch_gemv_stream(fmt, W, Wu, x + done * K, y + done * M, M, K, nt, ep, e, s);
            if (rows != 0) break;
            --nt;
        }
        if (nt == 0) break;
        if (rows < M) launch_gemv_sliced(fmt, W, Wu, x + done * K, y + done * M, M, K, nt, 1, rows, ep, e, s);
        done += nt;
    }
    // F16, or x too large for LDS: the sliced kernel, 4 tokens per pass (grid.y
    // indexes the pass) and a remainder pass.
    constexpr int64_t kMaxChunks = 65535;
    while (N - done >= 4) {
        const int64_t chunks = std::min<int64_t>((N - done) / 4, kMaxChunks);
        launch_gemv_sliced(fmt, W, Wu, x + done * K, y + done * M, M, K, 4, chunks, 0, ep, at(done), s);
        done += 4 * chunks;
    }
    if (N - done > 0)
        launch_gemv_sliced(fmt, W, Wu, x + done * K, y + done * M, M, K, static_cast<int>(N - done), 1, 0, ep,
                           at(done), s);
    return hipGetLastError();
}

}  // namespace qmm
