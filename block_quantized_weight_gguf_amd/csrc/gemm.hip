// Prefill GEMM on fp16 MFMA: Y[t][m] = sum_k W[m][k] X[t][k].
//
// Prefill is a genuine dense contraction, so it runs on the matrix cores
// ("alpaca.swift", Capabilities and Design: prefill GEMMs on the matrix hardware
// with half-precision activations; "llama.cpp Metal ...", section 3.2 and P9: a
// tiled matrix-matrix kernel once the token count passes a threshold).
//
// Work layout (gfx950, wave64, 160 KB LDS per CU):
//   * A workgroup computes a 256 (weight rows) x 256 (tokens) tile with 4 waves in
//     a 2 x 2 arrangement; each wave owns 128 x 128 outputs as 8 x 8 fragments of
//     v_mfma_f32_16x16x32_f16 (fp16 inputs, fp32 accumulation).
//   * K advances 64 weights (two blocks) per step.  Each thread owns one weight row
//     of the tile: it loads that row's two raw blocks from HBM, decodes them in
//     registers, rounds d*q to fp16 (nearest even) and writes 64 halfs to the LDS
//     weight tile.  The decode therefore happens once per (tile, block), not once
//     per MFMA.
//   * The activation tile (256 tokens x 64 halfs) is copied with coalesced 16-byte
//     loads.  Tokens are fp16; fp32 ones (the batched-GEMV hand-off) arrive scaled
//     per token (scale_tokens_kernel) and the epilogue multiplies by tscale[t].
//   * Global loads for step k+1 are issued before the MFMAs of step k, so HBM
//     latency hides behind the matrix work; LDS holds one stage.
//   * LDS rows are padded from 128 to 144 bytes so the 16-lane groups of each
//     16-byte fragment read fall on distinct banks.
//   * Gated instance (SwiGLU): the 256 tile rows are 64 gate rows, the same 64 up
//     rows, then the next 64 gate and up rows, so each thread ends holding g and u
//     for the same outputs and applies h = silu(g) * u in registers.
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int GM_BM = 256;      // tile rows (weights)
constexpr int GM_BN = 256;      // tile columns (tokens)
constexpr int GM_BK = 64;       // K per step (two 32-weight blocks)
constexpr int GM_LDK = GM_BK + 8;  // padded LDS row length in halfs (144 bytes)
constexpr int GM_THREADS = 256;

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    const _Float16 ha = static_cast<_Float16>(a);  // round to nearest even
    const _Float16 hb = static_cast<_Float16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// Raw bytes of one tile row for one K step, held in registers between the global
// load and the decode.
template <int FMT>
struct RawRow;
template <>
struct RawRow<8> {
    uint32_t w[17];  // two Q8_0 blocks: 68 bytes
};
template <>
struct RawRow<2> {
    uint32_t w[9];  // two Q4_0 blocks: 36 bytes
};
template <>
struct RawRow<3> {
    uint32_t w[10];  // two Q4_1 blocks: 40 bytes
};
template <>
struct RawRow<6> {
    uint32_t w[11];  // two Q5_0 blocks: 44 bytes
};
template <>
struct RawRow<7> {
    uint32_t w[12];  // two Q5_1 blocks: 48 bytes
};
template <>
struct RawRow<1> {
    uint4 w[8];  // 64 halfs
};

// Load the two blocks (k-blocks kb, kb+1) of one row.  `two` is false when only
// block kb exists (odd block count, last step).  Rows whose byte stride is a
// multiple of 4 use dword loads; otherwise (Q8_0 with an odd block count) the
// bytes are fetched as 2-byte units.
template <int FMT>
__device__ __forceinline__ void load_raw(RawRow<FMT>& rr, const uint8_t* rowp, int kb, bool two, bool valid,
                                         bool align4) {
    if constexpr (FMT == 1) {
        const uint4* p = reinterpret_cast<const uint4*>(rowp + static_cast<int64_t>(kb) * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) rr.w[i] = (valid && (two || i < 4)) ? p[i] : make_uint4(0, 0, 0, 0);
    } else {
        constexpr int BB = Fmt<FMT>::BB;
        constexpr int ND = (2 * BB) / 4;
        const uint8_t* p = rowp + static_cast<int64_t>(kb) * BB;
        const int nbytes = two ? 2 * BB : BB;
        if (align4) {
            const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
            for (int i = 0; i < ND; ++i) rr.w[i] = (valid && 4 * i < nbytes) ? q[i] : 0u;
        } else {
            const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                const uint32_t lo = (valid && 4 * i < nbytes) ? q[2 * i] : 0u;
                const uint32_t hi = (valid && 4 * i + 2 < nbytes) ? q[2 * i + 1] : 0u;
                rr.w[i] = lo | (hi << 16);
            }
        }
    }
}

// Byte i (a constant after unrolling) of the raw bytes held as dwords.
template <int N>
__device__ __forceinline__ uint32_t raw_byte(const uint32_t (&w)[N], int i) {
    return (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

// Decode one row's two blocks into 64 fp16 values fp16(w) and store them to LDS.
template <int FMT>
__device__ __forceinline__ void decode_store(const RawRow<FMT>& rr, _Float16* dst) {
    uint32_t o[32];
    if constexpr (FMT == 3 || FMT == 6 || FMT == 7) {
        // Q4_1 / Q5_0 / Q5_1 (fields as in qmm_common.hpp), block b at byte b * BB.  The
        // biased weights round once through an fp16 fma; Q5_0's d * (u - 16) is exact
        // in fp32 and rounds once on the conversion.
        using T = Nib<FMT>;
        constexpr int BB = Fmt<FMT>::BB;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int base = b * BB;
            const uint16_t dbits = static_cast<uint16_t>(raw_byte(rr.w, base) | (raw_byte(rr.w, base + 1) << 8));
            const uint16_t mbits = static_cast<uint16_t>(raw_byte(rr.w, base + 2) | (raw_byte(rr.w, base + 3) << 8));
            uint32_t qh = 0;
            if constexpr (T::FIVE)
#pragma unroll
                for (int i = 0; i < 4; ++i) qh |= raw_byte(rr.w, base + T::QH + i) << (8 * i);
#pragma unroll
            for (int e = 0; e < 32; e += 2) {
                uint32_t u[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int el = e + t;
                    const uint32_t byte = raw_byte(rr.w, base + T::QS + (el & 15));
                    u[t] = ((el < 16 ? byte : byte >> 4) & 15u) | (((qh >> el) & 1u) << 4);
                }
                if constexpr (T::BIAS) {
                    const _Float16 d = __builtin_bit_cast(_Float16, dbits), m = __builtin_bit_cast(_Float16, mbits);
                    const _Float16 w0 = __builtin_fmaf16(d, static_cast<_Float16>(static_cast<int>(u[0])), m);
                    const _Float16 w1 = __builtin_fmaf16(d, static_cast<_Float16>(static_cast<int>(u[1])), m);
                    o[16 * b + e / 2] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, w0)) |
                                        (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, w1)) << 16);
                } else {
                    const float d = half_bits_to_float(dbits);
                    o[16 * b + e / 2] = pack_half2(d * static_cast<float>(static_cast<int>(u[0]) - 16),
                                                   d * static_cast<float>(static_cast<int>(u[1]) - 16));
                }
            }
        }
    } else if constexpr (FMT == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            o[4 * i] = rr.w[i].x;
            o[4 * i + 1] = rr.w[i].y;
            o[4 * i + 2] = rr.w[i].z;
            o[4 * i + 3] = rr.w[i].w;
        }
    } else if constexpr (FMT == 8) {
        // [d0][q0 x32][d1][q1 x32]: block 0's codes start at byte 2.
        const float d0 = half_bits_to_float(rr.w[0]);
        const float d1 = half_bits_to_float(rr.w[8] >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t q0 = align_bytes(rr.w[i + 1], rr.w[i], 2);
            o[2 * i] = pack_half2(d0 * sbyte_to_float(q0, 0), d0 * sbyte_to_float(q0, 1));
            o[2 * i + 1] = pack_half2(d0 * sbyte_to_float(q0, 2), d0 * sbyte_to_float(q0, 3));
            const uint32_t q1 = rr.w[9 + i];
            o[16 + 2 * i] = pack_half2(d1 * sbyte_to_float(q1, 0), d1 * sbyte_to_float(q1, 1));
            o[16 + 2 * i + 1] = pack_half2(d1 * sbyte_to_float(q1, 2), d1 * sbyte_to_float(q1, 3));
        }
    } else {
        // [d0][16 code bytes][d1][16 code bytes]; byte j: low nibble -> j, high -> j + 16.
        const float d0 = half_bits_to_float(rr.w[0]);
        const float d1 = half_bits_to_float(rr.w[4] >> 16);
        uint32_t c0[4], c1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c0[i] = align_bytes(rr.w[i + 1], rr.w[i], 2);
            c1[i] = rr.w[5 + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t cw = b ? c1[i] : c0[i];
                const float d = b ? d1 : d0;
                const uint32_t lo = cw & 0x0F0F0F0Fu, hi = (cw >> 4) & 0x0F0F0F0Fu;
                // weights 4i..4i+3 (low nibbles) and 16+4i..16+4i+3 (high nibbles)
                o[16 * b + 2 * i] = pack_half2(d * (ubyte_to_float(lo, 0) - 8.0f), d * (ubyte_to_float(lo, 1) - 8.0f));
                o[16 * b + 2 * i + 1] = pack_half2(d * (ubyte_to_float(lo, 2) - 8.0f), d * (ubyte_to_float(lo, 3) - 8.0f));
                o[16 * b + 8 + 2 * i] = pack_half2(d * (ubyte_to_float(hi, 0) - 8.0f), d * (ubyte_to_float(hi, 1) - 8.0f));
                o[16 * b + 8 + 2 * i + 1] = pack_half2(d * (ubyte_to_float(hi, 2) - 8.0f), d * (ubyte_to_float(hi, 3) - 8.0f));
            }
        }
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int i = 0; i < 8; ++i) d4[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

template <int FMT, bool GATED>
__global__ __launch_bounds__(GM_THREADS) void gemm_mfma_kernel(const uint8_t* __restrict__ Wg,
                                                                const uint8_t* __restrict__ Wu,
                                                                const void* __restrict__ Xv,
                                                                const float* __restrict__ tscale, float* __restrict__ Y,
                                                                int M, int K, int T, int align4) {
    __shared__ __align__(16) _Float16 Ws[GM_BM * GM_LDK];
    __shared__ __align__(16) _Float16 Xs[GM_BN * GM_LDK];

    constexpr int BB = Fmt<FMT>::BB;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nb = K / kQK;
    const int64_t rb = static_cast<int64_t>(nb) * BB;

    // Output rows covered by this tile: 256 (plain) or 128 (gated: 128 gate + 128 up tile rows).
    const int m0 = blockIdx.x * (GATED ? GM_BM / 2 : GM_BM);
    const int t0 = blockIdx.y * GM_BN;

    // The weight row this thread decodes each step.
    int wrow;
    const uint8_t* wbase;
    if constexpr (GATED) {
        const int grp = tid >> 6;  // 64-row groups: gate, up, gate, up
        wrow = m0 + (grp >> 1) * 64 + (tid & 63);
        wbase = (grp & 1) ? Wu : Wg;
    } else {
        wrow = m0 + tid;
        wbase = Wg;
    }
    const bool wvalid = wrow < M;
    const uint8_t* rowp = wbase + static_cast<int64_t>(wvalid ? wrow : 0) * rb;

    // Activation copy: 256 token rows x 64 halfs = 2048 chunks of 8 halfs; 8 per thread.
    uint4 xr[8];
    auto load_x = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + GM_THREADS * i;
            const int tr = c >> 3, kc = (c & 7) * 8;
            const int t = t0 + tr;
            const bool ok = t < T && k0 + kc < K;
            const _Float16* xp = static_cast<const _Float16*>(Xv) + static_cast<int64_t>(t) * K + k0 + kc;
            xr[i] = ok ? *reinterpret_cast<const uint4*>(xp) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + GM_THREADS * i;
            const int tr = c >> 3, kc = (c & 7) * 8;
            *reinterpret_cast<uint4*>(&Xs[tr * GM_LDK + kc]) = xr[i];
        }
    };

    float4_t acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    RawRow<FMT> rr;
    load_raw<FMT>(rr, rowp, 0, nb > 1, wvalid, align4 != 0);
    load_x(0);

    const int a_row = wm * 128 + (lane & 15);
    const int b_row = wn * 128 + (lane & 15);
    const int kq = (lane >> 4) * 8;

    for (int kb = 0; kb < nb; kb += 2) {
        __syncthreads();  // previous step's MFMA reads are done
        decode_store<FMT>(rr, &Ws[tid * GM_LDK]);
        store_x();
        __syncthreads();
        if (kb + 2 < nb) {  // prefetch the next step while the matrix cores work
            load_raw<FMT>(rr, rowp, kb + 2, kb + 3 < nb, wvalid, align4 != 0);
            load_x((kb + 2) * kQK);
        }
#pragma unroll
        for (int ks = 0; ks < GM_BK; ks += 32) {
            half8_t af[8], bf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                af[i] = *reinterpret_cast<const half8_t*>(&Ws[(a_row + 16 * i) * GM_LDK + ks + kq]);
                bf[i] = *reinterpret_cast<const half8_t*>(&Xs[(b_row + 16 * i) * GM_LDK + ks + kq]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }

    // D fragment layout: lane l holds rows 4*(l/16) + e (e = 0..3) of column l%16.
    const int er = 4 * (lane >> 4);
    const int ec = lane & 15;
    if constexpr (!GATED) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = m0 + wm * 128 + 16 * i + er;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int t = t0 + wn * 128 + 16 * j + ec;
                if (t < T) {
                    const float sc = tscale != nullptr ? tscale[t] : 1.0f;
                    float* yp = Y + static_cast<int64_t>(t) * M + m;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (m + e < M) yp[e] = acc[i][j][e] * sc;
                }
            }
        }
    } else {
        // Fragments i = 0..3 are gate rows, i = 4..7 the matching up rows.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 64 + 16 * i + er;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int t = t0 + wn * 128 + 16 * j + ec;
                if (t < T) {
                    const float sc = tscale != nullptr ? tscale[t] : 1.0f;
                    float* yp = Y + static_cast<int64_t>(t) * M + m;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (m + e < M) yp[e] = silu(acc[i][j][e] * sc) * (acc[i + 4][j][e] * sc);
                }
            }
        }
    }
}

template <int FMT, bool GATED>
static void launch_t(const void* W, const void* Wu, const void* X, const float* tscale, float* Y, int64_t M, int64_t K,
                     int64_t T, hipStream_t s) {
    const int rows_per_tile = GATED ? GM_BM / 2 : GM_BM;
    const dim3 grid(static_cast<unsigned>((M + rows_per_tile - 1) / rows_per_tile),
                    static_cast<unsigned>((T + GM_BN - 1) / GM_BN));
    const int64_t rb = (K / 32) * static_cast<int64_t>(Fmt<FMT>::BB);
    hipLaunchKernelGGL((gemm_mfma_kernel<FMT, GATED>), grid, dim3(GM_THREADS), 0, s, static_cast<const uint8_t*>(W),
                       static_cast<const uint8_t*>(Wu), X, tscale, Y, static_cast<int>(M), static_cast<int>(K),
                       static_cast<int>(T), static_cast<int>(rb % 4 == 0));
}

template <int FMT>
static void launch_f(const void* W, const void* Wu, const void* X, const float* tscale, float* Y, int64_t M, int64_t K,
                     int64_t T, hipStream_t s) {
    if (Wu) launch_t<FMT, true>(W, Wu, X, tscale, Y, M, K, T, s);
    else launch_t<FMT, false>(W, Wu, X, tscale, Y, M, K, T, s);
}

size_t gemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t T, bool gated) {
    const TilePlan p = plan_gemm_tile(fmt, M, K, T, gated);
    return p.ok ? p.ws_bytes : 0;
}

hipError_t launch_gemm_mfma(int fmt, const void* W, const void* Wu, const void* X, const float* tscale, float* Y,
                            int64_t M, int64_t K, int64_t T, float* ws, hipStream_t s) {
    // The tiled kernel covers 16-byte aligned rows; this one covers every other shape.
    const TilePlan p = plan_gemm_tile(fmt, M, K, T, Wu != nullptr);
    if (p.ok) {
        launch_gemm_tile(p, fmt, W, Wu, X, tscale, Y, M, K, T, ws, s);
        return hipGetLastError();
    }
    // grid.y is limited to 65535 tiles of 256 tokens; larger T is split into passes.
    constexpr int64_t kMaxT = 65535LL * GM_BN;
    for (int64_t t = 0; t < T; t += kMaxT) {
        const int64_t tt = std::min(kMaxT, T - t);
        const void* Xp = static_cast<const char*>(X) + t * K * 2;
        const float* tsp = tscale != nullptr ? tscale + t : nullptr;
        float* Yp = Y + t * M;
        switch (fmt) {
            case 8: launch_f<8>(W, Wu, Xp, tsp, Yp, M, K, tt, s); break;
            case 2: launch_f<2>(W, Wu, Xp, tsp, Yp, M, K, tt, s); break;
            case 3: launch_f<3>(W, Wu, Xp, tsp, Yp, M, K, tt, s); break;
            case 6: launch_f<6>(W, Wu, Xp, tsp, Yp, M, K, tt, s); break;
            case 7: launch_f<7>(W, Wu, Xp, tsp, Yp, M, K, tt, s); break;
            default: launch_f<1>(W, Wu, Xp, tsp, Yp, M, K, tt, s); break;
        }
    }
    return hipGetLastError();
}

}  // namespace qmm
