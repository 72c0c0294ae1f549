// Prefill GEMM, tiled for gfx950: Y[t][m] = sum_k W[m][k] X[t][k], fp16 MFMA, fp32 accumulate.
//
// ("alpaca.swift", Capabilities and Design: prefill GEMMs on the matrix hardware
// with half-precision activations; "llama.cpp Metal ...", section 3.2 and P9: a
// tiled matrix-matrix kernel above a token threshold.)  Weights are decoded from
// their GGUF blocks into fp16 LDS tiles once per (tile, K step) and fed to
// v_mfma_f32_16x16x32_f16.
//
// Work layout (wave64, 160 KB LDS per CU, 8 XCDs):
//   * A workgroup owns a 256 (weight rows) x 256 (tokens) output tile with 8 waves
//     (2 per SIMD) in a 2 x 4 arrangement; each wave computes 128 x 64 outputs as
//     8 x 4 MFMA fragments accumulating in AGPRs.
//   * Token operands never touch LDS: each wave loads its MFMA B fragments (16
//     contiguous bytes of one token row per lane) straight from L2 into VGPRs, one
//     32-wide K sub-step ahead of use.
//   * Weight operands: per K step of 64 (two blocks) the raw blocks are fetched with
//     coalesced 16-byte loads (consecutive lanes walk one row's window).  Rows are
//     16-byte aligned (K % 256 == 0), so a step's two-block segment sits at the same
//     dword offset s in its window for every row.  The bytes go through a raw LDS
//     area, then two threads per row decode one block each in the fp16 domain (a
//     code byte c becomes the half 1024 + c via v_perm with 0x64 bytes,
//     v_pk_add_f16 removes the offset exactly, v_pk_mul_f16 by the fp16 scale gives
//     fp16(d*q) with a single rounding) into the fp16 weight tile (rows padded to
//     144 bytes so each 16-lane fragment read hits distinct banks).
//   * Pipeline with one barrier per step: during step k the waves store the raw
//     bytes of step k+2, decode step k+1 into the other weight stage, run the MFMAs
//     of step k, and have the raw loads of step k+3 in flight (F16 rows skip the
//     raw area: step k copies step k+1 into the other stage).  The loop is
//     unrolled by two so that every stage is its own LDS array and the compiler can
//     overlap the decode with the MFMAs.
//   * Tile order is XCD-aware: each XCD (workgroup id % 8) takes a contiguous run
//     of tiles, walked in groups of 4 weight-row tiles so that concurrently
//     running tiles share both weight and token K slices in that XCD's L2.
//   * Gated instance: the 256 tile rows are 64 gate rows, the same 64 up rows, and
//     the next 64 of each, so each thread ends holding g and u for the same
//     outputs and applies h = silu(g) * u before the store.
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int GT_BM = 256;
constexpr int GT_BN = 256;
constexpr int GT_BK = 64;
constexpr int GT_THREADS = 512;
constexpr int GT_WLD = GT_BK + 8;          // padded weight-tile row, halfs
constexpr int GT_RAW = 80;                 // raw staging bytes per row
constexpr int GT_GROUP_M = 4;

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

template <int FMT>
struct TileGeom {
    // 16-byte loads per thread per step for the weights: F16 rows are 128-byte
    // slices (8 chunks x 256 rows / 512 threads); the block formats fetch the
    // window holding the two-block segment (68 + up to 12 bytes for Q8_0 -> 5
    // chunks, 36 + up to 12 for Q4_0 -> 3 chunks) for every row.
    static constexpr int CPR = (FMT == 1) ? 8 : (FMT == 8 ? 5 : 3);  // chunks per row
    static constexpr int NLD = (GT_BM * CPR + GT_THREADS - 1) / GT_THREADS;
};

template <int FMT, bool GATED, bool XF32>
__global__ __launch_bounds__(GT_THREADS) void gemm_tile_kernel(const uint8_t* __restrict__ Wg,
                                                                const uint8_t* __restrict__ Wu,
                                                                const void* __restrict__ Xv,
                                                                float* __restrict__ Y, int M, int K, int T,
                                                                int vec) {
    __shared__ __align__(16) _Float16 Wf0[GT_BM * GT_WLD];
    __shared__ __align__(16) _Float16 Wf1[GT_BM * GT_WLD];
    __shared__ __align__(16) uint8_t Raw0[(FMT == 1) ? 16 : GT_BM * GT_RAW];
    __shared__ __align__(16) uint8_t Raw1[(FMT == 1) ? 16 : GT_BM * GT_RAW];

    using G = TileGeom<FMT>;
    constexpr int BB = Fmt<FMT>::BB;
    constexpr int CPR = G::CPR, NLD = G::NLD;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int nb = K / kQK;
    const int64_t rb = static_cast<int64_t>(nb) * BB;
    const int nsteps = nb / 2;  // K % 64 == 0 here

    // ---- tile selection: contiguous run per XCD, grouped by GT_GROUP_M weight tiles
    const int rows_per_tile = GATED ? GT_BM / 2 : GT_BM;
    const int nMt = (M + rows_per_tile - 1) / rows_per_tile;
    const int nTt = (T + GT_BN - 1) / GT_BN;
    const int ntiles = nMt * nTt;
    const int per_xcd = (ntiles + 7) / 8;
    const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (tile >= ntiles) return;
    const int group = tile / (GT_GROUP_M * nTt);
    const int first_m = group * GT_GROUP_M;
    const int gm = min(GT_GROUP_M, nMt - first_m);
    const int in_group = tile - group * GT_GROUP_M * nTt;
    const int mt = first_m + in_group % gm;
    const int tt = in_group / gm;
    const int m0 = mt * rows_per_tile;
    const int t0 = tt * GT_BN;

    // Tile row r -> pointer to the start of its weight row (rows past the end
    // re-read the last row; their outputs are never stored).
    auto row_ptr = [&](int r) -> const uint8_t* {
        int mrow;
        const uint8_t* base;
        if constexpr (GATED) {
            const int grp = r >> 6;  // 64-row groups: gate, up, gate, up
            mrow = m0 + (grp >> 1) * 64 + (r & 63);
            base = (grp & 1) ? Wu : Wg;
        } else {
            mrow = m0 + r;
            base = Wg;
        }
        return base + min(mrow, M - 1) * rb;
    };

    // ---- weight loads: chunk c = tid + 512 * i -> tile row c / CPR, chunk c % CPR
    uint4 wr[NLD];
    auto load_w = [&](int step) {
        const int64_t seg = static_cast<int64_t>(2 * step) * BB;
        const int64_t a = (FMT == 1) ? static_cast<int64_t>(step) * 128 : (seg & ~int64_t(15));
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int c = min(tid + GT_THREADS * i, GT_BM * CPR - 1);
            const int r = c / CPR, ch = c - CPR * (c / CPR);
            // A window never passes its row's end: on a row's last step the segment ends
            // exactly at the 16-byte aligned row end; the clamp only trims the Q4_0 window.
            const int64_t o = min(a + 16 * ch, rb - 16);
            wr[i] = load16_nt(row_ptr(r) + o);
        }
    };
    // Park the loaded bytes: block formats into a raw area, F16 directly into a weight stage.
    auto store_w = [&](uint8_t* raw, _Float16* wf) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int c = tid + GT_THREADS * i;
            if (c < GT_BM * CPR) {
                const int r = c / CPR, ch = c - CPR * (c / CPR);
                if constexpr (FMT == 1) *reinterpret_cast<uint4*>(wf + r * GT_WLD + 8 * ch) = wr[i];
                else *reinterpret_cast<uint4*>(raw + r * GT_RAW + 16 * ch) = wr[i];
            }
        }
    };
    // Two threads per row: thread tid decodes block (tid & 1) of tile row tid >> 1.
    auto decode_w = [&](int step, const uint8_t* raw, _Float16* wf) {
        if constexpr (FMT != 1) {
            const int r = tid >> 1, h = tid & 1;
            const int64_t seg = static_cast<int64_t>(2 * step) * BB;
            const int sh = static_cast<int>(seg & 15) >> 2;  // dword offset of the segment in the window
            const uint32_t* src = reinterpret_cast<const uint32_t*>(raw + r * GT_RAW);
            uint32_t o[16];
            if constexpr (FMT == 8) {
                // [d0][q0 x32][d1][q1 x32]: block 0 = dwords 0..8 (codes from byte 2),
                // block 1 = scale in the high half of dword 8, codes in dwords 9..16.
                uint32_t w[9];
#pragma unroll
                for (int i = 0; i < 9; ++i) w[i] = src[sh + 8 * h + i];
                const uint32_t d = h ? (w[0] >> 16) : (w[0] & 0xFFFFu);
                const half2_t d2 = bits_h2(d | (d << 16));
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t codes = h ? w[1 + i] : align_bytes(w[i + 1], w[i], 2);
                    q8_4(codes, d2, o[2 * i], o[2 * i + 1]);
                }
            } else {
                // [d0][16 code bytes][d1][16 code bytes]: block 0 = dwords 0..4 (codes from
                // byte 2), block 1 = scale in the high half of dword 4, codes in dwords 5..8.
                uint32_t w[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) w[i] = src[sh + 4 * h + i];
                const uint32_t d = h ? (w[0] >> 16) : (w[0] & 0xFFFFu);
                const half2_t d2 = bits_h2(d | (d << 16));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t cw = h ? w[1 + i] : align_bytes(w[i + 1], w[i], 2);
                    q4_4(cw & 0x0F0F0F0Fu, d2, o[2 * i], o[2 * i + 1]);            // weights 4i..4i+3
                    q4_4((cw >> 4) & 0x0F0F0F0Fu, d2, o[8 + 2 * i], o[8 + 2 * i + 1]);  // 16+4i..
                }
            }
            uint4* dst = reinterpret_cast<uint4*>(wf + r * GT_WLD + 32 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        }
    };

    // ---- token fragments: lane l of fragment j holds X[t][k .. k+7], t = row of the
    // fragment, k = 8 * (l / 16) within the 32-wide sub-step.
    const int b_tok0 = t0 + wn * 64 + (lane & 15);
    const int b_k = 8 * (lane >> 4);
    auto load_b = [&](int kk, half8_t (&bf)[4]) {  // kk = absolute K offset of the sub-step
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = min(b_tok0 + 16 * j, T - 1);
            if constexpr (XF32) {
                const float* xp = static_cast<const float*>(Xv) + static_cast<int64_t>(t) * K + kk + b_k;
                const float4 a = reinterpret_cast<const float4*>(xp)[0];
                const float4 b = reinterpret_cast<const float4*>(xp)[1];
                const uint4 u = make_uint4(pack_h2(a.x, a.y), pack_h2(a.z, a.w), pack_h2(b.x, b.y), pack_h2(b.z, b.w));
                bf[j] = __builtin_bit_cast(half8_t, u);
            } else {
                const _Float16* xp = static_cast<const _Float16*>(Xv) + static_cast<int64_t>(t) * K + kk + b_k;
                bf[j] = *reinterpret_cast<const half8_t*>(xp);
            }
        }
    };

    float4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int a_row = wm * 128 + (lane & 15);
    const int a_k = 8 * (lane >> 4);
    half8_t bcur[4], bnxt[4];

    // One K step: MFMAs on weight stage `wc` with token fragments for K offset k0,
    // prefetching the fragments of the next sub-steps.
    auto mfma_step = [&](const _Float16* wc, int step) {
        const int k0 = step * GT_BK;
        load_b(k0 + 32, bnxt);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const half8_t af = *reinterpret_cast<const half8_t*>(wc + (a_row + 16 * i) * GT_WLD + a_k);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bcur[j], acc[i][j], 0, 0, 0);
        }
        if (step + 1 < nsteps) load_b(k0 + GT_BK, bcur);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const half8_t af = *reinterpret_cast<const half8_t*>(wc + (a_row + 16 * i) * GT_WLD + 32 + a_k);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bnxt[j], acc[i][j], 0, 0, 0);
        }
    };

    if constexpr (FMT == 1) {
        // F16: the loaded rows are copied straight into a weight stage.
        // Step k: copy data(k+1) -> Wf[(k+1)%2], issue loads of data(k+2), MFMAs on Wf[k%2].
        load_b(0, bcur);
        load_w(0);
        store_w(nullptr, Wf0);
        if (nsteps > 1) load_w(1);
        __syncthreads();
        for (int step = 0; step < nsteps; step += 2) {
            if (step + 1 < nsteps) store_w(nullptr, Wf1);
            if (step + 2 < nsteps) load_w(step + 2);
            mfma_step(Wf0, step);
            __syncthreads();
            if (step + 1 < nsteps) {
                if (step + 2 < nsteps) store_w(nullptr, Wf0);
                if (step + 3 < nsteps) load_w(step + 3);
                mfma_step(Wf1, step + 1);
                __syncthreads();
            }
        }
    } else {
        // Block formats.  Prologue: stage 0 decoded, raw(1) parked in Raw1, raw(2) in flight.
        load_b(0, bcur);
        load_w(0);
        store_w(Raw0, nullptr);
        if (nsteps > 1) load_w(1);
        __syncthreads();
        decode_w(0, Raw0, Wf0);
        if (nsteps > 1) store_w(Raw1, nullptr);
        if (nsteps > 2) load_w(2);
        __syncthreads();
        // Step k: park raw(k+2) in Raw[k%2], issue loads of raw(k+3), decode raw(k+1)
        // from Raw[(k+1)%2] into Wf[(k+1)%2], MFMAs on Wf[k%2]; one barrier.
        for (int step = 0; step < nsteps; step += 2) {
            if (step + 2 < nsteps) store_w(Raw0, nullptr);
            if (step + 3 < nsteps) load_w(step + 3);
            if (step + 1 < nsteps) decode_w(step + 1, Raw1, Wf1);
            mfma_step(Wf0, step);
            __syncthreads();
            if (step + 1 < nsteps) {
                if (step + 3 < nsteps) store_w(Raw1, nullptr);
                if (step + 4 < nsteps) load_w(step + 4);
                if (step + 2 < nsteps) decode_w(step + 2, Raw0, Wf0);
                mfma_step(Wf1, step + 1);
                __syncthreads();
            }
        }
    }

    // ---- epilogue.  D fragment: lane l holds rows 4*(l/16) + e of column l%16.
    const int er = 4 * (lane >> 4);
    const int ec = lane & 15;
    if constexpr (!GATED) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = m0 + wm * 128 + 16 * i + er;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + wn * 64 + 16 * j + ec;
                if (t < T && m < M) {
                    float* yp = Y + static_cast<int64_t>(t) * M + m;
                    if (vec) {
                        *reinterpret_cast<float4*>(yp) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (m + e < M) yp[e] = acc[i][j][e];
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 64 + 16 * i + er;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + wn * 64 + 16 * j + ec;
                if (t < T && m < M) {
                    float h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = silu(acc[i][j][e]) * acc[i + 4][j][e];
                    float* yp = Y + static_cast<int64_t>(t) * M + m;
                    if (vec) {
                        *reinterpret_cast<float4*>(yp) = make_float4(h[0], h[1], h[2], h[3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (m + e < M) yp[e] = h[e];
                    }
                }
            }
        }
    }
}

template <int FMT, bool GATED, bool XF32>
static void launch_tile_t(const void* W, const void* Wu, const void* X, float* Y, int64_t M, int64_t K, int64_t T,
                          hipStream_t s) {
    const int64_t rows_per_tile = GATED ? GT_BM / 2 : GT_BM;
    const int64_t ntiles = ((M + rows_per_tile - 1) / rows_per_tile) * ((T + GT_BN - 1) / GT_BN);
    const int64_t grid = (ntiles + 7) / 8 * 8;  // whole runs per XCD
    hipLaunchKernelGGL((gemm_tile_kernel<FMT, GATED, XF32>), dim3(static_cast<unsigned>(grid)), dim3(GT_THREADS), 0,
                       s, static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Wu), X, Y, static_cast<int>(M),
                       static_cast<int>(K), static_cast<int>(T),
                       static_cast<int>(M % 4 == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0));
}

bool launch_gemm_tile(int fmt, const void* W, const void* Wu, const void* X, bool x_is_f32, float* Y, int64_t M,
                      int64_t K, int64_t T, hipStream_t s) {
    // Block formats need 16-byte aligned rows (K % 256 == 0); F16 needs K % 64 == 0.
    if (fmt != 1 && K % 256 != 0) return false;
    if (K % 64 != 0) return false;
    const int64_t rows_per_tile = Wu ? GT_BM / 2 : GT_BM;
    const int64_t ntiles = ((M + rows_per_tile - 1) / rows_per_tile) * ((T + GT_BN - 1) / GT_BN);
    if (ntiles > (int64_t{1} << 30)) return false;
#define QMM_TILE_CASE(F)                                                                      \
    if (Wu) {                                                                                 \
        if (x_is_f32) launch_tile_t<F, true, true>(W, Wu, X, Y, M, K, T, s);                  \
        else launch_tile_t<F, true, false>(W, Wu, X, Y, M, K, T, s);                          \
    } else {                                                                                  \
        if (x_is_f32) launch_tile_t<F, false, true>(W, Wu, X, Y, M, K, T, s);                 \
        else launch_tile_t<F, false, false>(W, Wu, X, Y, M, K, T, s);                         \
    }
    if (fmt == 8) { QMM_TILE_CASE(8) }
    else if (fmt == 2) { QMM_TILE_CASE(2) }
    else { QMM_TILE_CASE(1) }
#undef QMM_TILE_CASE
    return true;
}

}  // namespace qmm
