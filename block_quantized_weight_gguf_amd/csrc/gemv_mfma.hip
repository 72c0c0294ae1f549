// Small-batch decode GEMV on the matrix cores: y[n][m] = sum_k W[m][k] x[n][k] for a
// few tokens (2..32), block-format weights, fp32 x and y, fp32 accumulate.
//
// ("llama.cpp Metal ...", section 3.2 and P9: a batched mat-vec for a handful of
// tokens, each weight read once and reused for every token; "EdgeRunner Core
// Architecture", section 3.4 Tier 1: the raw blocks are the only large operand.)
//
// Like single-token decode this is bound by the weight stream, so the kernel is a
// weight-streaming loop whose dot products happen to run on v_mfma_f32_16x16x32_f16:
//   * A workgroup (8 waves, one per CU: LDS-limited) owns 256 weight rows and a
//     range of K.  Each wave owns 32 rows: 2 MFMA row fragments; the tokens (padded
//     to 16 or 32) are 1 or 2 column fragments.
//   * Weights stream through a ring of 3 LDS stages by buffer->LDS DMA.  A stage
//     holds the raw GGUF bytes of 4 blocks of all 256 rows (16-byte chunks of the row
//     windows, whole 128-byte lines per load instruction) and the fp16 x of the same
//     128-wide K range for every token (16-byte chunks XOR-swizzled by token, so that
//     the 16 token rows of a fragment read hit distinct banks).  Two stages are always
//     in flight, ~80 KB per CU, which covers HBM latency at the per-CU share of the
//     bandwidth.
//   * x arrives as fp32 and is turned into the fp16 MFMA operand here, one stage
//     ahead of its use: the stage's 128 values of every token are loaded into
//     registers while the weight DMA runs, and after the current stage's MFMAs they
//     are scaled by a power of two 2^S and rounded once to fp16 into the ring slot.
//     S is a running per-token exponent: the smallest min(126, 14 - floor(log2 max))
//     over the stages converted so far, so no scaled value reaches 2^15 (fp16 holds
//     it) and each keeps fp16's relative precision unless it lies about 2^28 below
//     the largest |x| seen so far.  When S drops, the accumulators of that token are
//     multiplied by the exact power of two that moves them to the new scale; the
//     epilogue multiplies by 2^-S.  fp32 tokens thus need no conversion pass of their
//     own ("alpaca.swift", Design: half-precision activations on the matrix
//     hardware; Limitations: the activations stay unquantised).
//   * Each wave decodes its A fragments straight from the raw bytes in the fp16
//     domain (shared with the prefill GEMM) and issues 2 x (tokens / 16) MFMAs per
//     block: the matrix cores do the multiply-adds, the VALU only decodes.
//   * When the rows alone cannot fill the machine (or K is long), K is split over
//     several workgroups; their partial sums (already at the tokens' true scale) go
//     to the caller's workspace and a second kernel adds them in a fixed order and
//     applies the gated epilogue.
//   * Gated instance: stage rows 0..127 are 128 gate rows and 128..255 the up rows
//     of the same outputs; each wave takes 16 gate and the matching 16 up rows.
#include <algorithm>
#include <type_traits>

#include "mfma_tile.hpp"
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int GM_BM = 256;       // weight rows per workgroup
constexpr int GM_THREADS = 512;  // 8 waves
constexpr int GM_WAVES = GM_THREADS / 64;

// Blocks per ring stage.  4 for every format: 8-block Q4_0 stages (144 bytes, 9
// aligned chunks) double the work per barrier but halve the stages a K range splits
// into, and on the 4096-row matrices the lost parallelism costs more than the
// barriers save (measured).
template <int FMT, int NJ>
constexpr int gm_stage_blocks() { return 4; }

template <int FMT, bool GATED, int NJ, bool SPLIT>
__global__ __launch_bounds__(GM_THREADS) void gemv_mfma_kernel(const uint8_t* __restrict__ Wg,
                                                                const uint8_t* __restrict__ Wu,
                                                                const float* __restrict__ x, float* __restrict__ Y,
                                                                int M, int K, int N, int nsplit, int kst, int vec) {
    constexpr int BB = Fmt<FMT>::BB;
    constexpr int SB = gm_stage_blocks<FMT, NJ>();
    constexpr int STAGE_K = 32 * SB;
    constexpr int SEG = SB * BB;                       // row segment bytes per stage
    constexpr bool SHIFT = SEG % 16 != 0;              // odd stages start 8 bytes into their window
    constexpr int WCH = (SEG + (SHIFT ? 8 : 0) + 15) / 16;  // 16-byte chunks per row window
    constexpr int WROW = WCH * 16;        // bytes per row in a weight stage
    constexpr int WBYTES = GM_BM * WROW;  // weight bytes per stage
    constexpr int WINST = WBYTES / 1024;  // wave-wide DMA instructions per stage (weights)
    // Every wave issues WPER weight instructions per stage; surplus ones repeat the
    // stage's last instruction (same bytes to the same place), keeping the wait counts
    // fixed.
    constexpr int WPER = (WINST + GM_WAVES - 1) / GM_WAVES;
    static_assert(WINST % 2 == 0, "gate / up halves must split on instruction boundaries");
    constexpr int NTOK = 16 * NJ;                    // token rows of x per stage
    constexpr int XROW = STAGE_K * 2;                // fp16 x bytes per token row and stage
    constexpr int XC = XROW / 16;                    // 16-byte chunks per token row
    static_assert(XC == 16, "the swizzle key (token & 15) stays inside a row");
    constexpr int XBYTES = NTOK * XROW;              // x bytes per stage
    constexpr int SLOT = WBYTES + XBYTES + 4 * NTOK;  // one ring slot: weights, x, the tokens' S

    __shared__ __align__(16) uint8_t R0[SLOT];
    __shared__ __align__(16) uint8_t R1[SLOT];
    __shared__ __align__(16) uint8_t R2[SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = K / kQK;
    const int64_t rb = static_cast<int64_t>(nb) * BB;
    const int nst = K / STAGE_K;

    // ---- work unit: (row tile, K split); the splits of a tile are adjacent.
    const int rows_per_tile = GATED ? GM_BM / 2 : GM_BM;
    const int ntiles = (M + rows_per_tile - 1) / rows_per_tile;
    const int unit = blockIdx.x;
    if (unit >= ntiles * nsplit) return;
    const int tile = unit / nsplit;
    const int split = unit - tile * nsplit;
    const int m0 = tile * rows_per_tile;
    const int st0 = split * kst;
    const int st1 = min(st0 + kst, nst);

    // ---- DMA sources: a buffer resource per operand, lane offsets fixed, the stage's
    // position in the scalar offset.
    const int wrows = min(rows_per_tile, M - m0);
    const __amdgpu_buffer_rsrc_t wgr = make_rsrc(Wg + static_cast<int64_t>(m0) * rb, wrows * rb);
    const __amdgpu_buffer_rsrc_t wur = GATED ? make_rsrc(Wu + static_cast<int64_t>(m0) * rb, wrows * rb) : wgr;
    uint32_t woffs[WPER];
#pragma unroll
    for (int i = 0; i < WPER; ++i) {
        // Wave instruction n covers items 64 n .. 64 n + 63: item q = chunk q % WCH of
        // stage row q / WCH.  Rows past the end re-read the last row (never stored).
        const int n = min(wave + GM_WAVES * i, WINST - 1);
        const int q = 64 * n + lane;
        const int R = q / WCH;
        const int r = GATED ? (R & 127) : R;
        woffs[i] = static_cast<uint32_t>(min(r, wrows - 1) * rb) + 16 * (q % WCH);
    }
    // Stage st: the 16-byte aligned windows around the row segment [SEG st, SEG st +
    // SEG) of every row (with SHIFT the segment starts 0 or 8 bytes into the window).
    auto issue = [&](QMM_L3 uint8_t* S, int st) {
        const uint32_t a = (static_cast<uint32_t>(st) * SEG) & ~15u;
#pragma unroll
        for (int i = 0; i < WPER; ++i) {
            const int n = min(wave + GM_WAVES * i, WINST - 1);
            dma16((GATED && n >= WINST / 2) ? wur : wgr, woffs[i], a, S + 1024 * n);
        }
    };

    // x: thread tid converts floats 4 (tid % 32) .. 4 (tid % 32) + 3 of the stage's
    // STAGE_K for tokens tid / 32 + 16 j.  Tokens past N read token N - 1 and use
    // zeros.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, static_cast<int64_t>(N) * K * 4);
    const int ct = tid >> 5, ck = tid & 31;
    // Destination: token row t, 16-byte chunk ck / 2 (8 halfs) at slot chunk ^ (t & 15),
    // half ck % 2 of it; t & 15 == ct for every j.
    const int xdst = WBYTES + ct * XROW + 16 * ((ck >> 1) ^ ct) + 8 * (ck & 1);
    int xs[NJ];  // running exponent S of tokens ct + 16 j (127: nothing seen yet)
#pragma unroll
    for (int j = 0; j < NJ; ++j) xs[j] = 127;
    auto load_x = [&](int st, float4_t (&v)[NJ]) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            v[j] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    xr, (min(ct + 16 * j, N - 1) * K + 4 * ck) * 4, st * (STAGE_K * 4), 0));
    };
    // Scale by 2^S and round to fp16 into ring slot S_; S of every token to the slot's
    // tail (one lane per token writes it).
    auto store_x = [&](QMM_L3 uint8_t* S_, float4_t (&v)[NJ]) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (ct + 16 * j >= N) v[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            float m = fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3])));
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
            const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu) - 127;  // floor(log2 m); -127 for 0
            xs[j] = min(xs[j], min(126, 14 - e));                                     // in [-114, 126]
            const float sc = __uint_as_float(static_cast<uint32_t>(xs[j] + 127) << 23);
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t h = {pack_h2(v[j][0] * sc, v[j][1] * sc), pack_h2(v[j][2] * sc, v[j][3] * sc)};
            *reinterpret_cast<QMM_L3 u32x2_t*>(S_ + xdst + 16 * j * XROW) = h;
            if (ck == 0) reinterpret_cast<QMM_L3 int*>(S_ + WBYTES + XBYTES)[ct + 16 * j] = xs[j];
        }
    };

    QMM_L3 uint8_t* W0 = (QMM_L3 uint8_t*)R0;
    QMM_L3 uint8_t* W1 = (QMM_L3 uint8_t*)R1;
    QMM_L3 uint8_t* W2 = (QMM_L3 uint8_t*)R2;
    {
        // x loads first: waiting for them leaves the weight DMA in flight.
        float4_t v0[NJ], v1[NJ];
        load_x(st0, v0);
        load_x(min(st0 + 1, st1 - 1), v1);
        __builtin_amdgcn_sched_barrier(0);
        issue(W0, st0);
        issue(W1, min(st0 + 1, st1 - 1));
        store_x(W0, v0);
        store_x(W1, v1);
    }

    float4_t acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    int as[NJ];  // exponent S of the accumulators' token 16 j + lane % 16
#pragma unroll
    for (int j = 0; j < NJ; ++j) as[j] = 127;

    const int q4 = lane >> 4;
    // A fragment i: stage row 32 w + 16 i + l % 16; gated: fragment 0 is gate row
    // 16 w + l % 16, fragment 1 the up row of the same output.
    auto arow = [&](int i) -> int {
        if constexpr (GATED) return (i == 0 ? 16 * wave : 128 + 16 * wave) + (lane & 15);
        else return 32 * wave + 16 * i + (lane & 15);
    };
    const int arow0 = arow(0) * WROW, arow1 = arow(1) * WROW;
    // Token fragment j of block b: token 16 j + l % 16, halfs 8 q4 .. 8 q4 + 7 of the
    // block's 32 = chunk 4 b + q4 of the token row, stored at slot chunk ^ (l % 16).
    const int xrow = WBYTES + (lane & 15) * XROW;
    const int xsw = lane & 15;
    auto frag_x = [&](const QMM_L3 uint8_t* S, int j, int b) -> half8_t {
        const int c = 4 * b + q4;
        return *reinterpret_cast<const QMM_L3 half8_t*>(S + xrow + j * 16 * XROW + 16 * (c ^ xsw));
    };

    // Stage st from ring slot Wc: wait for its weight DMA (the next stage's may stay
    // in flight), barrier, load stage st + 2's x and refill the slot read on the
    // previous stage with its weights (past the end: the last stage again, into a slot
    // nobody reads), move the accumulators to the stage's S, compute, then convert
    // stage st + 2's x into that slot (the wait for the x loads leaves the new weight
    // DMA in flight).  PAR_ is the stage's parity (st0 is even), which fixes the
    // segment offset at compile time; with a run-time offset the compiler cannot tell
    // the ring slots' reads from the DMA in flight and waits for all of it.
    auto stage = [&](auto PAR_, QMM_L3 uint8_t* Wc, QMM_L3 uint8_t* Wn2, int st) {
        constexpr int sh = SHIFT ? 8 * decltype(PAR_)::value : 0;
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<WPER>();
        lds_barrier();
        float4_t v[NJ];
        load_x(min(st + 2, st1 - 1), v);
        __builtin_amdgcn_sched_barrier(0);  // the x loads stay ahead of the weight DMA
        issue(Wn2, min(st + 2, st1 - 1));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int sv = reinterpret_cast<const QMM_L3 int*>(Wc + WBYTES + XBYTES)[16 * j + (lane & 15)];
            if (__builtin_amdgcn_ballot_w64(sv != as[j])) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_amdgcn_ldexpf(acc[i][j][e], sv - as[j]);
                as[j] = sv;
            }
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const half8_t a0 = frag_raw<FMT>(Wc + arow0, sh + BB * b, q4);
            const half8_t a1 = frag_raw<FMT>(Wc + arow1, sh + BB * b, q4);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const half8_t bf = frag_x(Wc, j, b);
                acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bf, acc[0][j], 0, 0, 0);
                acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bf, acc[1][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        store_x(Wn2, v);
    };
    // Two turns of the ring per iteration (static slots and parities, no branches
    // inside, which keeps the compiler's own wait tracking exact); the remaining
    // 0-5 stages after it.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int st = st0;
    for (; st + 6 <= st1; st += 6) {
        stage(P0{}, W0, W2, st);
        stage(P1{}, W1, W0, st + 1);
        stage(P0{}, W2, W1, st + 2);
        stage(P1{}, W0, W2, st + 3);
        stage(P0{}, W1, W0, st + 4);
        stage(P1{}, W2, W1, st + 5);
    }
    if (st < st1) stage(P0{}, W0, W2, st);
    if (st + 1 < st1) stage(P1{}, W1, W0, st + 1);
    if (st + 2 < st1) stage(P0{}, W2, W1, st + 2);
    if (st + 3 < st1) stage(P1{}, W0, W2, st + 3);
    if (st + 4 < st1) stage(P0{}, W1, W0, st + 4);
    // Drain the trailing re-load DMAs before the workgroup can exit.
    wait_vm<0>();

    // ---- epilogue.  D fragment: lane l holds rows 4 (l / 16) + e of token l % 16,
    // at scale 2^S: the sums are multiplied by 2^-S.
    const int er = 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int t = 16 * j + (lane & 15);
        if (t >= N) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_amdgcn_ldexpf(acc[i][j][e], -as[j]);
        auto store4 = [&](float* yp, int m, const float (&h)[4]) {
            if (vec) {
                *reinterpret_cast<float4*>(yp) = make_float4(h[0], h[1], h[2], h[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (m + e < M) yp[e] = h[e];
            }
        };
        if constexpr (SPLIT) {
            const int Mo = GATED ? 2 * M : M;
            float* P = Y + (static_cast<int64_t>(split) * N + t) * Mo;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int m = GATED ? m0 + 16 * wave + er : m0 + 32 * wave + 16 * i + er;
                const int col = (GATED && i == 1 ? M : 0) + m;
                if (m < M) {
                    const float h[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                    store4(P + col, m, h);
                }
            }
        } else if constexpr (GATED) {
            const int m = m0 + 16 * wave + er;
            if (m < M) {
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = silu(acc[0][j][e]) * acc[1][j][e];
                store4(Y + static_cast<int64_t>(t) * M + m, m, h);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int m = m0 + 32 * wave + 16 * i + er;
                if (m < M) {
                    const float h[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                    store4(Y + static_cast<int64_t>(t) * M + m, m, h);
                }
            }
        }
    }
}

template <int FMT, bool GATED, int NJ, bool SPLIT>
static void launch_gm_t(const void* W, const void* Wu, const float* x, float* Y, int64_t M, int64_t K, int64_t N,
                        int nsplit, int kst, hipStream_t s) {
    const int64_t rows_per_tile = GATED ? GM_BM / 2 : GM_BM;
    const int64_t ntiles = (M + rows_per_tile - 1) / rows_per_tile;
    const int vec = M % 4 == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
    hipLaunchKernelGGL((gemv_mfma_kernel<FMT, GATED, NJ, SPLIT>), dim3(static_cast<unsigned>(ntiles * nsplit)),
                       dim3(GM_THREADS), 0, s, static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Wu),
                       x, Y, static_cast<int>(M), static_cast<int>(K),
                       static_cast<int>(N), nsplit, kst, vec);
}

// K is split only when the row tiles cannot give every CU a workgroup (and each split
// keeps at least 2 stages); kst is even, so that every split starts on an even stage
// (the kernel's parity bookkeeping relies on it).  32-bit lane offsets: 256 weight rows
// must span less than 2^31 bytes (K <= 2^20).
GemvMfmaPlan plan_gemv_mfma(int fmt, int64_t M, int64_t K, int64_t N, bool gated) {
    GemvMfmaPlan p;
    if (fmt == 1 || K % 256 != 0 || N < 1 || N > 32 || K > (int64_t{1} << 20)) return p;
    p.nj = N > 16 ? 2 : 1;
    const int64_t rows_per_tile = gated ? GM_BM / 2 : GM_BM;
    const int64_t ntiles = (M + rows_per_tile - 1) / rows_per_tile;
    const int64_t nst = K / (32 * 4);
    int64_t kst = nst;
    if (ntiles < 256) {
        const int64_t want = std::max<int64_t>(1, std::min<int64_t>(256 / ntiles, nst / 2));
        kst = (nst + want - 1) / want;
    }
    kst = std::min<int64_t>((kst + 1) / 2 * 2, nst);
    p.kst = static_cast<int>(kst);
    p.nsplit = static_cast<int>((nst + kst - 1) / kst);
    if (ntiles * p.nsplit > (int64_t{1} << 30)) return p;
    p.ws_bytes = p.nsplit > 1 ? static_cast<size_t>(p.nsplit) * N * (gated ? 2 * M : M) * sizeof(float) : 0;
    p.ok = true;
    return p;
}

template <int FMT, int NJ>
static void launch_gm_nj(const GemvMfmaPlan& p, const void* W, const void* Wu, const float* x, float* y, int64_t M,
                         int64_t K, int64_t N, float* ws, hipStream_t s) {
    const bool gated = Wu != nullptr;
    if (p.nsplit == 1) {
        if (gated) launch_gm_t<FMT, true, NJ, false>(W, Wu, x, y, M, K, N, 1, p.kst, s);
        else launch_gm_t<FMT, false, NJ, false>(W, Wu, x, y, M, K, N, 1, p.kst, s);
        return;
    }
    if (gated) launch_gm_t<FMT, true, NJ, true>(W, Wu, x, ws, M, K, N, p.nsplit, p.kst, s);
    else launch_gm_t<FMT, false, NJ, true>(W, Wu, x, ws, M, K, N, p.nsplit, p.kst, s);
    launch_splitk_reduce(ws, y, nullptr, N, M, p.nsplit, gated, s);
}

void launch_gemv_mfma(const GemvMfmaPlan& p, int fmt, const void* W, const void* Wu, const float* x, float* y,
                      int64_t M, int64_t K, int64_t N, float* ws, hipStream_t s) {
    const bool two = p.nj == 2;
#define QMM_GM(F)                                                   \
    if (two) launch_gm_nj<F, 2>(p, W, Wu, x, y, M, K, N, ws, s);   \
    else launch_gm_nj<F, 1>(p, W, Wu, x, y, M, K, N, ws, s);
    switch (fmt) {
        case 8: QMM_GM(8) break;
        case 2: QMM_GM(2) break;
        case 3: QMM_GM(3) break;
        case 6: QMM_GM(6) break;
        default: QMM_GM(7) break;
    }
#undef QMM_GM
}

}  // namespace qmm
