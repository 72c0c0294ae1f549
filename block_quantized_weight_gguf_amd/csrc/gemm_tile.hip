// Prefill GEMM, tiled for gfx950: Y[t][m] = sum_k W[m][k] X[t][k], fp16 MFMA, fp32 accumulate.
//
// ("alpaca.swift", Capabilities and Design: prefill GEMMs on the matrix hardware
// with half-precision activations; "llama.cpp Metal ...", section 3.2 and P9: a
// tiled matrix-matrix kernel above a token threshold.)  Weights stay in their GGUF
// blocks in HBM and are decoded to fp16 MFMA operands inside the kernel.
//
// Work layout (wave64, 160 KB LDS per CU, 8 XCDs):
//   * A workgroup owns a 256 (weight rows) x 256 (tokens) output tile (256 x 128 up
//     to 128 tokens) with 8 waves, two per SIMD: each wave computes 32 weight rows
//     x all the tile's tokens as 2 x 16 (2 x 8) v_mfma_f32_16x16x32_f16 fragments,
//     128 (64) fp32 accumulators.
//   * Both operands reach LDS by buffer->LDS DMA (buffer_load_dwordx4 ... lds): no
//     VGPRs are spent on staging and every load instruction reads whole 128-byte
//     lines.  Token tile: 256 rows x 64 halfs per K step, 16-byte chunks stored
//     XOR-swizzled by row (the swizzle is applied to the source address, since the
//     DMA writes lane L's 16 bytes at base + 16 L), so fragment reads hit distinct
//     banks.
//   * Block formats: a weight stage holds the raw GGUF bytes of two K steps (four
//     blocks) of all 256 rows.  Rows are 16-byte aligned (K % 256 == 0), so the
//     four-block segment of every row sits at the same offset (0 or 8) inside a
//     window of whole 16-byte chunks (Q8_0: 136 bytes in 9 chunks, Q4_0: 72 bytes
//     in 5, Q4_1 80 in 5, Q5_0 88 in 6, Q5_1 96 in 6).  Each wave then decodes its
//     own MFMA A fragments straight from the raw bytes (each weight row belongs to
//     one wave, so nothing is decoded twice): lane l needs 8 consecutive weights of
//     row l % 16, i.e. the block scale (and bias) and 8 code bytes (nibble formats:
//     8 nibbles, plus one byte of fifth bits).  Decoding is done in the fp16 domain:
//     a code byte c becomes the half 1024 + c via v_perm with 0x64 bytes,
//     v_pk_add_f16 removes the offset exactly and v_pk_mul_f16 by the fp16 scale (the
//     biased formats: v_pk_fma_f16 with the bias) gives the weight with a single
//     rounding.  F16 weights use the token-tile layout.
//   * Inside a K step the token fragments are read one group ahead of the MFMAs
//     that use them, in scheduling regions of their own (the compiler would
//     otherwise read each just before its MFMA and expose the LDS latency), after
//     the LDS words of the A fragments decoded in the same group.
//   * Pipeline: one barrier per K step.  After it, the DMA of the next token stage
//     (and, every second step, of the next weight stage) is issued into the buffer
//     that every wave has finished reading, then the step's fragments are read and
//     multiplied.  Before the next barrier each wave waits for its own DMA of the
//     stage about to be read; the barrier makes every wave's DMA visible.  The loop
//     is unrolled so that each stage is its own LDS array, which lets the compiler
//     see that reads of one stage do not depend on the DMA into another.
//   * Tile order is XCD-aware: each XCD (workgroup id % 8) takes a contiguous run
//     of tiles, walked in groups of 4 weight-row tiles so that concurrently
//     running tiles share both weight and token K slices in that XCD's L2.
//   * Gated instance: stage rows 0..127 hold 128 gate rows and rows 128..255 the up
//     rows of the same outputs (so each DMA instruction reads one matrix); each wave
//     takes 32 gate and the matching 32 up rows, so every lane ends holding g and u
//     for the same outputs and applies h = silu(g) * u before the store.
//   * Tokens are always fp16.  fp32 tokens (batched decode through the MFMA path)
//     arrive pre-scaled: scale_tokens_kernel wrote fp16(2^s_t x_t) per token t, and the
//     epilogue (or the split-K reduce) multiplies token t's outputs by tscale[t] =
//     2^-s_t.
#include <algorithm>
#include <type_traits>

#include "mfma_tile.hpp"
#include "qmm_common.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int GT_BM = 256;
constexpr int GT_BN = 256;
constexpr int GT_BK = 64;
constexpr int GT_THREADS = 512;
constexpr int GT_WAVES = GT_THREADS / 64;
constexpr int GT_GROUP_M = 4;


// SPLIT: the workgroup computes the K steps [split * ksteps, (split + 1) * ksteps) of
// its tile and stores its raw accumulators, as the lanes hold them, to the partial
// block of (split, tile) in Y: per wave, per fragment (i, j), 64 lanes x 16 bytes in
// lane order, so every store instruction writes 1 KB of contiguous memory (stored in
// output order, a wave's float4s land in 16 token rows, 64 bytes each: the partials,
// nsplit times the output, went out several times slower).  splitk_reduce_tiles adds
// the splits in order, maps the lanes back to outputs and applies the epilogue.
template <int FMT, bool GATED, bool SPLIT, int BN>
__global__ __launch_bounds__(GT_THREADS) void gemm_tile_kernel(const uint8_t* __restrict__ Wg,
                                                                const uint8_t* __restrict__ Wu,
                                                                const void* __restrict__ Xv,
                                                                const float* __restrict__ tscale,
                                                                float* __restrict__ Y, int M, int K, int T,
                                                                int vec, int nsplit, int ksteps) {
    using G = WStage<FMT>;
    constexpr int BB = Fmt<FMT>::BB;
    constexpr int WROW = G::WCH * 16;         // bytes per row in a weight stage
    constexpr int WBYTES = GT_BM * WROW;      // bytes per weight stage
    constexpr int WINST = WBYTES / 1024;      // wave-wide DMA instructions per weight stage
    // Weight DMA instructions per wave and stage.  When the stage does not split evenly
    // over the waves, the surplus instructions repeat the stage's last instruction
    // (same bytes to the same place), so that every wave issues the same count:
    // constant wait counts, no branch, and a destination the compiler can tell apart
    // from the other stage.
    constexpr int WPER = (WINST + GT_WAVES - 1) / GT_WAVES;
    constexpr int KPS = G::KPS;
    constexpr int XBYTES = BN * GT_BK * 2;
    constexpr int XINST = XBYTES / 1024 / GT_WAVES;          // token DMA instructions per wave and step
    constexpr int XE = 2;                     // token element bytes
    static_assert(WINST % 2 == 0, "gate / up halves must split on instruction boundaries");
    // Wave layout: 8 waves along the weight rows (each weight row is decoded by one
    // wave only), each holding GT_NI x GT_NJ 16x16 fragments (128 accumulators).
    constexpr int GT_WN = 1;
    constexpr int GT_RW = GT_BM / (GT_WAVES / GT_WN);  // weight rows per wave
    constexpr int GT_TW = BN / GT_WN;                  // tokens per wave
    constexpr int GT_NI = GT_RW / 16;
    constexpr int GT_NJ = GT_TW / 16;

    // 128-token tiles (T <= 128, block formats, fp16 tokens) do half the MFMA work per
    // K step of a 256-token tile, too little to cover HBM latency with the token DMA one
    // step ahead.  Their token stages span two K steps like the weight stages, so both
    // operands are fetched a whole stage (two steps) ahead, and only the first step of
    // a stage needs a wait and a barrier.
    constexpr bool X2 = BN == 128 && KPS == 2;
    constexpr int XSTAGE = X2 ? 2 * XBYTES : XBYTES;  // bytes per token stage
    __shared__ __align__(16) uint8_t Xs0[XSTAGE];
    __shared__ __align__(16) uint8_t Xs1[XSTAGE];
    __shared__ __align__(16) uint8_t Ws0[WBYTES];
    __shared__ __align__(16) uint8_t Ws1[WBYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / GT_WN, wn = wave % GT_WN;  // GT_RW weight rows x GT_TW tokens per wave
    const int nb = K / kQK;
    const int64_t rb = static_cast<int64_t>(nb) * BB;
    const int nsteps = K / GT_BK;

    // ---- tile selection: contiguous run per XCD, grouped by GT_GROUP_M weight tiles
    const int rows_per_tile = GATED ? GT_BM / 2 : GT_BM;
    const int nMt = (M + rows_per_tile - 1) / rows_per_tile;
    const int nTt = (T + BN - 1) / BN;
    const int ntiles = nMt * nTt;
    const int nunits = ntiles * (SPLIT ? nsplit : 1);
    const int per_xcd = (nunits + 7) / 8;
    const int unit = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (unit >= nunits) return;
    const int tile = SPLIT ? unit / nsplit : unit;
    const int split = SPLIT ? unit - tile * nsplit : 0;
    // K steps of this workgroup (a multiple of 4 steps per split, so that block-format
    // weight stages keep their global parity).
    const int kbeg = SPLIT ? split * ksteps : 0;
    const int kend = SPLIT ? min(kbeg + ksteps, nsteps) : nsteps;
    const int group = tile / (GT_GROUP_M * nTt);
    const int first_m = group * GT_GROUP_M;
    const int gm = min(GT_GROUP_M, nMt - first_m);
    const int in_group = tile - group * GT_GROUP_M * nTt;
    const int mt = first_m + in_group % gm;
    const int tt = in_group / gm;
    const int m0 = mt * rows_per_tile;
    const int t0 = tt * BN;

    // ---- DMA sources: a buffer resource per operand tile (uniform) plus a 32-bit
    // lane offset fixed for the whole K loop; the K position goes in the scalar
    // offset.  A tile spans 256 rows, so offsets stay below 2^31 (the launcher checks).
    // Swizzled 128-byte-row tiles (tokens, F16 weights): wave instruction n = wave + 8 i
    // fills rows 8n .. 8n+7; lane L writes slot L & 7 of row 8n + L / 8, which holds
    // chunk (L & 7) ^ (row & 7) of that row.
    const int sw_chunk = (lane & 7) ^ ((lane >> 3) & 7);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(static_cast<const uint8_t*>(Xv) + static_cast<int64_t>(t0) * K * XE,
                                                static_cast<int64_t>(T - t0) * K * XE);
    uint32_t xoffs[XINST];
#pragma unroll
    for (int i = 0; i < XINST; ++i) {
        const int R = 8 * (wave + GT_WAVES * i) + (lane >> 3);
        xoffs[i] = static_cast<uint32_t>((min(t0 + R, T - 1) - t0) * K * XE + 8 * XE * sw_chunk);
    }
    // Weight stage rows: tile row R is global row m0 + R; gated tiles hold the 128 gate
    // rows in stage rows 0..127 and the same 128 up rows in 128..255.  Rows past the
    // end re-read the last row; their outputs are never stored.
    const int wrows = min(rows_per_tile, M - m0);
    const __amdgpu_buffer_rsrc_t wgr = make_rsrc(Wg + static_cast<int64_t>(m0) * rb, wrows * rb);
    const __amdgpu_buffer_rsrc_t wur = GATED ? make_rsrc(Wu + static_cast<int64_t>(m0) * rb, wrows * rb) : wgr;
    auto row_off = [&](int R) -> uint32_t {
        const int r = GATED ? (R & 127) : R;
        return static_cast<uint32_t>(min(r, wrows - 1) * rb);
    };
    uint32_t woffs[WPER];
#pragma unroll
    for (int i = 0; i < WPER; ++i) {
        if constexpr (FMT == 1) {
            const int R = 8 * (wave + GT_WAVES * i) + (lane >> 3);
            woffs[i] = row_off(R) + 16 * sw_chunk;
        } else {
            // Block formats: wave instruction n covers items 64 n .. 64 n + 63 of the
            // stage, item q = chunk q % WCH of tile row q / WCH.
            const int n = min(wave + GT_WAVES * i, WINST - 1);
            const int q = 64 * n + lane;
            woffs[i] = row_off(q / G::WCH) + 16 * (q % G::WCH);
        }
    }

    // Issue the DMA of weight stage `st` (K steps st*KPS ..) into buffer Wd.
    auto issue_w = [&](QMM_L3 uint8_t* Wd, int st) {
        uint32_t a;
        if constexpr (FMT == 1) a = static_cast<uint32_t>(st) * 128;
        else a = (static_cast<uint32_t>(st) * (2 * KPS * BB)) & ~15u;
#pragma unroll
        for (int i = 0; i < WPER; ++i) {
            const int n = min(wave + GT_WAVES * i, WINST - 1);
            dma16((GATED && n >= WINST / 2) ? wur : wgr, woffs[i], a, Wd + 1024 * n);
        }
    };

    // Token step k: DMA into Xd.
    auto issue_x = [&](QMM_L3 uint8_t* Xd, int k) {
#pragma unroll
        for (int i = 0; i < XINST; ++i)
            dma16(xr, xoffs[i], static_cast<uint32_t>(k) * 128, Xd + 1024 * (wave + GT_WAVES * i));
    };

    float4_t acc[GT_NI][GT_NJ];
#pragma unroll
    for (int i = 0; i < GT_NI; ++i)
#pragma unroll
        for (int j = 0; j < GT_NJ; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Fragment addressing.  Token fragment j of sub-step ks: row GT_TW wn + 16 j + l % 16,
    // chunk 4 ks + l / 16 (swizzled by row & 7 = l & 7).
    const int q4 = lane >> 4;
    int xoff[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        xoff[ks] = (GT_TW * wn + (lane & 15)) * 128 + (((4 * ks + q4) ^ (lane & 7)) << 4);
    // Weight fragment i: stage row GT_RW wm + 16 i + l % 16; gated: the first half of the
    // fragments are gate rows (GT_RW / 2) wm + 16 i + l % 16, the second half the up
    // rows of the same outputs.
    constexpr int NH = GT_NI / 2;
    constexpr int ND = (GT_NI + 1) / 2;   // A fragments decoded per decode group
    constexpr int NDG = GT_NI / ND;       // decode groups per sub-step (1 or 2)
    auto arow = [&](int i) -> int {
        if constexpr (GATED) return (i < NH ? (GT_RW / 2) * wm + 16 * i : 128 + (GT_RW / 2) * wm + 16 * (i - NH)) + (lane & 15);
        else return GT_RW * wm + 16 * i + (lane & 15);
    };

    // Decode A fragment i (weights 8 q4 .. 8 q4 + 7 of block b of the stage) from a raw
    // weight stage.  `sh` is the segment's offset in the row window (8 for odd stages).
    auto frag_a = [&](const QMM_L3 uint8_t* Wsrc, int i, int b, int sh) -> half8_t {
        const int rowb = arow(i) * WROW;
        if constexpr (FMT == 1) {
            (void)sh;
            // Swizzled 128-byte rows; the row's swizzle key is l & 7.
            return *reinterpret_cast<const QMM_L3 half8_t*>(Wsrc + rowb + (((4 * b + q4) ^ (lane & 7)) << 4));
        } else {
            return frag_raw<FMT>(Wsrc + rowb, sh + BB * b, q4);  // block start inside the row window
        }
    };

    half8_t a0[GT_NI], a1[GT_NI];
    // Decode fragments i0 .. i0 + NH - 1 of block b into a.
    auto decode2 = [&](half8_t (&a)[GT_NI], int i0, const QMM_L3 uint8_t* Wc, int b, int sh) {
#pragma unroll
        for (int i = i0; i < i0 + ND; ++i) a[i] = frag_a(Wc, i, b, sh);
    };
    // The MFMAs of both sub-steps of a K step.  Token fragments are read in groups of
    // NJG, one group ahead of the MFMAs that use them: each group's reads sit in their
    // own scheduling region, after the LDS reads of the A fragments decoded in that
    // group, so that waiting for the decode's words never waits for the token reads
    // (LDS waits count in issue order) and the LDS latency of a group is covered by the
    // previous group's MFMAs.  The decode of the next A fragments (sub-step 0: a1 from
    // block nb0; sub-step 1: a0 of the next step from block nb1; skipped when negative)
    // is spread over the first two groups of each sub-step.
    using RawT = std::conditional_t<FMT == 1, half8_t, RawA>;
    auto load_a = [&](const QMM_L3 uint8_t* Wsrc, int i, int b, int sh) -> RawT {
        const int rowb = arow(i) * WROW;
        if constexpr (FMT == 1) {
            (void)sh;
            return *reinterpret_cast<const QMM_L3 half8_t*>(Wsrc + rowb + (((4 * b + q4) ^ (lane & 7)) << 4));
        } else {
            return frag_load<FMT>(Wsrc + rowb, sh + BB * b, q4);
        }
    };
    auto dec_a = [&](const RawT& r, int b, int sh) -> half8_t {
        if constexpr (FMT == 1) return r;
        else return frag_decode<FMT>(r, sh + BB * b, q4);
    };
    // Group size: as many fragments read ahead as the registers allow (the 256-token
    // tile holds 128 accumulators; the gated instance needs more besides).
    constexpr int NJG_MAX = BN == 128 ? 4 : GATED ? 1 : 2;
    constexpr int NJG = (GT_NJ / 2 < NJG_MAX) ? GT_NJ / 2 : NJG_MAX;
    constexpr int NG = GT_NJ / NJG;
    static_assert(GT_NJ % NJG == 0 && NG >= 2, "token fragment groups");
    auto mfma_step = [&](half8_t (&a0r)[GT_NI], half8_t (&a1r)[GT_NI], const QMM_L3 uint8_t* Xc, int nb0, int nb1,
                         const QMM_L3 uint8_t* Wc, int sh) {
        half8_t bf[2][NJG];
        auto readg = [&](half8_t (&b)[NJG], int q) {
            const int ks = q / NG, g = q % NG;
#pragma unroll
            for (int jj = 0; jj < NJG; ++jj)
                b[jj] = *reinterpret_cast<const QMM_L3 half8_t*>(Xc + xoff[ks] + (NJG * g + jj) * 16 * 128);
        };
        readg(bf[0], 0);
#pragma unroll
        for (int q = 0; q < 2 * NG; ++q) {
            const int ks = q / NG, g = q % NG;
            const int nbq = ks == 0 ? nb0 : nb1;
            const bool dec = g < NDG && nbq >= 0;
            __builtin_amdgcn_sched_barrier(0);
            RawT raw[ND];
            if (dec) {
#pragma unroll
                for (int i = 0; i < ND; ++i) raw[i] = load_a(Wc, ND * g + i, nbq, sh);
            }
            if (q + 1 < 2 * NG) readg(bf[(q + 1) & 1], q + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (dec) {
#pragma unroll
                for (int i = 0; i < ND; ++i) {
                    if (ks == 0) a1r[ND * g + i] = dec_a(raw[i], nbq, sh);
                    else a0r[ND * g + i] = dec_a(raw[i], nbq, sh);
                }
            }
#pragma unroll
            for (int jj = 0; jj < NJG; ++jj) {
#pragma unroll
                for (int i = 0; i < GT_NI; ++i) {
                    const half8_t ai = ks == 0 ? a0r[i] : a1r[i];
                    acc[i][NJG * g + jj] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(ai, bf[q & 1][jj], acc[i][NJG * g + jj], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    QMM_L3 uint8_t* X0 = (QMM_L3 uint8_t*)Xs0;
    QMM_L3 uint8_t* X1 = (QMM_L3 uint8_t*)Xs1;
    QMM_L3 uint8_t* W0 = (QMM_L3 uint8_t*)Ws0;
    QMM_L3 uint8_t* W1 = (QMM_L3 uint8_t*)Ws1;
    const int send = kend / KPS;  // one past the last weight stage

    // Step k with token stage XS (= k % 2), weight stage WS, block pair KK.  Order:
    // finish own DMA / staging of this step's stages, barrier, issue the prefetch of
    // token step k+1 (and of weight stage k/KPS + 1 on the first step of a stage),
    // compute.  Prefetches past the end re-load the last step into the free buffer,
    // which keeps the loop body free of branches (and the wait counts constant): on
    // the second step of a block-format stage the weight DMA issued on the previous
    // step, after the token DMA needed now, may stay in flight.
    //
    // Two-step token stages (X2): the stage's token and weight DMAs were issued on the
    // first step of the previous stage and nothing after them, so that step waits for
    // all DMA and then issues the next stage of both; the second step needs neither a
    // wait nor a barrier (its data arrived with the first step's).
    auto step = [&](auto XS_, auto WS_, auto KK_, int k) {
        constexpr int XS = decltype(XS_)::value, WS = decltype(WS_)::value, KK = decltype(KK_)::value;
        QMM_L3 uint8_t* Xc = X2 ? (WS ? X1 : X0) + KK * XBYTES : (XS ? X1 : X0);
        QMM_L3 uint8_t* Xn = XS ? X0 : X1;
        QMM_L3 uint8_t* Wc = WS ? W1 : W0;
        QMM_L3 uint8_t* Wn = WS ? W0 : W1;
        if constexpr (X2) {
            if constexpr (KK == 0) {
                wait_vm<0>();
                lds_barrier();
                QMM_L3 uint8_t* Xs = WS ? X0 : X1;  // the other token stage
                issue_x(Xs, min(k + 2, kend - 1));
                issue_x(Xs + XBYTES, min(k + 3, kend - 1));
                issue_w(Wn, min(k / KPS + 1, send - 1));
            }
        } else {
            if constexpr (KPS == 2 && KK == 1) wait_vm<WPER>();
            else wait_vm<0>();
            lds_barrier();
            issue_x(Xn, min(k + 1, kend - 1));
            if constexpr (KK == 0) issue_w(Wn, min(k / KPS + 1, send - 1));
        }
        constexpr int SH = stage_shift<FMT>(WS);
        // a0 holds this step's first sub-step when it was decoded on the previous step
        // (second step of a block-format stage); otherwise decode it now.
        constexpr bool PRE = KPS == 2;
        if constexpr (!(PRE && KK == 1)) {
            decode2(a0, 0, Wc, 2 * KK, SH);
            if constexpr (NDG > 1) decode2(a0, ND, Wc, 2 * KK, SH);
        }
        mfma_step(a0, a1, Xc, 2 * KK + 1, (PRE && KK == 0) ? 2 : -1, Wc, SH);
        __builtin_amdgcn_sched_barrier(0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // ---- prologue: stage 0 of both operands
    issue_w(W0, kbeg / KPS);
    issue_x(X0, kbeg);
    if constexpr (X2) issue_x(X0 + XBYTES, min(kbeg + 1, kend - 1));
    if constexpr (KPS == 2) {
        // K % 256 == 0: whole groups of 4 steps (weight stages 0, 0, 1, 1).
        for (int k = kbeg; k < kend; k += 4) {
            step(I0{}, I0{}, I0{}, k);
            step(I1{}, I0{}, I1{}, k + 1);
            step(I0{}, I1{}, I0{}, k + 2);
            step(I1{}, I1{}, I1{}, k + 3);
        }
    } else {
        int k = kbeg;
        for (; k + 2 <= kend; k += 2) {
            step(I0{}, I0{}, I0{}, k);
            step(I1{}, I1{}, I0{}, k + 1);
        }
        if (k < kend) step(I0{}, I0{}, I0{}, k);
    }
    // Drain the trailing re-load DMAs before the workgroup can exit.
    wait_vm<0>();

    // ---- epilogue.  D fragment: lane l holds rows 4*(l/16) + e of column l%16.
    const int er = 4 * (lane >> 4);
    const int ec = lane & 15;
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
        // Partial block (split, tile): GT_WAVES x GT_NI x GT_NJ x 64 float4, lane fastest.
        float4* P = reinterpret_cast<float4*>(Y) +
                    ((static_cast<int64_t>(split) * ntiles + tile) * GT_WAVES + wave) * (GT_NI * GT_NJ * 64) + lane;
#pragma unroll
        for (int i = 0; i < GT_NI; ++i)
#pragma unroll
            for (int j = 0; j < GT_NJ; ++j)
                P[(i * GT_NJ + j) * 64] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    } else {
        constexpr int NOUT = GATED ? NH : GT_NI;  // output fragments per wave
#pragma unroll
        for (int j = 0; j < GT_NJ; ++j) {
            const int t = t0 + GT_TW * wn + 16 * j + ec;
            const float sc = (tscale != nullptr && t < T) ? tscale[t] : 1.0f;
#pragma unroll
            for (int i = 0; i < NOUT; ++i) {
                const int m = m0 + (GATED ? (GT_RW / 2) * wm : GT_RW * wm) + 16 * i + er;
                if (t < T && m < M) {
                    float h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[e] = GATED ? silu(acc[i][j][e] * sc) * (acc[i + NH][j][e] * sc) : acc[i][j][e] * sc;
                    store4(Y + static_cast<int64_t>(t) * M + m, m, h);
                }
            }
        }
    }
}

// Sums the split-K partials P[s][T][Mo] in split order, scales token t's sums by
// tscale[t] (when given) and applies the epilogue (gated: h = silu(sum of gate
// partials) * (sum of up partials)).  Four outputs per thread when M % 4 == 0 (16-byte
// aligned rows), else one.  The partials of each output are loaded 8 at a time
// (independent loads in flight together) and added in split order, so the result
// does not depend on the launch.
template <bool GATED>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ P, float* __restrict__ Y,
                                                     const float* __restrict__ tscale, int64_t T, int64_t M,
                                                     int nsplit, int vec) {
    constexpr int B = 8;
    const int64_t Mo = GATED ? 2 * M : M;
    const int64_t plane = T * Mo;
    const int W = vec ? 4 : 1;
    const int64_t n = T * M / W;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t t = e * W / M, m = e * W - t * M;
        const float* p = P + t * Mo + m;
        const float sc = tscale != nullptr ? tscale[t] : 1.0f;
        if (vec) {
            float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
            int s = 0;
            for (; s + B <= nsplit; s += B) {
                float4 a[B], c[B];
#pragma unroll
                for (int i = 0; i < B; ++i) {
                    a[i] = *reinterpret_cast<const float4*>(p + (s + i) * plane);
                    if (GATED) c[i] = *reinterpret_cast<const float4*>(p + (s + i) * plane + M);
                }
#pragma unroll
                for (int i = 0; i < B; ++i) {
                    g.x += a[i].x; g.y += a[i].y; g.z += a[i].z; g.w += a[i].w;
                    if (GATED) { u.x += c[i].x; u.y += c[i].y; u.z += c[i].z; u.w += c[i].w; }
                }
            }
            for (; s < nsplit; ++s) {
                const float4 a = *reinterpret_cast<const float4*>(p + s * plane);
                g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
                if (GATED) {
                    const float4 c = *reinterpret_cast<const float4*>(p + s * plane + M);
                    u.x += c.x; u.y += c.y; u.z += c.z; u.w += c.w;
                }
            }
            g.x *= sc, g.y *= sc, g.z *= sc, g.w *= sc;
            if (GATED) {
                u.x *= sc, u.y *= sc, u.z *= sc, u.w *= sc;
                g = make_float4(silu(g.x) * u.x, silu(g.y) * u.y, silu(g.z) * u.z, silu(g.w) * u.w);
            }
            *reinterpret_cast<float4*>(Y + t * M + m) = g;
        } else {
            float g = 0.0f, u = 0.0f;
            int s = 0;
            for (; s + B <= nsplit; s += B) {
                float a[B], c[B];
#pragma unroll
                for (int i = 0; i < B; ++i) {
                    a[i] = p[(s + i) * plane];
                    if (GATED) c[i] = p[(s + i) * plane + M];
                }
#pragma unroll
                for (int i = 0; i < B; ++i) {
                    g += a[i];
                    if (GATED) u += c[i];
                }
            }
            for (; s < nsplit; ++s) {
                g += p[s * plane];
                if (GATED) u += p[s * plane + M];
            }
            Y[t * M + m] = GATED ? silu(g * sc) * (u * sc) : g * sc;
        }
    }
}

// Sums the tiled kernel's split-K partial blocks in split order and writes the outputs.
// Thread e handles float4 element e of a split's partials (the same element of every
// split's block, read 8 splits at a time), i.e. wave w, fragment (i, j), lane l of tile
// `tile`: four consecutive weight rows of token t0 + 16 j + l % 16.  Gated: fragment i <
// GT_NI / 2 holds gate sums and fragment i + GT_NI / 2 the up sums of the same outputs;
// the thread of the gate element does both.  Token t's sums are scaled by tscale[t]
// (when given) before the epilogue.  The order of the additions does not depend on the
// launch.
template <bool GATED, int BN>
__global__ __launch_bounds__(256) void splitk_reduce_tiles(const float4* __restrict__ P, float* __restrict__ Y,
                                                           const float* __restrict__ tscale, int M, int T,
                                                           int nsplit, int ntiles, int vec) {
    constexpr int B = 8;
    constexpr int NJ = BN / 16;
    constexpr int NI = GT_BM / GT_WAVES / 16;   // fragments per wave along the weight rows
    constexpr int RW = GT_BM / GT_WAVES;        // weight rows per wave
    constexpr int PER_TILE = GT_WAVES * NI * NJ * 64;
    constexpr int NOUT = GATED ? NI / 2 : NI;   // output fragments per wave
    const int rows_per_tile = GATED ? GT_BM / 2 : GT_BM;
    const int nMt = (M + rows_per_tile - 1) / rows_per_tile;
    const int64_t plane = static_cast<int64_t>(ntiles) * PER_TILE;
    const int64_t n = static_cast<int64_t>(ntiles) * GT_WAVES * NOUT * NJ * 64;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int lane = static_cast<int>(e & 63);
        int64_t q = e >> 6;
        const int j = static_cast<int>(q % NJ);
        q /= NJ;
        const int i = static_cast<int>(q % NOUT);
        q /= NOUT;
        const int wave = static_cast<int>(q % GT_WAVES);
        const int tile = static_cast<int>(q / GT_WAVES);
        // The tiled kernel's tile order: weight-row tiles in groups of GT_GROUP_M.
        const int group = tile / (GT_GROUP_M * ((T + BN - 1) / BN));
        const int first_m = group * GT_GROUP_M;
        const int gm = min(GT_GROUP_M, nMt - first_m);
        const int in_group = tile - group * GT_GROUP_M * ((T + BN - 1) / BN);
        const int mt = first_m + in_group % gm;
        const int t = (in_group / gm) * BN + 16 * j + (lane & 15);
        const int m = mt * rows_per_tile + (GATED ? RW / 2 : RW) * wave + 16 * i + 4 * (lane >> 4);
        if (t >= T || m >= M) continue;
        const int64_t idx = static_cast<int64_t>(tile) * PER_TILE + ((wave * NI + i) * NJ + j) * 64 + lane;
        const int64_t idu = idx + (NI / 2) * NJ * 64;  // gated: the up fragment i + NI / 2
        float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
        int s = 0;
        for (; s + B <= nsplit; s += B) {
            float4 a[B], c[B];
#pragma unroll
            for (int k = 0; k < B; ++k) {
                a[k] = P[(s + k) * plane + idx];
                if (GATED) c[k] = P[(s + k) * plane + idu];
            }
#pragma unroll
            for (int k = 0; k < B; ++k) {
                g.x += a[k].x; g.y += a[k].y; g.z += a[k].z; g.w += a[k].w;
                if (GATED) { u.x += c[k].x; u.y += c[k].y; u.z += c[k].z; u.w += c[k].w; }
            }
        }
        for (; s < nsplit; ++s) {
            const float4 a = P[s * plane + idx];
            g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
            if (GATED) {
                const float4 c = P[s * plane + idu];
                u.x += c.x; u.y += c.y; u.z += c.z; u.w += c.w;
            }
        }
        const float sc = tscale != nullptr ? tscale[t] : 1.0f;
        float h[4] = {g.x * sc, g.y * sc, g.z * sc, g.w * sc};
        if (GATED) {
            h[0] = silu(h[0]) * (u.x * sc);
            h[1] = silu(h[1]) * (u.y * sc);
            h[2] = silu(h[2]) * (u.z * sc);
            h[3] = silu(h[3]) * (u.w * sc);
        }
        float* yp = Y + static_cast<int64_t>(t) * M + m;
        if (vec) {
            *reinterpret_cast<float4*>(yp) = make_float4(h[0], h[1], h[2], h[3]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (m + k < M) yp[k] = h[k];
        }
    }
}

template <int FMT, bool GATED, bool SPLIT, int BN>
static void launch_tile_t(const void* W, const void* Wu, const void* X, const float* tscale, float* Y, int64_t M,
                          int64_t K, int64_t T, int nsplit, int ksteps, hipStream_t s) {
    const int64_t rows_per_tile = GATED ? GT_BM / 2 : GT_BM;
    const int64_t ntiles = ((M + rows_per_tile - 1) / rows_per_tile) * ((T + BN - 1) / BN);
    const int64_t grid = (ntiles * (SPLIT ? nsplit : 1) + 7) / 8 * 8;  // whole runs per XCD
    hipLaunchKernelGGL((gemm_tile_kernel<FMT, GATED, SPLIT, BN>), dim3(static_cast<unsigned>(grid)),
                       dim3(GT_THREADS), 0, s, static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Wu), X,
                       tscale, Y, static_cast<int>(M), static_cast<int>(K), static_cast<int>(T),
                       static_cast<int>(M % 4 == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0), nsplit, ksteps);
}

// Adds the partial blocks the split instance of the tiled kernel left in P (nsplit x
// ntiles x GT_BM x BN fp32) into Y (T x M fp32).
template <bool GATED, int BN>
static void launch_reduce_tiles_t(const float* P, float* Y, const float* tscale, int64_t M, int64_t T, int nsplit,
                                  hipStream_t s) {
    const int64_t rows_per_tile = GATED ? GT_BM / 2 : GT_BM;
    const int64_t ntiles = ((M + rows_per_tile - 1) / rows_per_tile) * ((T + BN - 1) / BN);
    const int64_t n = ntiles * GT_WAVES * (GT_BM / GT_WAVES / 16 / (GATED ? 2 : 1)) * (BN / 16) * 64;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 256 * 16));
    hipLaunchKernelGGL((splitk_reduce_tiles<GATED, BN>), dim3(grid), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(P), Y, tscale, static_cast<int>(M), static_cast<int>(T),
                       nsplit, static_cast<int>(ntiles),
                       static_cast<int>(M % 4 == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0));
}

void launch_splitk_reduce(const float* P, float* Y, const float* tscale, int64_t T, int64_t M, int nsplit, bool gated,
                          hipStream_t s) {
    const int vec = M % 4 == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
    const int64_t n = T * M / (vec ? 4 : 1);
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 256 * 16));
    if (gated) hipLaunchKernelGGL(splitk_reduce<true>, dim3(grid), dim3(256), 0, s, P, Y, tscale, T, M, nsplit, vec);
    else hipLaunchKernelGGL(splitk_reduce<false>, dim3(grid), dim3(256), 0, s, P, Y, tscale, T, M, nsplit, vec);
}

// The tiled kernel's plan for a shape: whether it applies (block formats need 16-byte
// aligned rows, K % 256 == 0; F16 K % 64 == 0; 32-bit lane offsets inside a tile need
// K <= 2^20), the tile width, and the K split.  K is split when the tiles cannot fill
// the 256 CUs: at most one wave of workgroups, at least 4 K steps (256) per split,
// split boundaries on multiples of 4 steps.  The partials take one GT_BM x BN fp32
// block per tile and split of the caller's workspace.
TilePlan plan_gemm_tile(int fmt, int64_t M, int64_t K, int64_t T, bool gated) {
    TilePlan p;
    if (fmt != 1 && K % 256 != 0) return p;
    if (K % 64 != 0 || K > (int64_t{1} << 20)) return p;
    const int64_t rows_per_tile = gated ? GT_BM / 2 : GT_BM;
    p.narrow = T <= 128;
    const int64_t bn = p.narrow ? 128 : GT_BN;
    const int64_t ntiles = ((M + rows_per_tile - 1) / rows_per_tile) * ((T + bn - 1) / bn);
    if (ntiles > (int64_t{1} << 30)) return p;
    const int64_t nsteps = K / GT_BK;
    p.nsplit = 1;
    p.ksteps = static_cast<int>(nsteps);
    if (ntiles < 192 && nsteps >= 8) {
        const int64_t want = std::min<int64_t>(256 / ntiles, nsteps / 4);
        if (want >= 2) {
            p.ksteps = static_cast<int>((nsteps + want - 1) / want + 3) / 4 * 4;
            p.nsplit = static_cast<int>((nsteps + p.ksteps - 1) / p.ksteps);
        }
    }
    // Partial blocks: GT_BM x bn accumulators per tile and split (gated tiles: 128 gate
    // and 128 up rows).  nsplit * ntiles <= 256, so at most 64 MiB.
    p.ws_bytes = p.nsplit > 1 ? static_cast<size_t>(p.nsplit) * ntiles * GT_BM * bn * sizeof(float) : 0;
    p.ok = true;
    return p;
}

void launch_gemm_tile(const TilePlan& p, int fmt, const void* W, const void* Wu, const void* X, const float* tscale,
                      float* Y, int64_t M, int64_t K, int64_t T, float* ws, hipStream_t s) {
    const bool gated = Wu != nullptr;
    const bool split = p.nsplit > 1;
    float* out = split ? ws : Y;
#define QMM_TILE_BN(F, G, SP)                                                                           \
    if (p.narrow) launch_tile_t<F, G, SP, 128>(W, Wu, X, tscale, out, M, K, T, p.nsplit, p.ksteps, s);  \
    else launch_tile_t<F, G, SP, GT_BN>(W, Wu, X, tscale, out, M, K, T, p.nsplit, p.ksteps, s);
#define QMM_TILE_CASE(F, SP)                                                                            \
    if (gated) { QMM_TILE_BN(F, true, SP) }                                                             \
    else { QMM_TILE_BN(F, false, SP) }
    if (split) {
        if (fmt == 8) { QMM_TILE_CASE(8, true) }
        else if (fmt == 2) { QMM_TILE_CASE(2, true) }
        else if (fmt == 3) { QMM_TILE_CASE(3, true) }
        else if (fmt == 6) { QMM_TILE_CASE(6, true) }
        else if (fmt == 7) { QMM_TILE_CASE(7, true) }
        else { QMM_TILE_CASE(1, true) }
        if (p.narrow) {
            if (gated) launch_reduce_tiles_t<true, 128>(ws, Y, tscale, M, T, p.nsplit, s);
            else launch_reduce_tiles_t<false, 128>(ws, Y, tscale, M, T, p.nsplit, s);
        } else {
            if (gated) launch_reduce_tiles_t<true, GT_BN>(ws, Y, tscale, M, T, p.nsplit, s);
            else launch_reduce_tiles_t<false, GT_BN>(ws, Y, tscale, M, T, p.nsplit, s);
        }
    } else {
        if (fmt == 8) { QMM_TILE_CASE(8, false) }
        else if (fmt == 2) { QMM_TILE_CASE(2, false) }
        else if (fmt == 3) { QMM_TILE_CASE(3, false) }
        else if (fmt == 6) { QMM_TILE_CASE(6, false) }
        else if (fmt == 7) { QMM_TILE_CASE(7, false) }
        else { QMM_TILE_CASE(1, false) }
    }
#undef QMM_TILE_CASE
#undef QMM_TILE_BN
}

}  // namespace qmm
