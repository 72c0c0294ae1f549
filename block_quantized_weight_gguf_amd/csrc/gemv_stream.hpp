// Streaming decode GEMV for the block formats (Q8_0, Q4_0, Q4_1, Q5_0, Q5_1), a few
// tokens per pass.
//
// Single-token decode is bound by the weight stream ("EdgeRunner Core
// Architecture", section 3.4 Tier 1 and section 15 item 2: the raw blocks are the
// only large operand), so this kernel is organised to keep HBM busy with as few
// instructions per byte as possible:
//   * One workgroup per CU (LDS-limited).  x (all K, NT tokens) is copied into LDS
//     once, as block-scaled fp16 pairs (stage_x16); after that barrier (and, for the
//     biased formats, a second one for the blocks' sums of x) the waves never
//     synchronise again.  Dot products run on v_dot2_f32_f16 with the codes as exact
//     small fp16 numbers (block_dot), fewer VALU instructions than a convert and an
//     FMA per weight.
//   * Each wave walks a list of tasks.  A task is R rows (2R row units when gated:
//     R gate rows and the same R up rows) x one K slice of 64*BPL blocks (BPL = 1
//     for Q8_0, 2 for Q4_0, so a row slice is ~2.2 KB either way).  Each row
//     slice is contiguous in HBM: it is fetched with coalesced, non-temporal
//     16-byte loads (SGPR base + lane offset), parked in the wave's private LDS
//     buffer, and re-read by each lane as "its" block at any byte offset (blocks
//     are only 2-byte aligned).
//   * All task bookkeeping (row, slice, base addresses, byte counts) is
//     wave-uniform and lives in scalar registers; the vector units only decode
//     and multiply.
//   * Software pipeline: the loads of task t+1 are issued before task t is
//     decoded, so every wave keeps a task in flight while it computes.
//   * The host keeps every 16-byte chunk the kernel reads inside the weight
//     buffer: when the matrix size is not a multiple of 16 bytes, the last row is
//     left to the sliced kernel, so this one never needs a tail path.
//   * A row group's partial sums stay in registers across its K slices and are
//     reduced across the wave once, with a transposing butterfly.
#pragma once

#include <type_traits>

#include "dma.hpp"
#include "gemv_block.hpp"
#include "qmm_internal.hpp"

namespace qmm {


template <int FMT>
struct StreamGeom {
    static constexpr int BB = Fmt<FMT>::BB;
    static constexpr int BPL = (FMT == 8) ? 1 : 2;            // blocks per lane per row slice
    static constexpr int SLICE = kWave * BPL;                  // blocks per K slice
    static constexpr int CPR = (SLICE * BB + 15) / 16 + 1;     // 16-byte chunks per row slice, incl. shift
    static constexpr int LPR = (CPR + kWave - 1) / kWave;      // loads per lane per row slice
    static constexpr int ROWBUF = (SLICE * BB + 32 + 15) / 16 * 16;  // staged bytes per row unit
    static_assert(16 * CPR <= ROWBUF, "staging geometry");
};

// Wave-level ordering of LDS writes and reads: the hardware executes one wave's
// LDS operations in order; these fences stop the compiler from reordering them.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int FMT, int NT, int R, bool GATED, int WAVES, int D, int EP>
__global__ __launch_bounds__(WAVES * 64) void gemv_stream_kernel(const uint8_t* __restrict__ Wg,
                                                                  const uint8_t* __restrict__ Wu,
                                                                  const float* __restrict__ x,
                                                                  float* __restrict__ y, int M, int K,
                                                                  int64_t ldx, int64_t ldy, int xs_bytes,
                                                                  DecodeEpi epi) {
    using G = StreamGeom<FMT>;
    constexpr int BB = G::BB, BPL = G::BPL, SLICE = G::SLICE, CPR = G::CPR, LPR = G::LPR, ROWBUF = G::ROWBUF;
    constexpr int RU = GATED ? 2 * R : R;
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t* xs = reinterpret_cast<uint32_t*>(smem);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nb = K / kQK;
    const int xstride = nb * XS16;  // dwords per token in LDS
    const int64_t rb = static_cast<int64_t>(nb) * BB;

    uint8_t* my = smem + xs_bytes + wave * (RU * ROWBUF);
    const int ns = (nb + SLICE - 1) / SLICE;
    const int ngroups = (M - 1) / R + 1;  // (no overflow for M up to 2^31 - 1)
    const int nw = gridDim.x * WAVES;
    const int wid = blockIdx.x * WAVES + wave;
    const int my_groups = wid < ngroups ? (ngroups - 1 - wid) / nw + 1 : 0;
    const int ntask = my_groups * ns;

    uint4 regs[D][RU][LPR];
    // Loads of task t: for each row unit, the chunks [0, nch) of its 16-byte aligned
    // slice.  Every lane loads on every step (chunk index clamped to nch - 1), so no
    // load is predicated: a predicated load would have to be merged with the
    // register's old value, which waits for the load and defeats the pipeline.
    // The last chunk may extend up to 15 bytes past the slice; the host guarantees
    // those bytes lie inside the weight buffer.
    auto issue = [&](int t, uint4 (&rg)[RU][LPR]) {
        const int gi = t / ns;
        const int s = t - gi * ns;
        const int g = wid + gi * nw;
        const int s0 = s * SLICE;
        const int sb = min(SLICE, nb - s0);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            // Rows past the end re-read the last row (in bounds); their sums are never stored.
            const int row = min(g * R + (u % R), M - 1);
            const uint8_t* wbase = (GATED && u >= R) ? Wu : Wg;
            const int64_t off = row * rb + static_cast<int64_t>(s0) * BB;
            const int64_t a = off & ~int64_t(15);
            const int nch = static_cast<int>((off - a) + static_cast<int64_t>(sb) * BB + 15) >> 4;
            const uint8_t* src = wbase + a;
#pragma unroll
            for (int kk = 0; kk < LPR; ++kk) {
                const uint32_t j = static_cast<uint32_t>(min(lane + kWave * kk, nch - 1));
                rg[u][kk] = load16_nt(src + 16u * j);
            }
        }
    };

    float acc[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[u][n] = 0.0f;

    // x (with gamma) is requested first and the first D tasks' weights right after
    // it: converting x then waits only for its own loads, and the weight loads stay
    // in flight while x is staged.  x -> LDS once: NT tokens x nb blocks, 8 float4
    // per block (EP_NORM: gamma .* x, with the sum of squares of x gathered on the
    // way).  Lanes 8b..8b+7 of a round hold the 8 chunks of one block (nb * 8 is a
    // multiple of 8).  SU rounds of the workgroup are loaded before any is
    // converted, so their latencies overlap (one pass covers K <= 16384 with 16 waves).
    constexpr int SU = 4;
    constexpr int XR = SU * WAVES * kWave;
    float4 xv[SU][NT], gv[SU];
    float ss[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) ss[n] = 0.0f;
    bool wide = false;
    // Loads are unconditional (index clamped; surplus lanes re-read the last chunk
    // and stage nothing): loads under a branch make the compiler wait for every
    // outstanding load, the weight DMAs included, before their use.
    auto load_round = [&](int j0) {
#pragma unroll
        for (int r = 0; r < SU; ++r) {
            const int64_t j = min(j0 + r * WAVES * kWave, nb * 8 - 1);
            if constexpr (EP == EP_NORM) gv[r] = *reinterpret_cast<const float4*>(epi.gamma + 4 * j);
#pragma unroll
            for (int n = 0; n < NT; ++n) xv[r][n] = *reinterpret_cast<const float4*>(x + n * ldx + 4 * j);
        }
    };
    auto stage_round = [&](int j0) {
#pragma unroll
        for (int r = 0; r < SU; ++r) {
            const int j = j0 + r * WAVES * kWave;
            if (j < nb * 8) {
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    float4 v = xv[r][n];
                    if constexpr (EP == EP_NORM) {
                        const float4 gm = gv[r];
                        ss[n] = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss[n]))));
                        v.x *= gm.x, v.y *= gm.y, v.z *= gm.z, v.w *= gm.w;
                    }
                    wide |= stage_x16<FMT>(v, j & 7, xs + n * xstride + (j >> 3) * XS16);
                }
            }
        }
    };
    load_round(threadIdx.x);
#pragma unroll
    for (int q = 0; q < D; ++q)
        if (q < ntask) issue(q, regs[q]);
    stage_round(threadIdx.x);
    for (int j0 = threadIdx.x + XR; j0 < nb * 8; j0 += XR) {
        load_round(j0);
        stage_round(j0);
    }
    float* red = reinterpret_cast<float*>(smem + xs_bytes + WAVES * (RU * ROWBUF));
    uint32_t* wflag = reinterpret_cast<uint32_t*>(red + WAVES * NT);
    if constexpr (EP == EP_NORM) norm_partials<NT>(ss, red, wave, lane);
    publish_wide(wide, wflag, wave, lane);
    // LDS-only barriers: a full __syncthreads would also wait for the weight loads.
    lds_barrier();
    if constexpr (DotCode<FMT>::BIAS) {
        for (int b = threadIdx.x; b < NT * nb; b += WAVES * kWave) stage_chain<FMT>(xs + b * XS16);
        lds_barrier();
    }
    float scale = 1.0f;
    if constexpr (EP == EP_NORM) scale = norm_scale<NT>(red, WAVES, reduced_token<RU, NT>(lane), K, epi.eps);
    // A wide block of x (every workgroup stages all of x, so all of them see it): x
    // again, as fp32 in the same LDS (XS_STRIDE floats per block; the host sizes x's
    // region for it whenever that costs no occupancy), and the same loop on fp32
    // products (block_fma); when fp32 x does not fit, the exact path that reads
    // everything from global memory.
    const bool wide_x = any_wide<WAVES>(wflag);
    if (wide_x) {
        if (NT * nb * XS_STRIDE * 4 > xs_bytes) {
            gemv_rows_exact<FMT, NT, R, GATED, EP>(Wg, Wu, x, y, M, K, ldx, ldy, epi, scale, wid, nw, my_groups,
                                                   lane);
            return;
        }
        float* xf = reinterpret_cast<float*>(smem);
        for (int j = threadIdx.x; j < NT * nb * 8; j += WAVES * kWave) {
            const int n = j / (nb * 8), r = j - n * (nb * 8);
            const int64_t k = 4 * static_cast<int64_t>(r);
            float4 v = *reinterpret_cast<const float4*>(x + n * ldx + k);
            if constexpr (EP == EP_NORM) {
                const float4 gm = *reinterpret_cast<const float4*>(epi.gamma + k);
                v.x *= gm.x, v.y *= gm.y, v.z *= gm.z, v.w *= gm.w;
            }
            *reinterpret_cast<float4*>(xf + n * nb * XS_STRIDE + (r >> 3) * XS_STRIDE + 4 * (r & 7)) = v;
        }
        lds_barrier();
    }

    // XF_ selects the x form (fp32 for wide x, block floating point otherwise).
    auto run = [&](auto XF_) __attribute__((always_inline)) {
    constexpr bool XF = decltype(XF_)::value;
    for (int t0 = 0; t0 < ntask; t0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
        const int t = t0 + q;
        if (t >= ntask) break;
        wave_lds_sync();  // the previous task's LDS reads are complete
#pragma unroll
        for (int u = 0; u < RU; ++u)
#pragma unroll
            for (int kk = 0; kk < LPR; ++kk) {
                const int j = lane + kWave * kk;
                if (kk < LPR - 1 || j < CPR)
                    *reinterpret_cast<uint4*>(my + u * ROWBUF + 16 * j) = regs[q][u][kk];
            }
        wave_lds_sync();
        if (t + D < ntask) issue(t + D, regs[q]);

        const int gi = t / ns;
        const int s = t - gi * ns;
        const int g = wid + gi * nw;
        const int s0 = s * SLICE;
        const int sb = min(SLICE, nb - s0);
        const uint8_t* buf[RU];
        int sh[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int row = min(g * R + (u % R), M - 1);
            buf[u] = my + u * ROWBUF;
            sh[u] = static_cast<int>((row * rb + static_cast<int64_t>(s0) * BB) & 15);
        }
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            const int blk = lane + kWave * b;
            if (blk < sb) {
                int off[RU];
#pragma unroll
                for (int u = 0; u < RU; ++u) off[u] = sh[u] + blk * BB;
                if constexpr (XF) {
                    const float* xb[NT];
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        xb[n] = reinterpret_cast<const float*>(smem) + (n * nb + s0 + blk) * XS_STRIDE;
                    block_fma<FMT, RU, NT>(buf, off, xb, acc);
                } else {
                    const uint32_t* xb[NT];
#pragma unroll
                    for (int n = 0; n < NT; ++n) xb[n] = xs + n * xstride + (s0 + blk) * XS16;
                    block_dot<FMT, RU, NT>(buf, off, xb, acc);
                }
            }
        }
        if (s == ns - 1) {
            reduce_store<R, RU, NT, GATED, EP>(acc, lane, g * R, M, y, ldy, scale, epi.res);
#pragma unroll
            for (int u = 0; u < RU; ++u)
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[u][n] = 0.0f;
        }
    }
    }
    };
    if (wide_x) run(std::true_type{});
    else run(std::false_type{});
}

// Raise a kernel's dynamic LDS limit once per (kernel, device) (gemv_stream.hip).
void allow_dynamic_lds(const void* kern, int bytes);

// Returns the number of leading rows launched (M, or M - 1 when the matrix size is
// not a multiple of 16 bytes: the final row's last 16-byte chunk would cross the
// end of the buffer, so that row is left to the caller), or 0 when this kernel
// does not apply (LDS too small for x, or a single such row).
template <int FMT, int NT, int R, bool GATED, int WAVES, int D, int EP>
static int64_t launch_t(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                        const DecodeEpi& epi, hipStream_t s) {
    const int64_t ldy = M;
    using G = StreamGeom<FMT>;
    constexpr int RU = GATED ? 2 * R : R;
    const int64_t nb = K / 32;
    const int64_t rb = nb * G::BB;
    if ((M * rb) % 16 != 0) {
        if (M < 2) return 0;
        M -= 1;  // every chunk of the first M - 1 rows ends at most 15 bytes into the last row
    }
    int64_t xs_bytes = ((NT * nb * XS16 * 4) + 15) / 16 * 16;
    const int64_t rest = static_cast<int64_t>(WAVES) * RU * G::ROWBUF + WAVES * NT * 4 + WAVES * 4;
    int64_t lds = xs_bytes + rest;
    constexpr int64_t kMaxLds = 160 * 1024;
    if (lds > kMaxLds) return 0;
    auto kern = gemv_stream_kernel<FMT, NT, R, GATED, WAVES, D, EP>;
    allow_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(kMaxLds));
    const int64_t ngroups = (M + R - 1) / R;
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(16 / WAVES, kMaxLds / lds));
    // Room for x as fp32 (the kernel's path for wide blocks of x) when it leaves as
    // many workgroups per CU.
    const int64_t xs32 = NT * nb * XS_STRIDE * 4;
    if (xs32 > xs_bytes && (xs32 + rest) * per_cu <= kMaxLds) {
        xs_bytes = xs32;
        lds = xs32 + rest;
    }
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((ngroups + WAVES - 1) / WAVES, 256 * per_cu));
    const int64_t ns = (nb + G::SLICE - 1) / G::SLICE;
    if (((ngroups + grid * WAVES - 1) / (grid * WAVES) + D) * ns >= (int64_t{1} << 31)) return 0;  // int task counts
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(WAVES * kWave), static_cast<size_t>(lds), s,
                       static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Wu), x, y, static_cast<int>(M),
                       static_cast<int>(K), K, ldy, static_cast<int>(xs_bytes), epi);
    return M;
}

// Variant choice (measured on MI355X at the Llama-3-8B and SmolLM2-135M shapes).
// Large matrices: the plain GEMV runs 16 waves per workgroup (8 for 3-4 tokens) with 2
// rows per task from 16384 rows and 1 row otherwise; the gated kernel runs 8 waves
// with 1 gate + 1 up row per task, prefetching two tasks ahead when each wave owns
// only a few tasks, so that the whole matrix is in flight at once.  Small matrices
// are bound by the kernel's own latency chain (x staged, one workgroup barrier, the
// first weight bytes, the reduction), which shrinks with the workgroup: in HIP-graph
// replay a 576 x 576 (or 960 x 576, 576 x 1536) GEMV takes 2.4 us on 4-wave
// workgroups against 3.2-3.4 us on 16 waves (or the DMA-fed kernel), 1024 x 4096 3.2
// against 3.9 us with two tasks in flight; at 2048 rows 8 waves are best (2.75 against
// 3.4 us at K = 576, 3.7 against 3.9 us at K = 4096).  The gated product likewise runs
// 4 waves up to 1024 rows (Q8_0 1024 x 4096: 4.0 against 4.9 us).
template <int FMT, int NT, int EP>
static int64_t launch_nt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                         const DecodeEpi& epi, hipStream_t s) {
    const int64_t nb = K / 32;
    const int64_t slices = (nb + StreamGeom<FMT>::SLICE - 1) / StreamGeom<FMT>::SLICE;
    if (Wu) {
        if constexpr (EP == EP_RES) {
            return 0;  // no residual on the gated product
        } else {
            const bool deep = (M * slices) / (256 * 8) <= 2;  // tasks per wave
            if (M <= kSmallRows)
                return deep ? launch_t<FMT, NT, 1, true, 4, 2, EP>(W, Wu, x, y, M, K, epi, s)
                            : launch_t<FMT, NT, 1, true, 4, 1, EP>(W, Wu, x, y, M, K, epi, s);
            // Two Q5_1 tasks in flight at 3-4 tokens need more than the 256 VGPRs of a
            // wave in an 8-wave workgroup: one task.
            if constexpr (FMT == 7 && NT >= 3) return launch_t<FMT, NT, 1, true, 8, 1, EP>(W, Wu, x, y, M, K, epi, s);
            else
                return deep ? launch_t<FMT, NT, 1, true, 8, 2, EP>(W, Wu, x, y, M, K, epi, s)
                            : launch_t<FMT, NT, 1, true, 8, 1, EP>(W, Wu, x, y, M, K, epi, s);
        }
    }
    if (M <= kSmallRows) return launch_t<FMT, NT, 1, false, 4, 2, EP>(W, Wu, x, y, M, K, epi, s);
    if (M <= 2 * kSmallRows) return launch_t<FMT, NT, 1, false, 8, 1, EP>(W, Wu, x, y, M, K, epi, s);
    // 16 waves per workgroup cap a wave at 128 VGPRs; 3-4 tokens need more, and so do
    // 2 tokens on 2-row tasks (with the exact-code decode they spilled at 16 waves).
    constexpr int PW = NT <= 2 ? 16 : 8;
    constexpr int PW2 = NT == 1 ? 16 : 8;
    if (M >= 16384) return launch_t<FMT, NT, 2, false, PW2, 1, EP>(W, Wu, x, y, M, K, epi, s);
    return launch_t<FMT, NT, 1, false, PW, 1, EP>(W, Wu, x, y, M, K, epi, s);
}

template <int FMT, int EP>
static int64_t launch_fmt_ep(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K, int NT,
                             const DecodeEpi& epi, hipStream_t s) {
    switch (NT) {
        case 1: return launch_nt<FMT, 1, EP>(W, Wu, x, y, M, K, epi, s);
        case 2: return launch_nt<FMT, 2, EP>(W, Wu, x, y, M, K, epi, s);
        case 3: return launch_nt<FMT, 3, EP>(W, Wu, x, y, M, K, epi, s);
        default: return launch_nt<FMT, 4, EP>(W, Wu, x, y, M, K, epi, s);
    }
}

// One block format's streaming GEMV (launch_gemv_stream's contract); instantiated in
// gemv_stream_<format>.hip.
template <int FMT>
int64_t gemv_stream_fmt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K, int NT,
                        int ep, const DecodeEpi& epi, hipStream_t s) {
    switch (ep) {
        case EP_NORM: return launch_fmt_ep<FMT, EP_NORM>(W, Wu, x, y, M, K, NT, epi, s);
        case EP_RES: return launch_fmt_ep<FMT, EP_RES>(W, Wu, x, y, M, K, NT, epi, s);
        default: return launch_fmt_ep<FMT, EP_NONE>(W, Wu, x, y, M, K, NT, epi, s);
    }
}

extern template int64_t gemv_stream_fmt<8>(const void*, const void*, const float*, float*, int64_t, int64_t, int,
                                           int, const DecodeEpi&, hipStream_t);
extern template int64_t gemv_stream_fmt<2>(const void*, const void*, const float*, float*, int64_t, int64_t, int,
                                           int, const DecodeEpi&, hipStream_t);
extern template int64_t gemv_stream_fmt<3>(const void*, const void*, const float*, float*, int64_t, int64_t, int,
                                           int, const DecodeEpi&, hipStream_t);
extern template int64_t gemv_stream_fmt<6>(const void*, const void*, const float*, float*, int64_t, int64_t, int,
                                           int, const DecodeEpi&, hipStream_t);
extern template int64_t gemv_stream_fmt<7>(const void*, const void*, const float*, float*, int64_t, int64_t, int,
                                           int, const DecodeEpi&, hipStream_t);

}  // namespace qmm
