// DMA-fed streaming decode GEMV for the block formats (Q8_0, Q4_0, Q4_1, Q5_0, Q5_1)
// with 16-byte aligned rows (K % 256 == 0), a few tokens per pass.
//
// Single-token decode is bound by the weight stream ("EdgeRunner Core
// Architecture", section 3.4 Tier 1 and section 15 item 2: the raw blocks are the
// only large operand).  Keeping HBM busy takes tens of KB of reads in flight per
// CU.  Here the weights never pass through VGPRs: each wave owns a private ring of
// S LDS slots, and every task's raw bytes go straight from HBM into a slot by
// buffer->LDS DMA, S - 1 tasks ahead of the one being computed.
//   * One workgroup per CU (LDS-limited).  x (all K, NT tokens) is staged into LDS
//     once as block-scaled fp16 pairs, as in the register-staged streaming kernel;
//     after that the waves never synchronise again.
//   * A task is R rows (2R row units when gated: R gate rows and the same R up
//     rows) x one K slice of 64 * BPL blocks (BPL = 1 for Q8_0, 2 for the nibble
//     formats: Q8_0 2176, Q4_0 2304, Q4_1 2560, Q5_0 2816, Q5_1 3072 bytes, all
//     whole 16-byte chunks because rows are 16-byte aligned).  A row unit's slice
//     moves with three wave-wide DMA instructions (Q8_0, Q4_0: two of 16 bytes per
//     lane and one of 4 bytes per lane, 2304 bytes; the others: three of 16 bytes
//     per lane, 3072 bytes).  Each uses a
//     buffer resource that covers exactly that slice, so lanes past its end (and
//     tasks past the end of the list, and rows past M) read zeros without touching
//     memory; every task therefore issues the same number of DMA instructions and
//     the waits are compile-time constants.
//   * The ring slots are separate LDS arrays and the loop is unrolled over them,
//     so the compiler can tell the slot being read from the DMA still in flight
//     into the others.
//   * Lane l decodes block l (and l + 64) of the slice for every row unit with the
//     packed fp16 dot products of block_dot; partial sums stay in registers across
//     a row group's slices and are reduced across the wave once.
#include <type_traits>

#include "gemv_block.hpp"
#include "dma.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int DG_NI = 3;       // DMA instructions per row unit and task
constexpr int DG_PAD = 16;     // slack after each slot array (block reads may touch 4 bytes past a slice)
constexpr int DG_GMAX = 4;     // EP_RES: row groups per wave whose residuals are read before the loop

template <int FMT>
struct DmaGeom {
    static constexpr int BB = Fmt<FMT>::BB;
    static constexpr int BPL = (FMT == 8) ? 1 : 2;  // blocks per lane per row slice
    static constexpr int SLICE = kWave * BPL;       // blocks per K slice
    // Bytes per row unit and slot; the third DMA instruction moves 4 bytes per lane
    // (Q8_0, Q4_0: 2 x 1024 + 256) or 16 (the others: 3 x 1024).
    static constexpr bool WIDE = SLICE * BB > 2304;
    static constexpr int SLOT = WIDE ? 3072 : 2304;
    static_assert(SLICE * BB <= SLOT, "slice must fit a slot");
    static_assert((8 * BB) % 16 == 0, "8-block multiples are whole 16-byte chunks");
};

// LDS of one instance: S ring stages of WAVES * RU slots, the norm partials, the
// per-wave wide-block flags, and XCAP bytes left for x (NT tokens x K / 32 blocks x
// XS16 dwords).
template <int FMT, int NT, int RU, int WAVES, int S>
struct DmaLds {
    static constexpr int kMax = 160 * 1024;
    static constexpr int STAGE = WAVES * RU * DmaGeom<FMT>::SLOT + DG_PAD;
    static constexpr int RING = 2 * STAGE + (S > 2 ? STAGE : 16) + (S > 3 ? STAGE : 16);
    static constexpr int XCAP = (kMax - RING - WAVES * NT * 4 - WAVES * 4) / 16 * 16;
    static_assert(XCAP >= 16 * XS16 * 4, "room for x");
};

// Cursor over a wave's task list: task (gi, s) is slice s of the wave's gi-th row group.
struct TaskCursor {
    int gi, s;
    __device__ __forceinline__ void next(int ns) {
        if (++s == ns) {
            s = 0;
            ++gi;
        }
    }
};

// Reduce the RU x NT per-lane sums of a wave and store them (reduce_store's
// transposing reduction); `resv` is the residual of the element this lane stores
// (EP_RES), read before the loop.
template <int R, int RU, int NT, bool GATED, int EP>
__device__ __forceinline__ void dma_reduce_store(float (&acc)[RU][NT], int lane, int row0, int M, float* y,
                                                 int64_t ldy, float scale, float resv) {
    constexpr int NTP = (NT == 3) ? 4 : NT;
    constexpr int V = RU * NTP;
    float v[V];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NTP; ++n) v[u * NTP + n] = (n < NT) ? acc[u][n < NT ? n : 0] : 0.0f;
    wave_reduce_transpose<V>(v, lane);
    constexpr int LPI = kWave / V;
    const int idx = lane / LPI;
    const bool holder = (lane % LPI) == 0;
    const int u = idx / NTP;
    const int n = idx - u * NTP;
    const int r = row0 + u;
    if constexpr (!GATED) {
        if (holder && n < NT && r < M) {
            float val = v[0];
            if constexpr (EP == EP_NORM) val *= scale;
            if constexpr (EP == EP_RES) val += resv;
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

template <int FMT, int NT, int R, bool GATED, int WAVES, int S, int EP>
__global__ __launch_bounds__(WAVES * 64) void gemv_dma_kernel(const uint8_t* __restrict__ Wg,
                                                               const uint8_t* __restrict__ Wu,
                                                               const float* __restrict__ x, float* __restrict__ y,
                                                               int M, int K, int64_t ldx, int64_t ldy, DecodeEpi epi) {
    static_assert(S >= 2 && S <= 4, "ring depth");
    using G = DmaGeom<FMT>;
    constexpr int BB = G::BB, BPL = G::BPL, SLICE = G::SLICE, SLOT = G::SLOT;
    constexpr int RU = GATED ? 2 * R : R;
    constexpr int NI = RU * DG_NI;         // DMA instructions per task
    constexpr int WS = WAVES * RU * SLOT;  // bytes of one ring stage (all waves)
    // Q8_0 / Q4_0 blocks (34 / 18 bytes) sit at 2 mod 4 in a slot for even block
    // indices (slices start at even blocks, slots on 16 bytes): their codes are read
    // in the rotated order and x is staged to match (block_dot, stage_block).
    constexpr bool ROT = FMT == 8 || FMT == 2;
    __shared__ __align__(16) uint8_t RS0[WS + DG_PAD];
    __shared__ __align__(16) uint8_t RS1[WS + DG_PAD];
    __shared__ __align__(16) uint8_t RS2[S > 2 ? WS + DG_PAD : 16];
    __shared__ __align__(16) uint8_t RS3[S > 3 ? WS + DG_PAD : 16];
    // x and the norm partials take the rest of the CU's LDS, also as static arrays:
    // the compiler treats dynamic LDS as possibly written by any DMA in flight and
    // would wait for all of them before every read of x.
    using L = DmaLds<FMT, NT, RU, WAVES, S>;
    __shared__ __align__(16) uint32_t xs[L::XCAP / 4];
    __shared__ float red[WAVES * NT];
    __shared__ uint32_t wflag[WAVES];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nb = K / kQK;
    const int xstride = nb * XS16;
    const int64_t rb = static_cast<int64_t>(nb) * BB;
    const int ns = (nb + SLICE - 1) / SLICE;
    const int ngroups = (M - 1) / R + 1;  // (no overflow for M up to 2^31 - 1)
    const int nw = gridDim.x * WAVES;
    const int wid = blockIdx.x * WAVES + wave;
    const int my_groups = wid < ngroups ? (ngroups - 1 - wid) / nw + 1 : 0;
    const int ntask = my_groups * ns;  // the host keeps this below 2^31
    const int wslot = wave * RU * SLOT;  // this wave's part of a stage

    // DMA of the task at cursor c into stage array `stage`; tasks past the list read zeros.
    const uint32_t v16 = 16u * static_cast<uint32_t>(lane);
    const uint32_t v4 = 4u * static_cast<uint32_t>(lane) + 2048u;
    auto issue = [&](uint8_t* stage, const TaskCursor& c) {
        const bool real = c.gi < my_groups;
        const int64_t g = wid + static_cast<int64_t>(c.gi) * nw;  // past the list for the trailing dummies
        const int s0 = c.s * SLICE;
        const int sbytes = real ? min(SLICE, nb - s0) * BB : 0;
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int64_t row = g * R + (u % R);
            const bool ok = real && row < M;
            const uint8_t* wb = (GATED && u >= R) ? Wu : Wg;
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(wb + (ok ? row * rb + static_cast<int64_t>(s0) * BB : 0), ok ? sbytes : 0);
            QMM_L3 uint8_t* d = (QMM_L3 uint8_t*)(stage + wslot + u * SLOT);
            dma16<kCacheNT>(r, v16, 0, d);
            dma16<kCacheNT>(r, v16 + 1024u, 0, d + 1024);
            if constexpr (G::WIDE) dma16<kCacheNT>(r, v16 + 2048u, 0, d + 2048);
            else dma4<kCacheNT>(r, v4, d + 2048);
        }
    };

    float acc[RU][NT];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[u][n] = 0.0f;

    // x (with gamma, and the residuals) is requested first and the first S tasks'
    // weights right after it: converting x then waits only for its own loads, and the
    // weight DMAs stay in flight while x is staged.  x -> LDS once, one lane per
    // (token, 32-value block): the lane loads the block's 8 float4 (EP_NORM: times
    // gamma, with the sum of squares of x gathered on the way) and stages it
    // (stage_block), noting whether the block is wide.  Only the first round's loads
    // precede the DMAs.
    constexpr int XT = WAVES * kWave;  // blocks per round
    const int nxb = NT * nb;           // blocks to stage
    float4 xv[8], gv[8];
    float ss[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) ss[n] = 0.0f;
    bool wide = false;
    // Loads are unconditional (index clamped; surplus lanes re-read the last block
    // and stage nothing): loads under a branch make the compiler wait for every
    // outstanding load, the weight DMAs included, before their use.
    auto load_round = [&](int j0) {
        const int j = min(j0, nxb - 1);
        const int n = j / nb, b = j - (j / nb) * nb;
        const float4* src = reinterpret_cast<const float4*>(x + n * ldx + 32 * static_cast<int64_t>(b));
#pragma unroll
        for (int c = 0; c < 8; ++c) xv[c] = src[c];
        if constexpr (EP == EP_NORM) {
            const float4* gsrc = reinterpret_cast<const float4*>(epi.gamma + 32 * static_cast<int64_t>(b));
#pragma unroll
            for (int c = 0; c < 8; ++c) gv[c] = gsrc[c];
        }
    };
    auto stage_round = [&](int j0) {
        if (j0 < nxb) {
            const int n = j0 / nb, b = j0 - (j0 / nb) * nb;
            if constexpr (EP == EP_NORM) {
                float q = 0.0f;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    float4& t = xv[c];
                    q = fmaf(t.x, t.x, fmaf(t.y, t.y, fmaf(t.z, t.z, fmaf(t.w, t.w, q))));
                    t.x *= gv[c].x, t.y *= gv[c].y, t.z *= gv[c].z, t.w *= gv[c].w;
                }
#pragma unroll
                for (int k = 0; k < NT; ++k) ss[k] += (k == n) ? q : 0.0f;
            }
            wide |= stage_block<FMT>(xv, xs + n * xstride + b * XS16, ROT && (b & 1) == 0);
        }
    };
    load_round(threadIdx.x);

    // EP_RES: the residuals of this lane's output in the wave's first row groups.
    constexpr int NTP = (NT == 3) ? 4 : NT;
    constexpr int LPI = kWave / (RU * NTP);
    // res0 belongs to the current row group; the values move down one place per
    // group (registers only: a value selected by the group number is turned into an
    // indexed table in scratch memory, whose reads would wait for the weight DMAs).
    float res0 = 0.0f, res1 = 0.0f, res2 = 0.0f, res3 = 0.0f;
    static_assert(DG_GMAX == 4, "four read-ahead residuals");
    if constexpr (EP == EP_RES) {
        const int idx = lane / LPI;
        const int u = idx / NTP, n = idx - (idx / NTP) * NTP;
        auto res_at = [&](int gi) -> float {
            const int r = (wid + gi * nw) * R + u;
            const bool ok = gi < my_groups && lane % LPI == 0 && n < NT && r < M;
            const float v = epi.res[ok ? n * ldy + r : 0];  // unconditional load (see load_round)
            return ok ? v : 0.0f;
        };
        res0 = res_at(0);
        res1 = res_at(1);
        res2 = res_at(2);
        res3 = res_at(3);
    }

    TaskCursor ic{0, 0};
    issue(RS0, ic);
    ic.next(ns);
    issue(RS1, ic);
    ic.next(ns);
    if constexpr (S > 2) {
        issue(RS2, ic);
        ic.next(ns);
    }
    if constexpr (S > 3) {
        issue(RS3, ic);
        ic.next(ns);
    }

    stage_round(threadIdx.x);
    for (int j0 = threadIdx.x + XT; j0 < nxb; j0 += XT) {  // more blocks than lanes only
        load_round(j0);
        stage_round(j0);
    }
    if constexpr (EP == EP_NORM) norm_partials<NT>(ss, red, wave, lane);
    publish_wide(wide, wflag, wave, lane);
    // LDS-only barrier: a full __syncthreads would also wait for the weight DMAs.
    lds_barrier();
    float scale = 1.0f;
    if constexpr (EP == EP_NORM) scale = norm_scale<NT>(red, WAVES, reduced_token<RU, NT>(lane), K, epi.eps);
    // A wide block of x (every workgroup stages all of x, so all of them see it): x
    // again, as fp32 in the same LDS (XS_STRIDE floats per block), and the same loop
    // on fp32 products (block_fma); when fp32 x does not fit, the exact path that reads
    // everything from global memory.
    const bool wide_x = any_wide<WAVES>(wflag);
    if (wide_x) {
        if (NT * nb * XS_STRIDE * 4 > L::XCAP) {
            wait_vm<0>();  // the ring's DMAs land before the workgroup can exit
            gemv_rows_exact<FMT, NT, R, GATED, EP>(Wg, Wu, x, y, M, K, ldx, ldy, epi, scale, wid, nw, my_groups,
                                                   lane);
            return;
        }
        float* xf = reinterpret_cast<float*>(xs);
        if (nxb <= XT) {
            // One staging round: each lane still holds its block in xv (times gamma
            // under EP_NORM), so x is not read again.
            if (static_cast<int>(threadIdx.x) < nxb) {
                const int j = threadIdx.x;
                const int n = j / nb, b = j - (j / nb) * nb;
                float* dst = xf + (n * nb + b) * XS_STRIDE;
#pragma unroll
                for (int c = 0; c < 8; ++c) *reinterpret_cast<float4*>(dst + 4 * c) = xv[c];
            }
        } else {
            for (int j = threadIdx.x; j < NT * nb * 8; j += XT) {
                const int n = j / (nb * 8), r = j - n * (nb * 8);
                const int64_t k = 4 * static_cast<int64_t>(r);
                float4 v = *reinterpret_cast<const float4*>(x + n * ldx + k);
                if constexpr (EP == EP_NORM) {
                    const float4 gm = *reinterpret_cast<const float4*>(epi.gamma + k);
                    v.x *= gm.x, v.y *= gm.y, v.z *= gm.z, v.w *= gm.w;
                }
                *reinterpret_cast<float4*>(xf + n * nb * XS_STRIDE + (r >> 3) * XS_STRIDE + 4 * (r & 7)) = v;
            }
        }
        lds_barrier();
    }

    // One task from stage array `stage`, then its refill with the task S ahead; XF_
    // selects the x form (fp32 for wide x, block floating point otherwise).
    TaskCursor cc{0, 0};
    auto step = [&](uint8_t* stage, auto XF_) __attribute__((always_inline)) {
        constexpr bool XF = decltype(XF_)::value;
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<(S - 1) * NI>();  // this task's DMA has landed; the next S - 1 stay in flight
        __builtin_amdgcn_sched_barrier(0);
        if (cc.gi < my_groups) {
            const int s0 = cc.s * SLICE;
            const int sb = min(SLICE, nb - s0);
            const uint8_t* buf[RU];
#pragma unroll
            for (int u = 0; u < RU; ++u) buf[u] = stage + wslot + u * SLOT;
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
                const int blk = lane + kWave * b;
                if (blk < sb) {
                    int off[RU];
#pragma unroll
                    for (int u = 0; u < RU; ++u) off[u] = blk * BB;
                    if constexpr (XF) {
                        const float* xb[NT];
#pragma unroll
                        for (int n = 0; n < NT; ++n)
                            xb[n] = reinterpret_cast<const float*>(xs) + (n * nb + s0 + blk) * XS_STRIDE;
                        block_fma<FMT, RU, NT>(buf, off, xb, acc);
                    } else {
                        const uint32_t* xb[NT];
#pragma unroll
                        for (int n = 0; n < NT; ++n) xb[n] = xs + n * xstride + (s0 + blk) * XS16;
                        block_dot<FMT, RU, NT, ROT>(buf, off, xb, acc);
                    }
                }
            }
            if (cc.s == ns - 1) {
                dma_reduce_store<R, RU, NT, GATED, EP>(acc, lane, (wid + cc.gi * nw) * R, M, y, ldy, scale, res0);
                if constexpr (EP == EP_RES) {
                    res0 = res1;
                    res1 = res2;
                    res2 = res3;
                }
#pragma unroll
                for (int u = 0; u < RU; ++u)
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[u][n] = 0.0f;
            }
        }
        // The slot's LDS reads are complete before the DMA that overwrites it goes out.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        issue(stage, ic);
        ic.next(ns);
        cc.next(ns);
    };
    auto run = [&](auto XF_) __attribute__((always_inline)) {
        for (int t0 = 0; t0 < ntask; t0 += S) {
            step(RS0, XF_);
            step(RS1, XF_);
            if constexpr (S > 2) step(RS2, XF_);
            if constexpr (S > 3) step(RS3, XF_);
        }
    };
    if (wide_x) run(std::true_type{});
    else run(std::false_type{});
    // Drain the trailing DMAs (zero-length reads) before the workgroup can exit.
    wait_vm<0>();
}

template <int FMT, int NT, int R, bool GATED, int WAVES, int S, int EP>
static int64_t dma_launch(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                          const DecodeEpi& epi, hipStream_t s) {
    constexpr int RU = GATED ? 2 * R : R;
    const int64_t nb = K / 32;
    if (NT * nb * XS16 * 4 > DmaLds<FMT, NT, RU, WAVES, S>::XCAP) return 0;
    const int64_t ngroups = (M + R - 1) / R;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((ngroups + WAVES - 1) / WAVES, 256));
    const int64_t ns = (nb + DmaGeom<FMT>::SLICE - 1) / DmaGeom<FMT>::SLICE;
    if (((ngroups + grid * WAVES - 1) / (grid * WAVES) + S) * ns >= (int64_t{1} << 31)) return 0;  // int task counts
    if (EP == EP_RES) {
        const int64_t nw = grid * WAVES;
        if ((ngroups + nw - 1) / nw > DG_GMAX) return 0;
    }
    hipLaunchKernelGGL((gemv_dma_kernel<FMT, NT, R, GATED, WAVES, S, EP>), dim3(static_cast<unsigned>(grid)),
                       dim3(WAVES * kWave), 0, s, static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Wu), x,
                       y, static_cast<int>(M), static_cast<int>(K), K, M, epi);
    return M;
}

// Variant choice (durations on MI355X, weights streamed from HBM, the 8B shapes).
// Q8_0: 8 waves with a 3-slot ring and 1-row tasks is best or within noise at every
// size at K = 4096 (at 570 MB within 1% of the same kernel with the decode removed,
// i.e. of the stream itself).  The nibble formats decode more per byte (Q5_x about
// twice Q4_0), and there 2-row tasks (x read from LDS once per two rows) with a
// 2-slot ring win whenever they spread the rows as evenly over the 2048 waves of a
// full grid as 1-row tasks do: e.g. Q4_1 / Q5_0 / Q5_1 / Q4_0 at 4096 x 14336 10.3 /
// 12.4 / 12.8 / 10.2 us against 11.3 / 13.1 / 13.5 / 11.2 us, and the 128256-row LM
// head 52.8 / 63.9 / 66.2 / 50.2 against 58.3 / 68.8 / 70.6 / 57.0 us; at 6144 rows
// (3 rows per wave against 4) 1-row tasks stay ahead (Q4_1 6.5 against 6.9 us).
// With the exact-code decode the nibble formats' single-token LM heads (128256 rows,
// 21 two-row groups per wave) gain from a third wave per SIMD: 12-wave workgroups take
// Q4_0 / Q4_1 / Q5_0 / Q5_1 58.6 / 63.0 / 75.4 / 82.4 us against 62.7 / 65.9 / 79.2 /
// 86.4 us with 8 (same process), while at 4096 rows (fewer groups than waves) they
// lose 10-20%; so 12 waves from 49152 rows.  With 2-4 tokens the third wave still pays
// for Q4_0 (LM head, two passes each: 72.6-76.0 / 82.3 / 88.8-91.1 us against 80.0-84.0
// / 84.1-86.9 / 92.4-93.5 us with 8 waves at 2 / 3 / 4 tokens) and is within noise for
// the 20- to 24-byte formats (Q4_1 at 3 tokens 92-93 against 89-90 us), which keep 8.
// Q8_0 with 2-4 tokens is no longer bound by the stream alone, and on the LM head
// 2-row tasks on 12 waves win too: 93.7-97.4 / 99.5-101.7 / 107 us against 107-112 /
// 108.6-111.8 / 120-121.6 us for 1-row tasks on 8 waves (1-row tasks on 12 waves:
// 103.6-104.3 / 109.4-110.6 / 117.7-118.8).
// The gated product (gate and up rows in every task) at 2 x 14336 x 4096 (HIP-graph
// replays, weights rotated through 512 MB, two passes each): Q8_0 runs here with
// 1-row tasks, 8 waves and a 3-slot ring for 1-4 tokens (23.8 / 25.0-25.4 / 27.3-27.9 /
// 30.0-30.4 us against 25.0-25.3 / 26.0 / 33.0 / 34.2-34.5 us on the register-staged
// kernel), and Q4_0 from 2 tokens (21.8 / 24.7-25.0 / 26.7-27.2 against 24.6-25.6 /
// 25.2-26.0 / 29.9-30.3 us); the single-token Q4_0 product stays there (16.8 against
// 18.3 us here; 12- or 16-wave and 2-row gated instances were slower still), as do
// the 20- to 24-byte formats, whose gated rings leave no room for x (Q4_1 at one token
// 18.8-18.9 against 20.1-20.2 us here).
template <int FMT, int NT, int EP>
static int64_t dma_nt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                      const DecodeEpi& epi, hipStream_t s) {
    if (Wu) {
        if constexpr (FMT == 8 || (FMT == 2 && NT >= 2))
            return dma_launch<FMT, NT, 1, true, 8, 3, EP>(W, Wu, x, y, M, K, epi, s);
        return 0;
    }
    int64_t r = 0;
    if constexpr (FMT != 8) {
        constexpr int64_t kWaves = 256 * 8;
        const int64_t rows1 = (M + kWaves - 1) / kWaves;              // rows per wave, 1-row tasks
        const int64_t rows2 = 2 * ((M + 2 * kWaves - 1) / (2 * kWaves));  // and 2-row tasks
        if (20 * rows2 <= 21 * rows1) {
            if constexpr (NT == 1 || FMT == 2)
                if (M >= 49152) r = dma_launch<FMT, NT, 2, false, 12, 2, EP>(W, Wu, x, y, M, K, epi, s);
            if (!r) r = dma_launch<FMT, NT, 2, false, 8, 2, EP>(W, Wu, x, y, M, K, epi, s);
        }
    }
    if constexpr (FMT == 8 && NT >= 2)
        if (M >= 49152) r = dma_launch<FMT, NT, 2, false, 12, 2, EP>(W, Wu, x, y, M, K, epi, s);
    if (!r) r = dma_launch<FMT, NT, 1, false, 8, 3, EP>(W, Wu, x, y, M, K, epi, s);
    return r;
}

template <int FMT, int EP>
static int64_t dma_fmt_ep(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K, int NT,
                          const DecodeEpi& epi, hipStream_t s) {
    switch (NT) {
        case 1: return dma_nt<FMT, 1, EP>(W, Wu, x, y, M, K, epi, s);
        case 2: return dma_nt<FMT, 2, EP>(W, Wu, x, y, M, K, epi, s);
        case 3: return dma_nt<FMT, 3, EP>(W, Wu, x, y, M, K, epi, s);
        default: return dma_nt<FMT, 4, EP>(W, Wu, x, y, M, K, epi, s);
    }
}

template <int FMT>
static int64_t dma_fmt(const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K, int NT, int ep,
                       const DecodeEpi& epi, hipStream_t s) {
    switch (ep) {
        case EP_NORM: return dma_fmt_ep<FMT, EP_NORM>(W, Wu, x, y, M, K, NT, epi, s);
        case EP_RES: return dma_fmt_ep<FMT, EP_RES>(W, Wu, x, y, M, K, NT, epi, s);
        default: return dma_fmt_ep<FMT, EP_NONE>(W, Wu, x, y, M, K, NT, epi, s);
    }
}

int64_t launch_gemv_dma(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                        int NT, int ep, const DecodeEpi& epi, hipStream_t s) {
    if (K % 256 != 0 || NT < 1 || NT > 4) return 0;
    switch (fmt) {
        case 8: return dma_fmt<8>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 2: return dma_fmt<2>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 3: return dma_fmt<3>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 6: return dma_fmt<6>(W, Wu, x, y, M, K, NT, ep, epi, s);
        case 7: return dma_fmt<7>(W, Wu, x, y, M, K, NT, ep, epi, s);
        default: return 0;
    }
}

}  // namespace qmm
