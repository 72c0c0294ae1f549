// Host-side launch entry points of the qmm kernels (internal; the public C ABI
// in include/qmm.h validates arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stddef.h>

#include <algorithm>

namespace qmm {

// Fused steps around the decode GEMV ("EdgeRunner Core Architecture", section 9.2:
// the attention and FFN norms are folded into the QKV and gate+up GEMVs, the
// final norm into the LM head, and the O and down GEMVs add into the residual).
//   EP_NORM: y = s * (W (gamma .* x)), s = 1 / sqrt(mean_k x_k^2 + eps) per token
//            (RMSNorm, section 6).  gamma .* x is formed while x is staged in LDS;
//            the sum of squares is gathered on the same pass and s scales the
//            reduced dot products.
//   EP_RES:  y = W x + res, res laid out like y (it may be y itself: each element
//            is read and then written by the same lane).
enum : int { EP_NONE = 0, EP_NORM = 1, EP_RES = 2 };

struct DecodeEpi {
    const float* gamma = nullptr;  // EP_NORM: K norm weights
    float eps = 0.0f;
    const float* res = nullptr;    // EP_RES: residual input
};

hipError_t launch_dequant(int fmt, const void* W, float* out, int64_t M, int64_t K, hipStream_t s);

// out[i][k] = W[ids[i]][k] (fp32) for i < n; ids outside [0, M) give NaN rows.
hipError_t launch_get_rows(int fmt, const void* W, const int32_t* ids, float* out, int64_t M, int64_t K, int64_t n,
                           hipStream_t s);

// out[m][k] = fp16(W[m][k]), rounded to nearest even.
hipError_t launch_expand_f16(int fmt, const void* W, void* out, int64_t M, int64_t K, hipStream_t s);

// VALU GEMV over N tokens (any N >= 1): y[n][m] = sum_k W[m][k] x[n][k].
// Wu != nullptr selects the gate/up SwiGLU epilogue (W = gate, Wu = up, y = h).
// ep (EP_*) adds the norm prologue or the residual epilogue (not with Wu) from epi.
hipError_t launch_gemv_valu(int fmt, const void* W, const void* Wu, const float* x, float* y,
                            int64_t M, int64_t K, int64_t N, hipStream_t s, int ep = EP_NONE,
                            const DecodeEpi& epi = DecodeEpi{});

// Row counts up to which a GEMV counts as small: its time is the kernel's latency chain,
// and it runs on the register-staged streaming kernel with small workgroups (up to 2 x
// this many rows) instead of the DMA-fed one.
constexpr int64_t kSmallRows = 1024;

// Streaming GEMV for the block formats with NT <= 4 tokens in one pass.  Returns the
// number of leading rows it launched (M or M - 1); 0 means nothing was launched
// (format or LDS footprint of x does not fit).
int64_t launch_gemv_stream(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                           int NT, int ep, const DecodeEpi& epi, hipStream_t s);

// DMA-fed streaming GEMV for the block formats with K % 256 == 0 and NT <= 4 tokens in
// one pass.  Returns M when it launched, 0 when it does not apply (format, K, LDS
// footprint of x, or EP_RES with more row groups per wave than it reads ahead).
int64_t launch_gemv_dma(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                        int NT, int ep, const DecodeEpi& epi, hipStream_t s);

// Sliced GEMV for rows [row_begin, M), NT <= 4 tokens per pass, `chunks` passes
// of NT tokens (grid.y).  Handles every format and every size.
void launch_gemv_sliced(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                        int NT, int64_t chunks, int64_t row_begin, int ep, const DecodeEpi& epi, hipStream_t s);

// fp32 tokens -> fp16 for the MFMA products: per token t the power of two 2^s_t that
// brings max_k |x[t][k]| into [2^14, 2^15) (2^126 for an all-zero token),
// x16[t][k] = fp16(2^s_t x[t][k]) (round to nearest even) and inv[t] = 2^-s_t, which
// the products' epilogues multiply back.  x, x16 16-byte aligned; K % 32 == 0.
hipError_t launch_scale_tokens(const float* x, void* x16, float* inv, int64_t N, int64_t K, hipStream_t s);

// fp16-MFMA GEMM: Y[t][m] = tscale[t] * sum_k W[m][k] X[t][k] with X fp16 (tscale ==
// nullptr: no scale).  Wu != nullptr selects the SwiGLU epilogue.  ws: the split-K
// partials of the tiled kernel's plan (gemm_workspace_bytes), nullptr when it needs none.
hipError_t launch_gemm_mfma(int fmt, const void* W, const void* Wu, const void* X, const float* tscale, float* Y,
                            int64_t M, int64_t K, int64_t T, float* ws, hipStream_t s);

// Workspace bytes launch_gemm_mfma needs for a shape (0: none).
size_t gemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t T, bool gated);

// Plan of the tiled fp16-MFMA GEMM (256 x 256 tiles, coalesced raw loads, fp16-domain
// decode): ok is false for shapes it does not cover (block formats with K % 256 != 0).
struct TilePlan {
    bool ok = false;
    bool narrow = false;    // 128-token tiles (T <= 128)
    int nsplit = 1, ksteps = 0;
    size_t ws_bytes = 0;    // split-K partials
};
TilePlan plan_gemm_tile(int fmt, int64_t M, int64_t K, int64_t T, bool gated);
void launch_gemm_tile(const TilePlan& p, int fmt, const void* W, const void* Wu, const void* X, const float* tscale,
                      float* Y, int64_t M, int64_t K, int64_t T, float* ws, hipStream_t s);

// Plan of the weight-streaming fp16-MFMA GEMV for 2..32 tokens (block formats,
// K % 256 == 0, K <= 2^20): each weight byte is read once per call.
struct GemvMfmaPlan {
    bool ok = false;
    int nj = 1;             // 16-token column fragments
    int nsplit = 1, kst = 0;
    size_t ws_bytes = 0;    // split-K partials
};
GemvMfmaPlan plan_gemv_mfma(int fmt, int64_t M, int64_t K, int64_t N, bool gated);
// y[n][m] = sum_k W[m][k] x[n][k] (x fp32, turned into scaled fp16 inside the kernel).
void launch_gemv_mfma(const GemvMfmaPlan& p, int fmt, const void* W, const void* Wu, const float* x, float* y,
                      int64_t M, int64_t K, int64_t N, float* ws, hipStream_t s);

// Y[t][m] = tscale[t] (1 when nullptr) * sum over s < nsplit of P[s][t][m] (gated: P holds gate sums in
// columns 0..M-1 and up sums in M..2M-1 of each 2M-wide row, and Y = silu(gate) * up).
void launch_splitk_reduce(const float* P, float* Y, const float* tscale, int64_t T, int64_t M, int nsplit, bool gated,
                          hipStream_t s);

}  // namespace qmm
