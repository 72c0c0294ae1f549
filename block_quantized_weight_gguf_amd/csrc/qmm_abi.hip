// C ABI of the qmm library: host-side argument validation and variant dispatch.
// Every check runs before any HIP call, so an invalid call enqueues nothing.
// Size arithmetic is overflow-checked ("alpaca.swift", Highlights: untrusted
// lengths are bounded and all size arithmetic is checked).
#include <math.h>
#include <stdint.h>

#include "../../include/qmm.h"
#include "qmm_internal.hpp"

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFFLL;

bool fmt_ok(int fmt) {
    return fmt == QMM_F16 || fmt == QMM_Q4_0 || fmt == QMM_Q4_1 || fmt == QMM_Q5_0 || fmt == QMM_Q5_1 ||
           fmt == QMM_Q8_0;
}


bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    // a, b >= 0
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t row_bytes_unchecked(int fmt, int64_t K) {
    switch (fmt) {
        case QMM_F16: return 2 * K;
        case QMM_Q8_0: return (K / 32) * 34;
        case QMM_Q4_1: return (K / 32) * 20;
        case QMM_Q5_0: return (K / 32) * 22;
        case QMM_Q5_1: return (K / 32) * 24;
        default: return (K / 32) * 18;
    }
}

// Shape checks shared by all entry points: 1 <= M, K, N <= 2^31 - 1, K % 32 == 0,
// and the weight bytes M * row_bytes, activations N * K * 4 and outputs N * M * 4
// all fit in int64.
int check_shape(int fmt, int64_t M, int64_t K, int64_t N) {
    if (!fmt_ok(fmt)) return QMM_ERR_FMT;
    if (M < 1 || K < 1 || N < 1 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return QMM_ERR_SHAPE;
    if (K % 32) return QMM_ERR_SHAPE;
    int64_t t;
    if (!mul_ok(M, row_bytes_unchecked(fmt, K), &t)) return QMM_ERR_OVERFLOW;
    if (!mul_ok(N, K, &t) || !mul_ok(t, 4, &t)) return QMM_ERR_OVERFLOW;
    if (!mul_ok(N, M, &t) || !mul_ok(t, 4, &t)) return QMM_ERR_OVERFLOW;
    return QMM_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_HIP; }

int64_t round_ws(int64_t v) { return (v + QMM_WORKSPACE_ALIGN - 1) / QMM_WORKSPACE_ALIGN * QMM_WORKSPACE_ALIGN; }

// Weight bytes of a product (both matrices for the gated one), overflow-checked.
bool weight_bytes(int fmt, int64_t M, int64_t K, bool gated, int64_t* out) {
    int64_t t;
    if (!mul_ok(M, row_bytes_unchecked(fmt, K), &t)) return false;
    return mul_ok(gated ? 2 : 1, t, out);
}

// Workspace of an fp32-token MFMA product (qmm_gemv / qmm_gate_up_silu on the MFMA
// variant).  The weight-streaming MFMA GEMV serves 2..32 tokens (block formats, K %
// 256 == 0) and scales the tokens to fp16 itself: its workspace is the split-K
// partials alone.  The GEMM serves every other case: the tokens as scaled fp16 (N x K
// halfs), their scales (N floats), then the GEMM's split-K partials.  Each part starts
// on a QMM_WORKSPACE_ALIGN boundary.
struct MfmaWs {
    qmm::GemvMfmaPlan gp;
    int64_t x16 = 0, inv = 0, part = 0, total = 0;  // byte offsets of the parts, total size
    bool ok = false;
};
MfmaWs mfma_ws(int fmt, int64_t M, int64_t K, int64_t N, bool gated) {
    MfmaWs w;
    w.gp = qmm::plan_gemv_mfma(fmt, M, K, N, gated);
    if (w.gp.ok) {
        w.total = round_ws(static_cast<int64_t>(w.gp.ws_bytes));
        w.ok = true;
        return w;
    }
    const int64_t part = static_cast<int64_t>(qmm::gemm_workspace_bytes(fmt, M, K, N, gated));
    int64_t xb, ib;
    if (!mul_ok(N, K, &xb) || !mul_ok(xb, 2, &xb) || !mul_ok(N, 4, &ib)) return w;
    w.x16 = 0;
    w.inv = round_ws(xb);
    w.part = w.inv + round_ws(ib);
    if (part > INT64_MAX - w.part - QMM_WORKSPACE_ALIGN) return w;
    w.total = w.part + round_ws(part);
    w.ok = true;
    return w;
}

// Checks a caller's workspace against the bytes a call needs.
int check_ws(const void* ws, int64_t ws_bytes, int64_t need) {
    if (need == 0) return QMM_OK;
    if (!ws || ws_bytes < need) return QMM_ERR_WORKSPACE;
    if (!aligned(ws, QMM_WORKSPACE_ALIGN)) return QMM_ERR_ALIGN;
    return QMM_OK;
}

// VALU or MFMA variant for N tokens over `wbytes` of weights with rows of K (`gated`:
// the gate+up product), measured on MI355X at the Llama-3-8B projection shapes (QKV
// 6144 x 4096, O 4096 x 4096, gate+up 2 x 14336 x 4096, down 4096 x 14336, LM head
// 128256 x 4096) with the weights streamed from HBM; the ratios below are MFMA time /
// VALU time.
//   Block formats.  The VALU kernels take up to 4 tokens per weight pass, so from 5
//   tokens they read the weights twice and the single-pass MFMA kernel wins on every
//   shape (by 1.3-2x).  At 4 tokens: long rows (K >= 8192, the down projection) go to
//   MFMA (0.68-0.96: x of 4 such tokens does not fit the DMA-fed kernel's LDS, and the
//   register-staged kernel is slower); gate+up stays VALU (0.96-1.16); the LM heads
//   of Q4_0 and Q4_1 go to MFMA (1.00, 0.92), those of Q8_0, Q5_0 and Q5_1 stay VALU
//   (1.17, 1.12, 1.02: their 4-token VALU passes run on 12-wave workgroups, and the
//   5-bit MFMA decode costs the most); QKV and O stay VALU (1.21-1.30).  At 2-3 tokens
//   VALU (1.01-1.71; one tie, Q5_1 gate+up at 3 tokens 0.96).
//   F16 (its MFMA variant is the tiled GEMM): MFMA from 5 tokens; from 2 tokens on
//   long rows over 32 MiB (down 0.72-0.85); at 4 tokens from 64 MiB (gate+up 0.94, LM
//   head 0.65), at 3 from 256 MiB (LM head 0.94); VALU otherwise (QKV, O 1.23-1.37).
int choose_variant(int fmt, int64_t wbytes, int64_t K, int64_t N, bool gated) {
    constexpr int64_t MiB = int64_t{1} << 20;
    if (N >= 5) return QMM_VARIANT_MFMA;
    if (fmt == QMM_F16) {
        if (N >= 2 && K >= 8192 && wbytes >= 32 * MiB) return QMM_VARIANT_MFMA;
        if (N == 4 && wbytes >= 64 * MiB) return QMM_VARIANT_MFMA;
        if (N == 3 && wbytes >= 256 * MiB) return QMM_VARIANT_MFMA;
        return QMM_VARIANT_VALU;
    }
    if (N == 4) {
        if (K >= 8192 && wbytes >= 16 * MiB) return QMM_VARIANT_MFMA;
        if (gated || !(fmt == QMM_Q4_0 || fmt == QMM_Q4_1)) return QMM_VARIANT_VALU;
        return wbytes >= 256 * MiB ? QMM_VARIANT_MFMA : QMM_VARIANT_VALU;
    }
    return QMM_VARIANT_VALU;
}

// The fp32-token MFMA product: the MFMA GEMV straight from fp32 tokens, or tokens to
// scaled fp16 and then the GEMM.
int run_mfma_tokens(int fmt, const void* W, const void* Wu, const float* x, float* y, int64_t M, int64_t K,
                    int64_t N, void* ws, int64_t ws_bytes, hipStream_t s) {
    const MfmaWs w = mfma_ws(fmt, M, K, N, Wu != nullptr);
    if (!w.ok) return QMM_ERR_OVERFLOW;
    const int st = check_ws(ws, ws_bytes, w.total);
    if (st) return st;
    char* base = static_cast<char*>(ws);
    float* part = reinterpret_cast<float*>(base + w.part);
    if (w.gp.ok) {
        qmm::launch_gemv_mfma(w.gp, fmt, W, Wu, x, y, M, K, N, part, s);
        return from_hip(hipGetLastError());
    }
    void* x16 = base + w.x16;
    float* inv = reinterpret_cast<float*>(base + w.inv);
    hipError_t e = qmm::launch_scale_tokens(x, x16, inv, N, K, s);
    if (e != hipSuccess) return QMM_ERR_HIP;
    return from_hip(qmm::launch_gemm_mfma(fmt, W, Wu, x16, inv, y, M, K, N, part, s));
}

}  // namespace

extern "C" {

int qmm_version(void) { return 200; }

const char* qmm_strerror(int status) {
    switch (status) {
        case QMM_OK: return "ok";
        case QMM_ERR_NULL: return "a required pointer is NULL";
        case QMM_ERR_FMT: return "unknown weight format (expected 1=F16, 2=Q4_0, 3=Q4_1, 6=Q5_0, 7=Q5_1, 8=Q8_0)";
        case QMM_ERR_SHAPE: return "bad shape (need 1 <= M, K, N <= 2^31-1 and K % 32 == 0)";
        case QMM_ERR_ALIGN: return "misaligned pointer (W, x, X need 16 bytes; outputs 4 bytes; workspace 256 bytes)";
        case QMM_ERR_OVERFLOW: return "a byte count overflows int64";
        case QMM_ERR_HIP: return "HIP runtime error at launch";
        case QMM_ERR_VARIANT: return "unknown GEMV variant";
        case QMM_ERR_ARG: return "a scalar argument is out of range (eps must be finite and >= 0; op id)";
        case QMM_ERR_WORKSPACE: return "workspace missing or smaller than qmm_workspace_size reports";
        case QMM_ERR_SCRATCH: return "the call needs more scratch than qmm_gemm_noalloc's fixed array holds";
        default: return "unknown qmm status";
    }
}

int64_t qmm_row_bytes(int fmt, int64_t K) {
    if (!fmt_ok(fmt)) return QMM_ERR_FMT;
    if (K < 1 || K > kMaxDim || K % 32) return QMM_ERR_SHAPE;
    return row_bytes_unchecked(fmt, K);
}

int qmm_dequant(int fmt, const void* W, float* out, int64_t M, int64_t K, void* stream) {
    if (!W || !out) return QMM_ERR_NULL;
    int st = check_shape(fmt, M, K, 1);
    if (st) return st;
    int64_t t;
    if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &t)) return QMM_ERR_OVERFLOW;
    if (!aligned(W, 16) || !aligned(out, 16)) return QMM_ERR_ALIGN;
    return from_hip(qmm::launch_dequant(fmt, W, out, M, K, static_cast<hipStream_t>(stream)));
}

int qmm_get_rows(int fmt, const void* W, const int32_t* ids, float* out, int64_t M, int64_t K, int64_t n,
                 void* stream) {
    if (n == 0) return fmt_ok(fmt) ? QMM_OK : QMM_ERR_FMT;
    if (!W || !ids || !out) return QMM_ERR_NULL;
    if (n < 0) return QMM_ERR_SHAPE;
    int st = check_shape(fmt, M, K, n);
    if (st) return st;
    if (!aligned(W, 16) || !aligned(ids, 4) || !aligned(out, 16)) return QMM_ERR_ALIGN;
    return from_hip(qmm::launch_get_rows(fmt, W, ids, out, M, K, n, static_cast<hipStream_t>(stream)));
}

int qmm_expand_f16(int fmt, const void* W, void* out, int64_t M, int64_t K, void* stream) {
    if (!W || !out) return QMM_ERR_NULL;
    int st = check_shape(fmt, M, K, 1);
    if (st) return st;
    int64_t t;
    if (!mul_ok(M, K, &t) || !mul_ok(t, 2, &t)) return QMM_ERR_OVERFLOW;
    if (!aligned(W, 16) || !aligned(out, 16)) return QMM_ERR_ALIGN;
    return from_hip(qmm::launch_expand_f16(fmt, W, out, M, K, static_cast<hipStream_t>(stream)));
}

int qmm_gemv_choose(int fmt, int64_t M, int64_t K, int64_t N) {
    const int st = check_shape(fmt, M, K, N);
    if (st) return st;
    int64_t wb;
    if (!weight_bytes(fmt, M, K, false, &wb)) return QMM_ERR_OVERFLOW;
    return choose_variant(fmt, wb, K, N, false);
}

int64_t qmm_workspace_size(int op, int fmt, int64_t M, int64_t K, int64_t N, int variant) {
    const int st = check_shape(fmt, M, K, N);
    if (st) return st;
    const bool gated = op == QMM_OP_GATE_UP_SILU || op == QMM_OP_GEMM_GATE_UP_SILU;
    switch (op) {
        case QMM_OP_GEMV:
        case QMM_OP_GATE_UP_SILU: {
            if (variant == QMM_VARIANT_AUTO) {
                int64_t wb;
                if (!weight_bytes(fmt, M, K, gated, &wb)) return QMM_ERR_OVERFLOW;
                variant = choose_variant(fmt, wb, K, N, gated);
            }
            if (variant == QMM_VARIANT_VALU) return 0;
            if (variant != QMM_VARIANT_MFMA) return QMM_ERR_VARIANT;
            const MfmaWs w = mfma_ws(fmt, M, K, N, gated);
            return w.ok ? w.total : QMM_ERR_OVERFLOW;
        }
        case QMM_OP_GEMM:
        case QMM_OP_GEMM_GATE_UP_SILU:
            return round_ws(static_cast<int64_t>(qmm::gemm_workspace_bytes(fmt, M, K, N, gated)));
        default:
            return QMM_ERR_ARG;
    }
}

int qmm_gemv_variant(int fmt, const void* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
                     int variant, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!W || !x || !y) return QMM_ERR_NULL;
    int st = check_shape(fmt, M, K, N);
    if (st) return st;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return QMM_ERR_ALIGN;
    if (variant == QMM_VARIANT_AUTO) {
        variant = qmm_gemv_choose(fmt, M, K, N);
        if (variant < 0) return variant;
    }
    auto s = static_cast<hipStream_t>(stream);
    if (variant == QMM_VARIANT_VALU) return from_hip(qmm::launch_gemv_valu(fmt, W, nullptr, x, y, M, K, N, s));
    if (variant == QMM_VARIANT_MFMA) return run_mfma_tokens(fmt, W, nullptr, x, y, M, K, N, workspace, workspace_bytes, s);
    return QMM_ERR_VARIANT;
}

int qmm_gemv(int fmt, const void* W, const float* x, float* y, int64_t M, int64_t K, int64_t N, void* workspace,
             int64_t workspace_bytes, void* stream) {
    return qmm_gemv_variant(fmt, W, x, y, M, K, N, QMM_VARIANT_AUTO, workspace, workspace_bytes, stream);
}

int qmm_gate_up_silu_variant(int fmt, const void* Wg, const void* Wu, const float* x, float* h, int64_t I,
                             int64_t K, int64_t N, int variant, void* workspace, int64_t workspace_bytes,
                             void* stream) {
    if (!Wg || !Wu || !x || !h) return QMM_ERR_NULL;
    int st = check_shape(fmt, I, K, N);
    if (st) return st;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(x, 16) || !aligned(h, 4)) return QMM_ERR_ALIGN;
    if (variant == QMM_VARIANT_AUTO) {
        int64_t wb;
        if (!weight_bytes(fmt, I, K, true, &wb)) return QMM_ERR_OVERFLOW;
        variant = choose_variant(fmt, wb, K, N, true);
    }
    auto s = static_cast<hipStream_t>(stream);
    if (variant == QMM_VARIANT_VALU) return from_hip(qmm::launch_gemv_valu(fmt, Wg, Wu, x, h, I, K, N, s));
    if (variant == QMM_VARIANT_MFMA) return run_mfma_tokens(fmt, Wg, Wu, x, h, I, K, N, workspace, workspace_bytes, s);
    return QMM_ERR_VARIANT;
}

int qmm_gate_up_silu(int fmt, const void* Wg, const void* Wu, const float* x, float* h, int64_t I, int64_t K,
                     int64_t N, void* workspace, int64_t workspace_bytes, void* stream) {
    return qmm_gate_up_silu_variant(fmt, Wg, Wu, x, h, I, K, N, QMM_VARIANT_AUTO, workspace, workspace_bytes, stream);
}

int qmm_rmsnorm_gemv(int fmt, const void* W, const float* x, const float* gamma, float eps, float* y, int64_t M,
                     int64_t K, int64_t N, void* stream) {
    if (!W || !x || !gamma || !y) return QMM_ERR_NULL;
    int st = check_shape(fmt, M, K, N);
    if (st) return st;
    if (!(eps >= 0.0f) || !isfinite(eps)) return QMM_ERR_ARG;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(gamma, 16) || !aligned(y, 4)) return QMM_ERR_ALIGN;
    qmm::DecodeEpi epi;
    epi.gamma = gamma;
    epi.eps = eps;
    return from_hip(qmm::launch_gemv_valu(fmt, W, nullptr, x, y, M, K, N, static_cast<hipStream_t>(stream),
                                          qmm::EP_NORM, epi));
}

int qmm_rmsnorm_gate_up_silu(int fmt, const void* Wg, const void* Wu, const float* x, const float* gamma, float eps,
                             float* h, int64_t I, int64_t K, int64_t N, void* stream) {
    if (!Wg || !Wu || !x || !gamma || !h) return QMM_ERR_NULL;
    int st = check_shape(fmt, I, K, N);
    if (st) return st;
    if (!(eps >= 0.0f) || !isfinite(eps)) return QMM_ERR_ARG;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(x, 16) || !aligned(gamma, 16) || !aligned(h, 4))
        return QMM_ERR_ALIGN;
    qmm::DecodeEpi epi;
    epi.gamma = gamma;
    epi.eps = eps;
    return from_hip(qmm::launch_gemv_valu(fmt, Wg, Wu, x, h, I, K, N, static_cast<hipStream_t>(stream),
                                          qmm::EP_NORM, epi));
}

int qmm_gemv_add(int fmt, const void* W, const float* x, const float* r, float* y, int64_t M, int64_t K, int64_t N,
                 void* stream) {
    if (!W || !x || !r || !y) return QMM_ERR_NULL;
    int st = check_shape(fmt, M, K, N);
    if (st) return st;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(r, 4) || !aligned(y, 4)) return QMM_ERR_ALIGN;
    qmm::DecodeEpi epi;
    epi.res = r;
    return from_hip(qmm::launch_gemv_valu(fmt, W, nullptr, x, y, M, K, N, static_cast<hipStream_t>(stream),
                                          qmm::EP_RES, epi));
}

int qmm_gemm(int fmt, const void* W, const void* X, float* Y, int64_t M, int64_t K, int64_t T, void* workspace,
             int64_t workspace_bytes, void* stream) {
    if (!W || !X || !Y) return QMM_ERR_NULL;
    int st = check_shape(fmt, M, K, T);
    if (st) return st;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 4)) return QMM_ERR_ALIGN;
    st = check_ws(workspace, workspace_bytes, static_cast<int64_t>(qmm::gemm_workspace_bytes(fmt, M, K, T, false)));
    if (st) return st;
    return from_hip(qmm::launch_gemm_mfma(fmt, W, nullptr, X, nullptr, Y, M, K, T, static_cast<float*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

int qmm_gemm_gate_up_silu(int fmt, const void* Wg, const void* Wu, const void* X, float* H, int64_t I, int64_t K,
                          int64_t T, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!Wg || !Wu || !X || !H) return QMM_ERR_NULL;
    int st = check_shape(fmt, I, K, T);
    if (st) return st;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(X, 16) || !aligned(H, 4)) return QMM_ERR_ALIGN;
    st = check_ws(workspace, workspace_bytes, static_cast<int64_t>(qmm::gemm_workspace_bytes(fmt, I, K, T, true)));
    if (st) return st;
    return from_hip(qmm::launch_gemm_mfma(fmt, Wg, Wu, X, nullptr, H, I, K, T, static_cast<float*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
