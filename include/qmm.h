/*
 * qmm.h -- GGUF block-quantized weight x activation products on AMD MI355X (gfx950).
 *
 * The weights stay in their GGUF block bytes in device memory and are decoded in
 * registers (or into LDS tiles) inside the product kernels; no float copy of a
 * weight matrix is ever written.  ("EdgeRunner Core Architecture", section 3.4
 * Weight Dequantization Strategy, Tier 1: raw quantized buffers go straight into
 * the fused product kernels; section 15, item 2: this cuts the weight bytes read
 * by about 3.8x against decoding to float32 first.)
 *
 * Formats (GGUF type ids, "EdgeRunner Core Architecture" section 1.3; block sizes,
 * section 3.1; Q8_0 byte order, section 3.2):
 *   QMM_F16  = 1 : 2 bytes per weight, IEEE binary16, little endian.
 *   QMM_Q4_0 = 2 : 18 bytes per 32 weights: fp16 scale d, then 16 bytes; byte j holds
 *                  weight j in its low nibble and weight j+16 in its high nibble;
 *                  weight = d * (nibble - 8).
 *   QMM_Q8_0 = 8 : 34 bytes per 32 weights: fp16 scale d, then 32 int8 codes q;
 *                  weight = d * q.
 *   QMM_Q4_1 = 3 : 20 bytes per 32 weights: fp16 scale d, fp16 bias m, then 16 bytes
 *                  of nibbles in Q4_0's order; weight = d * n + m.
 *   QMM_Q5_0 = 6 : 22 bytes per 32 weights: fp16 scale d, a 32-bit little-endian word
 *                  qh whose bit e is the fifth bit of weight e, then 16 bytes of low
 *                  nibbles in Q4_0's order; u = n + 16 * bit, weight = d * (u - 16).
 *   QMM_Q5_1 = 7 : 24 bytes per 32 weights: fp16 d, fp16 m, qh, 16 bytes of nibbles;
 *                  weight = d * u + m.
 *   (Section 1.3 gives the ids 3, 6, 7 and section 3.1 the byte counts and the
 *   scale/bias/5-bit nature; the field order within the block is GGUF's.)
 *   Every entry point takes every format.
 *
 * Matrix convention (llama.cpp Metal end-to-end path, section 3.2 MUL_MAT: the
 * reduction length K is the contiguous weight dimension; the token count is the
 * second operand's row count):
 *   W : M rows, each row K weights = K/32 consecutive blocks (F16: K halfs),
 *       rows stored back to back (row stride = qmm_row_bytes(fmt, K)).
 *   x : N (or T) rows of K activations, row-major.
 *   y : N (or T) rows of M outputs, row-major, float32:  y[n][m] = sum_k W[m][k] x[n][k].
 *
 * Activations are never quantised ("alpaca.swift", Limitations): decode takes fp32
 * x; prefill takes fp16 X ("alpaca.swift", Design: half-precision prefill
 * activations).  Products accumulate in fp32.
 *
 * Common rules for every entry point:
 *   - All array arguments are device pointers owned by the caller.  The library
 *     allocates no memory and keeps no state: the MFMA products that need scratch
 *     memory (split-K partials; fp32 tokens converted to scaled fp16) take it from a
 *     caller-owned workspace whose size qmm_workspace_size reports for the same
 *     arguments; calls that need none accept NULL, 0.  The same arguments always
 *     run the same kernels, eagerly or while the stream is captured into a graph.
 *     Calls are re-entrant; two calls that run concurrently need separate
 *     workspaces.  (Pre-allocated scratch buffers and no allocation per pass:
 *     "EdgeRunner Core Architecture", section 10 Scratch Buffers and section 15,
 *     item 4.)
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).  All
 *     work is enqueued asynchronously on it; nothing synchronises.
 *   - Arguments are validated on the host before any HIP call; a failure returns
 *     a negative qmm_status and enqueues nothing.  A launch failure reported by
 *     hipGetLastError returns QMM_ERR_HIP.
 *   - Size checks follow the practice of bounding every length and checking
 *     every size product for overflow ("alpaca.swift", Highlights: the GGUF
 *     parser treats files as untrusted).
 *   - Outputs must not alias inputs (not checked), except where a call says so.
 *   - Alignment: W, x, X, gamma must be 16-byte aligned; y, Y, h, H, r 4-byte aligned
 *     (out of qmm_get_rows / qmm_expand_f16: 16 bytes); a workspace
 *     QMM_WORKSPACE_ALIGN (256) bytes.
 *   - Limits: 1 <= M, K, N, T <= 2^31 - 1 and K % 32 == 0 for every format (F16
 *     included, so that all formats share the 32-wide tiling).
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMM_F16 = 1,
    QMM_Q4_0 = 2,
    QMM_Q4_1 = 3,
    QMM_Q5_0 = 6,
    QMM_Q5_1 = 7,
    QMM_Q8_0 = 8
} qmm_fmt;

typedef enum {
    QMM_OK = 0,
    QMM_ERR_NULL = -1,        /* a required pointer is NULL                        */
    QMM_ERR_FMT = -2,         /* format id is not 1, 2, 3, 6, 7 or 8               */
    QMM_ERR_SHAPE = -3,       /* M, K, N or T out of range, or K % 32 != 0         */
    QMM_ERR_ALIGN = -4,       /* a pointer violates the alignment rule above       */
    QMM_ERR_OVERFLOW = -5,    /* a byte count does not fit in int64                */
    QMM_ERR_HIP = -6,         /* the HIP runtime reported an error at launch       */
    QMM_ERR_VARIANT = -7,     /* unknown variant id passed to a *_variant call     */
    QMM_ERR_ARG = -8,         /* a scalar argument is out of range (eps, op id)    */
    QMM_ERR_WORKSPACE = -9,   /* workspace NULL or smaller than the call needs     */
    QMM_ERR_SCRATCH = -10     /* qmm_gemm_noalloc: the call needs more than its fixed scratch */
} qmm_status;

/* Alignment every workspace pointer must have. */
#define QMM_WORKSPACE_ALIGN 256

/* Bytes of the fixed device scratch array qmm_gemm_noalloc uses on each GPU. */
#define QMM_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

/* Operation ids for qmm_workspace_size. */
typedef enum {
    QMM_OP_GEMV = 1,              /* qmm_gemv, qmm_gemv_variant                   */
    QMM_OP_GATE_UP_SILU = 2,      /* qmm_gate_up_silu, qmm_gate_up_silu_variant   */
    QMM_OP_GEMM = 3,              /* qmm_gemm                                     */
    QMM_OP_GEMM_GATE_UP_SILU = 4  /* qmm_gemm_gate_up_silu                        */
} qmm_op;

/* Variant ids for qmm_gemv_variant, qmm_gate_up_silu_variant and qmm_gemv_choose. */
typedef enum {
    QMM_VARIANT_AUTO = 0,     /* library picks from (fmt, M, K, N)                          */
    QMM_VARIANT_VALU = 1,     /* register-decode GEMV: one weight read, N fp32 FMAs          */
    QMM_VARIANT_MFMA = 2      /* LDS-tile decode + fp16 MFMA (x scaled per token, then fp16) */
} qmm_variant;

/* Library version (major*10000 + minor*100 + patch). */
int qmm_version(void);

/* Human-readable text for a qmm_status value (static storage; never NULL). */
const char* qmm_strerror(int status);

/*
 * Bytes of caller-owned device workspace that the call of operation `op`
 * (QMM_OP_*) with these arguments needs, 0 when it needs none; a negative
 * qmm_status for invalid arguments.  M is the output rows (I for the gated
 * products), N the token count (T for the GEMMs); `variant` is the variant passed
 * to qmm_gemv_variant / qmm_gate_up_silu_variant (QMM_VARIANT_AUTO for qmm_gemv,
 * qmm_gate_up_silu and the GEMMs, where it is ignored).  Host-only; makes no HIP
 * call.  The workspace holds a call's split-K partial sums (when the output tiles
 * cannot fill the GPU, K is split over several workgroups and a second kernel adds
 * their sums in a fixed order) and, for the fp32-token MFMA variant when it runs on
 * the GEMM (F16 weights, more than 32 tokens, or K not a multiple of 256), the
 * tokens converted to scaled fp16 and their scales.  Its contents need no initialisation
 * and are dead after the call's kernels finish.  ("EdgeRunner Core Architecture",
 * section 10 Scratch Buffers: scratch memory is allocated once and reused by every
 * pass.)
 */
int64_t qmm_workspace_size(int op, int fmt, int64_t M, int64_t K, int64_t N, int variant);

/*
 * Bytes per weight row: K/32 blocks of 34 (Q8_0), 18 (Q4_0), 20 (Q4_1), 22 (Q5_0) or
 * 24 (Q5_1) bytes; 2*K (F16).
 * ("EdgeRunner Core Architecture", section 3.1 bytes per block; section 3.2 block
 * count times 34.)  Returns a negative qmm_status for an unknown format, K < 1,
 * K % 32 != 0 or K > 2^31 - 1.  Host-only; makes no HIP call.
 */
int64_t qmm_row_bytes(int fmt, int64_t K);

/*
 * Decode a whole matrix to fp32: out[m][k] = W[m][k] (float32, row-major M x K).
 * Every decoded value d*q (or d*(n-8), d*(u-16), or an f16) is exact in fp32, so the
 * result is bit-exact; the biased formats give d*u + m rounded once to fp32.  ("EdgeRunner Core Architecture", section 3.4, Tier 2: GPU decode
 * kernels that write a float buffer; "alpaca.swift", Numerical validation:
 * dequantisation is bit-exact.)  Not used by the product paths; it is the
 * check of the decoders and the building block of decode-then-GEMM prefill.
 */
int qmm_dequant(int fmt, const void* W, float* out, int64_t M, int64_t K, void* stream);

/*
 * Quantised row gather (embedding lookup): out[i][k] = W[ids[i]][k] as float32,
 * for i < n; out is n x K row-major.  ids is a device array of n int32 row
 * indices (4-byte aligned; repeats allowed); only the rows named are read.
 * Values as in qmm_dequant (bit-exact against the same rounding).  An id outside
 * [0, M) cannot be checked on the host (ids live on the device): its output row
 * is filled with NaN and nothing outside W is read.  n == 0 is a no-op that
 * returns QMM_OK.  out must be 16-byte aligned.
 * ("llama.cpp Metal ...", section 3.2 Input embd and P8: token ids go through a
 * per-format get_rows kernel on the token-embedding matrix; "EdgeRunner Core
 * Architecture", section 3.4, Tier 3: embeddings decode straight into the
 * destination, with no float copy of the table.)
 */
int qmm_get_rows(int fmt, const void* W, const int32_t* ids, float* out,
                 int64_t M, int64_t K, int64_t n, void* stream);

/*
 * Expand a whole matrix to half precision: out[m][k] = fp16(W[m][k]), rounded to
 * nearest even (F16: a copy), M x K row-major, 16-byte aligned.  These are the
 * same fp16 values the fused qmm_gemm decodes into its LDS tiles, so
 * qmm_gemm(QMM_F16, out, ...) computes what qmm_gemm(fmt, W, ...) computes.  This
 * is the expand-then-GEMM prefill variant: the caller owns the M*K*2-byte buffer.
 * ("alpaca.swift", Design: quantised matrices are expanded one at a time into a
 * scratch buffer before the matrix-hardware GEMM; "EdgeRunner Core Architecture",
 * section 3.4, Tier 2: GPU decode kernels writing float16.)
 */
int qmm_expand_f16(int fmt, const void* W, void* out, int64_t M, int64_t K, void* stream);

/*
 * Decode GEMV: y[n][m] = sum_k W[m][k] * x[n][k] for n < N, fp32 x and y.
 * N = 1 is single-token decode; small N (a few tokens) reads every weight once
 * and reuses it N times.  ("EdgeRunner Core Architecture", section 2.1 fused
 * Q8_0 dequant + GEMV pipelines; "llama.cpp Metal ...", section 3.2 and P9:
 * per-format mat-vec kernels for one token and a batched mat-vec for 2..8 tokens.)
 * The variant is chosen from (fmt, M, K, N) as qmm_gemv_choose reports; workspace
 * (workspace_bytes of it) must hold qmm_workspace_size(QMM_OP_GEMV, ...) bytes
 * (NULL, 0 when that is 0, as it is for the register-decode variant), else
 * QMM_ERR_WORKSPACE.
 * Precision ("alpaca.swift", Numerical validation: each reduced-precision path has
 * a derived element-wise bound): accumulation is fp32 everywhere.
 *   Register-decode variant, block formats: x is held in block floating point
 *   (each 32-value block scaled by a power of two, then rounded to fp16) and every
 *   weight code enters packed fp16 dot products exactly, so
 *   |y - y_exact| <= (2^-11 + 3 (25 + K/2048) 2^-23)(1 + 2^-11) sum_k |W[m][k] x[n][k]|
 *   for every finite x (blocks whose dynamic range fp16 cannot hold take an exact
 *   fp32 path); x = e_k returns W[:, k] exactly (biased formats: d u + m rounded
 *   once).  F16 weights and rows left to its fallback use fp32 x and fp32 FMAs.
 *   MFMA variant: each token is scaled by a power of two and rounded to fp16 --
 *   on the GEMM one scale per token, which brings its largest |x| into [2^14,
 *   2^15); in the weight-streaming kernel (block formats, 2..32 tokens) a running
 *   scale per token and workgroup, which keeps the largest |x| read so far below
 *   2^15 -- and weights enter as fp16(w), one rounding; |y - y_exact| <= about
 *   2^-10 sum_k |W[m][k] x[n][k]| while every decoded |w| is below 65520 (larger
 *   ones overflow fp16) and no nonzero x lies more than 2^28 below its token's
 *   largest (such elements keep an absolute error of at most 2^-39 times that
 *   largest).
 * Fused QKV is this call on the row-concatenation [Wq; Wk; Wv] (M = q + 2 kv).
 */
int qmm_gemv(int fmt, const void* W, const float* x, float* y,
             int64_t M, int64_t K, int64_t N, void* workspace, int64_t workspace_bytes, void* stream);

/* As qmm_gemv with an explicit variant (QMM_VARIANT_*), for crossover sweeps. */
int qmm_gemv_variant(int fmt, const void* W, const float* x, float* y,
                     int64_t M, int64_t K, int64_t N, int variant,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The variant qmm_gemv would run for these sizes (a QMM_VARIANT_* value >= 1),
 * or a negative qmm_status for invalid sizes.  Host-only.  The GEMV/GEMM split
 * by token count follows "llama.cpp Metal ...", section 3.2 (mat-vec for few
 * tokens, the tiled matrix-matrix kernel above a threshold); the thresholds here
 * are measured on MI355X at the Llama-3-8B projection shapes: the block formats
 * switch to MFMA from 5 tokens, and at 4 tokens for rows of K >= 8192 over at least
 * 16 MiB of weights and for Q4_0 / Q4_1 matrices of 256 MiB or more; F16 (whose
 * MFMA variant is the tiled GEMM) from 5 tokens, from 2 for rows of K >= 8192 over
 * at least 32 MiB, at 4 from 64 MiB and at 3 from 256 MiB.  (qmm_gate_up_silu
 * applies the same rule to the combined gate and up weights, except that the block
 * formats' short rows stay on the register-decode variant at 4 tokens.)
 */
int qmm_gemv_choose(int fmt, int64_t M, int64_t K, int64_t N);

/*
 * Fused gate+up projection with the SwiGLU epilogue, fp32 x:
 *   g = x Wg^T, u = x Wu^T, h[n][i] = silu(g[n][i]) * u[n][i],  silu(z) = z / (1 + e^-z).
 * Wg and Wu are two I x K matrices in the same format (a concatenated [gate; up]
 * buffer is Wg = base, Wu = base + I * qmm_row_bytes(fmt, K)).  h is N x I fp32.
 * Workspace and precision of g and u as for qmm_gemv (QMM_OP_GATE_UP_SILU).
 * ("EdgeRunner Core Architecture", section 8 SwiGLU FFN: SiLU of the gate times
 * up, fused into one dispatch for single-token decode.)
 */
int qmm_gate_up_silu(int fmt, const void* Wg, const void* Wu, const float* x, float* h,
                     int64_t I, int64_t K, int64_t N, void* workspace, int64_t workspace_bytes, void* stream);

/* As qmm_gate_up_silu with an explicit variant (QMM_VARIANT_*), for crossover sweeps. */
int qmm_gate_up_silu_variant(int fmt, const void* Wg, const void* Wu, const float* x, float* h,
                             int64_t I, int64_t K, int64_t N, int variant,
                             void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Decode GEMV with the RMSNorm prologue fused in:
 *   x'[n][k] = x[n][k] / sqrt(mean_k x[n][k]^2 + eps) * gamma[k],
 *   y[n][m]  = sum_k W[m][k] * x'[n][k].
 * For the attention norm + fused QKV and the final norm + LM head.  gamma is K
 * fp32 norm weights (16-byte aligned); eps must be finite and >= 0 (else
 * QMM_ERR_ARG).  Runs the register-decode GEMV kernels (4 tokens per weight pass):
 * each workgroup forms gamma .* x while staging x and gathers the sum of squares on
 * the same pass, then scales its reduced dot products, so the norm adds only the
 * K * 4 bytes of gamma.  ("EdgeRunner Core Architecture", section 6 RMSNorm,
 * section 2.1 fused QKV with RMSNorm, section 9.2 fused decode pass with the final
 * norm folded into the LM head.  The page leaves open where eps enters: here it is
 * added to the mean square inside the root; Llama-style norms have no bias.)
 */
int qmm_rmsnorm_gemv(int fmt, const void* W, const float* x, const float* gamma, float eps, float* y,
                     int64_t M, int64_t K, int64_t N, void* stream);

/*
 * Gate+up SwiGLU with the FFN RMSNorm prologue: h = silu(x' Wg^T) * (x' Wu^T) with
 * x' as in qmm_rmsnorm_gemv.  ("EdgeRunner Core Architecture", section 8: RMSNorm,
 * gate, up and SiLU in one dispatch at a single token.)
 */
int qmm_rmsnorm_gate_up_silu(int fmt, const void* Wg, const void* Wu, const float* x, const float* gamma,
                             float eps, float* h, int64_t I, int64_t K, int64_t N, void* stream);

/*
 * Decode GEMV with the residual-add epilogue: y[n][m] = sum_k W[m][k] x[n][k] + r[n][m].
 * r has y's layout (N x M fp32, 4-byte aligned) and may be y itself (in-place add
 * into the residual stream; each element is read, then written, by one lane; any
 * other overlap is not allowed).  For the O and down projections.  Register-decode
 * GEMV kernels, 4 tokens per weight pass.  ("EdgeRunner Core Architecture",
 * section 9.1 steps 13-14 and section 9.2: the O and down GEMVs add into the
 * residual in the same dispatch.)
 */
int qmm_gemv_add(int fmt, const void* W, const float* x, const float* r, float* y,
                 int64_t M, int64_t K, int64_t N, void* stream);

/*
 * Prefill GEMM: Y[t][m] = sum_k W[m][k] * X[t][k], X fp16 (T x K), Y fp32 (T x M).
 * Weight blocks are decoded into fp16 MFMA operands, each exact weight (d*q, or
 * d*u + m) rounded once to nearest even -- the values qmm_expand_f16 writes -- and
 * fed to fp16 MFMA with fp32 accumulation.  Range: a decoded weight must satisfy
 * |w| < 65520 (fp16(w) is infinite beyond), i.e. |d q| < 65520 for the block
 * formats; within it |Y - Y_exact| <= about 2^-11 sum_k |W[m][k] X[t][k]| plus the
 * fp32 accumulation.  workspace (workspace_bytes of it) must hold
 * qmm_workspace_size(QMM_OP_GEMM, fmt, M, K, T, 0) bytes (the split-K partials when
 * the tiles alone cannot fill the GPU; NULL, 0 when that is 0), else
 * QMM_ERR_WORKSPACE.  ("alpaca.swift", Design and Capabilities: prefill on the
 * matrix hardware with half-precision activations; Numerical validation:
 * element-wise error bound proportional to sum |x w|.)
 */
int qmm_gemm(int fmt, const void* W, const void* X, float* Y,
             int64_t M, int64_t K, int64_t T, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qmm_gemm for callers that cannot allocate: code under graph capture that owns no
 * buffers, tight serving loops, harnesses that forbid hipMalloc.  The same kernels
 * and results as qmm_gemm with a workspace, but the split-K partials live in a fixed
 * device array of QMM_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends; the call allocates nothing of any kind.  Every call
 * on a GPU shares that GPU's array, so calls that overlap on one GPU race (serialise
 * them: one stream, or events).  A call whose partials would not fit returns
 * QMM_ERR_SCRATCH (qmm_gemm's plan needs at most 64 MiB).  The device address of the
 * array is looked up once per device, on the first call made with that device
 * current.  Other arguments and errors as qmm_gemm.
 */
int qmm_gemm_noalloc(int fmt, const void* W, const void* X, float* Y,
                     int64_t M, int64_t K, int64_t T, void* stream);

/*
 * Prefill gate+up with the SwiGLU epilogue: H[t][i] = silu((X Wg^T)[t][i]) * (X Wu^T)[t][i].
 * X fp16 (T x K), H fp32 (T x I).  Same tiles, rounding, range and workspace rule
 * as qmm_gemm (QMM_OP_GEMM_GATE_UP_SILU).
 */
int qmm_gemm_gate_up_silu(int fmt, const void* Wg, const void* Wu, const void* X, float* H,
                          int64_t I, int64_t K, int64_t T, void* workspace, int64_t workspace_bytes,
                          void* stream);

/* Workgroups of qmm_stream_read: the length of its sink array. */
#define QMM_STREAM_READ_BLOCKS 8192

/*
 * Streaming-read reference, a measurement aid rather than a step of the method: reads
 * `bytes` of device memory at buf with the 16-byte non-temporal loads of the
 * single-token decode stream and stores one word per workgroup, sink[b] = the XOR of
 * the 32-bit words of the b-th of QMM_STREAM_READ_BLOCKS ranges of 16-byte units, each
 * ceil(units / QMM_STREAM_READ_BLOCKS) long (the last ones shorter or empty: 0).
 * bytes / elapsed time is the read rate a plain kernel reaches on the GPU, the
 * achievable ceiling against which the decode GEMVs' weight streams are read beside
 * the nominal HBM peak.  buf 16-byte aligned, bytes a positive multiple of 16, sink
 * QMM_STREAM_READ_BLOCKS uint32 of device memory, 4-byte aligned; otherwise
 * QMM_ERR_NULL, QMM_ERR_SHAPE or QMM_ERR_ALIGN before any launch.  Asynchronous on
 * stream like every other call.
 */
int qmm_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
