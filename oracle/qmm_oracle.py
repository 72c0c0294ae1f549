"""Float64 CPU oracle for GGUF block-quantized matrix products.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports or calls this module.  Only the tests, the smoke check
in ``__graft_entry__.smoke`` and the CPU-baseline leg of ``bench.py`` use it.
It shares no code with the GPU path: it decodes the raw bytes itself with numpy.

Every function states the passage it follows.  Pages cited:

* "EdgeRunner Core Architecture" (EdgeRunner): section 1.3 TensorStorage &
  TensorDataType (GGUF type ids, bytes per block), section 3.1 Quantization
  Format Summary, section 3.2 Q8_0 Layout, section 3.4 Weight Dequantization
  Strategy (raw blocks used without materialising float weights; Tier 2 decode to
  float16; Tier 3 embedding rows), section 6 RMSNorm, section 8 SwiGLU FFN,
  sections 9.1 and 9.2 (norms and residual adds folded into the decode GEMVs).
* "llama.cpp Metal (MPS) End-to-End Inference Path" (llama.cpp Metal): section
  3.2 MUL_MAT 3-way kernel selection (ne00 is the contiguous reduction length K,
  ne11 the number of tokens) and Input embd; P8 GET_ROWS.
* "alpaca.swift": Capabilities (F16, Q8_0, Q4_0 weights used in place),
  Design (weights expanded to half precision for the prefill GEMM),
  Numerical validation (float64 reference, bit-exact dequantisation, the
  element-wise error bound 2^-10 * sum |x_k w_k| for the half-precision GEMM),
  Limitations (activations stay in floating point).

Readings of points the pages leave open (each also listed with the design notes):

* Q8_0: the fp16 scale is little-endian IEEE binary16 at byte 0; the 32 codes are
  two's-complement int8 at bytes 2..33; weight = d * q.
* Q4_0: the pages give only "4-bit, 32 per block, fp16 scale, 18 bytes".  Adopted:
  the GGUF arrangement, byte j of the 16 code bytes carries element j in its low
  nibble and element j + 16 in its high nibble; weight = d * (nibble - 8).
* Q4_1, Q5_0, Q5_1: the pages give the type ids (3, 6, 7), the bytes per block
  (20, 22, 24) and one phrase each (4-bit codes with an fp16 bias; 5-bit codes
  with an fp16 scale; 5-bit codes with an fp16 bias).  Adopted, the GGUF
  arrangement: fp16 scale d at byte 0; for the biased formats the fp16 bias m
  follows at byte 2; the 5-bit formats then hold a 32-bit little-endian word qh
  whose bit e is the fifth (high) bit of element e; the last 16 bytes hold the
  low four bits in Q4_0's nibble order.  With u the element's 4- or 5-bit code:
  Q4_1 w = d*u + m, Q5_0 w = d*(u - 16), Q5_1 w = d*u + m.  d*u + m is exact in
  float64 (every fp16 is a multiple of 2^-24 below 2^16, so the sum spans fewer
  than 53 bits).  These layouts are not printed on the pages: the pins below fix
  the oracle to this reading, not the reading to an outside specification.
* Orientation: W is row-major [M][K] (rows of K/32 blocks), y = x W^T with x
  token-major [N][K].
* Fp16 scales decode with IEEE semantics, subnormals included; inf and NaN
  propagate.

Parity pins (tests under tests/test_oracle.py): hand-computed blocks stored in
tests/golden (decode and nibble order; one block for the fp16 expansion's
ties-to-even), all 65536 fp16 patterns against a manual sign/exponent/mantissa
decode, exact rational brute force on tiny shapes, pack/unpack round trip, SiLU
and RMSNorm closed forms, row gathers of golden blocks, the golden dots reached
through the norm and residual references, and the soundness of the fused-output
bounds by perturbation.  Q4_1 / Q5_0 / Q5_1: hand-computed blocks (field order,
fifth-bit order, offset and bias sign; one block whose fp16 expansion needs a
single rounding of the exact value), identities that reduce each to the pinned
Q4_0 decoder or to one another, the per-bit placement of the fifth bits, round
trips, the pages' byte counts, and exact rational brute force.
"""
from __future__ import annotations

import math

import numpy as np

FMT_F16 = 1   # GGUF type ids (EdgeRunner, section 1.3)
FMT_Q4_0 = 2
FMT_Q4_1 = 3
FMT_Q5_0 = 6
FMT_Q5_1 = 7
FMT_Q8_0 = 8

QK = 32                         # weights per block (EdgeRunner, section 3.1)
BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q4_0: 18, FMT_Q4_1: 20, FMT_Q5_0: 22, FMT_Q5_1: 24}

# Acceptance constants: |y_gpu - y_ref| <= REL * S + ABS, S = sum_k |w_k x_k|.
# REL = 2e-3 is about 2x the 2^-10 element-wise bound alpaca.swift states for its
# half-precision GEMM (Numerical validation).
TOL_REL = 2e-3
TOL_ABS = 1e-6


# ---------------------------------------------------------------- unpacking
def row_bytes(fmt: int, K: int) -> int:
    """Bytes per row: K/32 blocks of 34 (Q8_0), 18 (Q4_0), 20 (Q4_1), 22 (Q5_0) or
    24 (Q5_1) bytes; 2K (F16).

    EdgeRunner, section 3.1 (bytes per block) and section 3.2 (block count times 34).
    """
    if fmt == FMT_F16:
        return 2 * K
    if fmt not in BLOCK_BYTES or K % QK:
        raise ValueError("bad format or K")
    return K // QK * BLOCK_BYTES[fmt]


def _blocks(raw: np.ndarray, fmt: int, M: int, K: int) -> np.ndarray:
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(-1)
    if raw.size != M * row_bytes(fmt, K):
        raise ValueError("byte count does not match M x K")
    return raw.reshape(M, K // QK, BLOCK_BYTES[fmt])


def _scale64(blk: np.ndarray, at: int = 0) -> np.ndarray:
    """fp16 at bytes at..at+1 (little endian) -> float64, IEEE semantics."""
    d16 = np.ascontiguousarray(blk[..., at:at + 2]).view("<f2")[..., 0]
    return d16.astype(np.float64)


def _nibbles(qs: np.ndarray) -> np.ndarray:
    """16 code bytes -> 32 four-bit codes: low nibbles are elements 0..15, high
    nibbles elements 16..31 (the adopted GGUF order, shared by Q4_0/Q4_1/Q5_x)."""
    b = qs.astype(np.int64)
    return np.concatenate([b & 15, b >> 4], axis=-1)


def _high_bits(qh: np.ndarray) -> np.ndarray:
    """4 bytes of a little-endian 32-bit word -> its 32 bits, bit e at index e."""
    word = np.ascontiguousarray(qh).view("<u4")[..., 0].astype(np.int64)
    return (word[..., None] >> np.arange(32)) & 1


def unpack_q8_0(raw, M: int, K: int) -> np.ndarray:
    """Q8_0 -> float64 [M][K]: w_i = d * q_i, q_i = int8 at byte 2 + i.

    EdgeRunner, section 3.2 Q8_0 Layout (scale first, then 32 one-byte codes).
    """
    blk = _blocks(raw, FMT_Q8_0, M, K)
    d = _scale64(blk)                                         # [M][nb]
    q = np.ascontiguousarray(blk[..., 2:34]).view(np.int8)    # [M][nb][32]
    with np.errstate(invalid="ignore"):                       # inf scale * 0 code -> NaN
        return (d[..., None] * q.astype(np.float64)).reshape(M, K)


def unpack_q4_0(raw, M: int, K: int) -> np.ndarray:
    """Q4_0 -> float64 [M][K]: w_j = d*((b_j & 15) - 8), w_{j+16} = d*((b_j >> 4) - 8).

    EdgeRunner, sections 1.3 and 3.1 (4-bit codes, fp16 scale, 18 bytes); nibble
    order and the -8 offset are the adopted GGUF reading.
    """
    blk = _blocks(raw, FMT_Q4_0, M, K)
    d = _scale64(blk)
    b = blk[..., 2:18].astype(np.int64)                       # [M][nb][16]
    lo = (b & 15) - 8
    hi = (b >> 4) - 8
    q = np.concatenate([lo, hi], axis=-1).astype(np.float64)  # element j, then j + 16
    with np.errstate(invalid="ignore"):
        return (d[..., None] * q).reshape(M, K)


def unpack_q4_1(raw, M: int, K: int) -> np.ndarray:
    """Q4_1 -> float64 [M][K]: w_e = d * u_e + m, u_e the 4-bit code of element e.

    EdgeRunner, sections 1.3 and 3.1 (type id 3, 20 bytes: 4-bit codes with an fp16
    bias).  Byte positions (d at 0, m at 2, codes at 4..19) and nibble order are the
    adopted GGUF reading.
    """
    blk = _blocks(raw, FMT_Q4_1, M, K)
    d, m = _scale64(blk, 0), _scale64(blk, 2)
    u = _nibbles(blk[..., 4:20]).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (d[..., None] * u + m[..., None]).reshape(M, K)


def unpack_q5_0(raw, M: int, K: int) -> np.ndarray:
    """Q5_0 -> float64 [M][K]: w_e = d * (u_e - 16), u_e = nibble_e + 16 * bit e of qh.

    EdgeRunner, sections 1.3 and 3.1 (type id 6, 22 bytes: 5-bit codes with an fp16
    scale).  d at 0, qh at 2..5, low nibbles at 6..21, and the offset 16 (the
    middle of the 5-bit range, as 8 is for Q4_0) are the adopted GGUF reading.
    """
    blk = _blocks(raw, FMT_Q5_0, M, K)
    d = _scale64(blk, 0)
    u = _nibbles(blk[..., 6:22]) + 16 * _high_bits(blk[..., 2:6])
    with np.errstate(invalid="ignore"):
        return (d[..., None] * (u - 16).astype(np.float64)).reshape(M, K)


def unpack_q5_1(raw, M: int, K: int) -> np.ndarray:
    """Q5_1 -> float64 [M][K]: w_e = d * u_e + m, u_e = nibble_e + 16 * bit e of qh.

    EdgeRunner, sections 1.3 and 3.1 (type id 7, 24 bytes: 5-bit codes with an fp16
    bias).  d at 0, m at 2, qh at 4..7, low nibbles at 8..23: adopted GGUF reading.
    """
    blk = _blocks(raw, FMT_Q5_1, M, K)
    d, m = _scale64(blk, 0), _scale64(blk, 2)
    u = (_nibbles(blk[..., 8:24]) + 16 * _high_bits(blk[..., 4:8])).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (d[..., None] * u + m[..., None]).reshape(M, K)


def unpack_f16(raw, M: int, K: int) -> np.ndarray:
    """F16 -> float64 [M][K] (EdgeRunner, section 1.3: type id 1)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(-1)
    if raw.size != M * K * 2:
        raise ValueError("byte count does not match M x K")
    return raw.view("<f2").astype(np.float64).reshape(M, K)


def dequant(fmt: int, raw, M: int, K: int) -> np.ndarray:
    if fmt == FMT_Q8_0:
        return unpack_q8_0(raw, M, K)
    if fmt == FMT_Q4_0:
        return unpack_q4_0(raw, M, K)
    if fmt == FMT_Q4_1:
        return unpack_q4_1(raw, M, K)
    if fmt == FMT_Q5_0:
        return unpack_q5_0(raw, M, K)
    if fmt == FMT_Q5_1:
        return unpack_q5_1(raw, M, K)
    if fmt == FMT_F16:
        return unpack_f16(raw, M, K)
    raise ValueError(f"unknown format {fmt}")


def dequant_rows(fmt: int, raw, K: int, rows) -> np.ndarray:
    """Decode only the listed rows of a large matrix (for sampled checks)."""
    rb = row_bytes(fmt, K)
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
    rows = np.asarray(rows, dtype=np.int64)
    sel = raw.reshape(-1, rb)[rows]
    return dequant(fmt, sel, len(rows), K)


def get_rows_ref(fmt: int, raw, M: int, K: int, ids) -> np.ndarray:
    """Row gather of a quantised matrix: out[i] = W[ids[i]] decoded, float64 [n][K].

    llama.cpp Metal, section 3.2 Input embd (token ids select rows of the
    token-embedding matrix through get_rows) and P8 (one get_rows kernel per
    weight format); EdgeRunner, section 3.4 Tier 3 (embedding rows decoded straight
    into the destination).  An id outside [0, M) gives a NaN row (the library's
    stated behaviour for ids it cannot check on the host).
    """
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.full((ids.size, K), np.nan)
    ok = (ids >= 0) & (ids < M)
    if ok.any():
        out[ok] = dequant_rows(fmt, raw, K, ids[ok])
    return out


def expand_f16_ref(fmt: int, raw, M: int, K: int) -> np.ndarray:
    """Whole-matrix expansion to half precision, float16 [M][K].

    alpaca.swift, Design (quantised matrices expanded into a half-precision buffer
    ahead of the matrix-hardware GEMM); EdgeRunner, section 3.4 Tier 2 (decode
    kernels writing float16).  Each exact decoded weight is rounded once to the
    nearest fp16, ties to even.
    """
    return fp16_round(dequant(fmt, raw, M, K)).astype(np.float16)


# ------------------------------------------------------------------ packing
def pack_q8_0(q: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """Inverse of unpack_q8_0 for codes q int8 [M][K] and fp16 scales [M][K/32]."""
    M, K = q.shape
    out = np.empty((M, K // QK, 34), dtype=np.uint8)
    out[..., 0:2] = np.ascontiguousarray(d16, dtype="<f2").view(np.uint8).reshape(M, K // QK, 2)
    out[..., 2:34] = np.asarray(q, dtype=np.int8).view(np.uint8).reshape(M, K // QK, 32)
    return out.reshape(-1)


def pack_q4_0(n: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """Inverse of unpack_q4_0 for nibbles n in 0..15 [M][K] and fp16 scales [M][K/32]."""
    M, K = n.shape
    n = np.asarray(n, dtype=np.uint8).reshape(M, K // QK, 32)
    if (n > 15).any():
        raise ValueError("nibbles must be in 0..15")
    out = np.empty((M, K // QK, 18), dtype=np.uint8)
    out[..., 0:2] = np.ascontiguousarray(d16, dtype="<f2").view(np.uint8).reshape(M, K // QK, 2)
    out[..., 2:18] = n[..., :16] | (n[..., 16:] << 4)
    return out.reshape(-1)


def _pack_common(fmt, codes, d16, m16, nbits):
    M, K = codes.shape
    u = np.asarray(codes, dtype=np.int64).reshape(M, K // QK, 32)
    if (u < 0).any() or (u >= (1 << nbits)).any():
        raise ValueError(f"codes must be in 0..{(1 << nbits) - 1}")
    bb = BLOCK_BYTES[fmt]
    out = np.zeros((M, K // QK, bb), dtype=np.uint8)
    out[..., 0:2] = np.ascontiguousarray(d16, dtype="<f2").view(np.uint8).reshape(M, K // QK, 2)
    at = 2
    if m16 is not None:
        out[..., 2:4] = np.ascontiguousarray(m16, dtype="<f2").view(np.uint8).reshape(M, K // QK, 2)
        at = 4
    if nbits == 5:
        word = ((u >> 4) << np.arange(32)).sum(axis=-1).astype("<u4")
        out[..., at:at + 4] = word[..., None].view(np.uint8).reshape(M, K // QK, 4)
        at += 4
    lo = u & 15
    out[..., at:at + 16] = (lo[..., :16] | (lo[..., 16:] << 4)).astype(np.uint8)
    return out.reshape(-1)


def pack_q4_1(n: np.ndarray, d16: np.ndarray, m16: np.ndarray) -> np.ndarray:
    """Inverse of unpack_q4_1 for codes n in 0..15 [M][K], fp16 scales and biases [M][K/32]."""
    return _pack_common(FMT_Q4_1, n, d16, m16, 4)


def pack_q5_0(u: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """Inverse of unpack_q5_0 for codes u in 0..31 [M][K] and fp16 scales [M][K/32]."""
    return _pack_common(FMT_Q5_0, u, d16, None, 5)


def pack_q5_1(u: np.ndarray, d16: np.ndarray, m16: np.ndarray) -> np.ndarray:
    """Inverse of unpack_q5_1 for codes u in 0..31 [M][K], fp16 scales and biases [M][K/32]."""
    return _pack_common(FMT_Q5_1, u, d16, m16, 5)


# ------------------------------------------------------------ matmul, SwiGLU
def _w_rows(fmt, raw, M, K, r0, r1):
    rb = row_bytes(fmt, K)
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
    return dequant(fmt, raw[r0 * rb:r1 * rb], r1 - r0, K)


def matmul_ref(fmt: int, raw, x, M: int, K: int, rows=None, chunk_rows: int = 8192):
    """y = x W^T in float64 and S = |x| |W|^T (the scale of the error bound).

    x: [N][K] holding exactly the values the GPU consumed (fp32 for decode, fp16
    for prefill), upcast to float64.  Orientation as in llama.cpp Metal section
    3.2 (K contiguous, tokens as the second operand).  ``rows`` restricts the
    output to selected rows (sampled checks of very large matrices).
    Returns (y, S), each [N][M] (or [N][len(rows)]).
    """
    x64 = np.asarray(x).astype(np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    ax = np.abs(x64)
    if rows is not None:
        W = dequant_rows(fmt, raw, K, rows)
        return x64 @ W.T, ax @ np.abs(W).T
    N = x64.shape[0]
    y = np.empty((N, M))
    S = np.empty((N, M))
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        W = _w_rows(fmt, raw, M, K, r0, r1)
        y[:, r0:r1] = x64 @ W.T
        S[:, r0:r1] = ax @ np.abs(W).T
    return y, S


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z) (EdgeRunner, section 8 SwiGLU FFN)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gate_up_silu_ref(fmt: int, raw_g, raw_u, x, I: int, K: int, rows=None):
    """h = silu(x Wg^T) * (x Wu^T) with its error scales.

    EdgeRunner, section 8: the SwiGLU output is SiLU of the gate projection times
    the up projection.  Returns (h, g, u, Sg, Su).
    """
    g, Sg = matmul_ref(fmt, raw_g, x, I, K, rows=rows)
    u, Su = matmul_ref(fmt, raw_u, x, I, K, rows=rows)
    return silu(g) * u, g, u, Sg, Su


def rmsnorm_ref(x, gamma, eps: float):
    """RMSNorm of each token row: x / sqrt(mean_k x_k^2 + eps) * gamma, float64 [N][K].

    EdgeRunner, section 6 RMSNorm: the input times the inverse of its root mean
    square, times the norm weight; the epsilon is a parameter of the norm (the
    model configuration gives 1e-5 as an example).  Reading where the page is
    silent: eps is added to the mean square inside the square root, and Llama-style
    norms carry no bias.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    ms = np.mean(x64 * x64, axis=1, keepdims=True)
    return x64 / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)[None, :]


def rmsnorm_matmul_ref(fmt: int, raw, x, gamma, eps: float, M: int, K: int, rows=None):
    """RMSNorm prologue fused with a projection: y = rmsnorm(x) W^T, with S of the
    normalised input (EdgeRunner, section 2.1 and section 9.2: the attention norm
    folded into the fused QKV GEMV, the final norm into the LM head)."""
    return matmul_ref(fmt, raw, rmsnorm_ref(x, gamma, eps), M, K, rows=rows)


def rmsnorm_gate_up_silu_ref(fmt: int, raw_g, raw_u, x, gamma, eps: float, I: int, K: int, rows=None):
    """FFN norm folded into gate+up+SwiGLU (EdgeRunner, section 8: one dispatch for
    RMSNorm, gate, up and SiLU at a single token)."""
    return gate_up_silu_ref(fmt, raw_g, raw_u, rmsnorm_ref(x, gamma, eps), I, K, rows=rows)


def matmul_add_ref(fmt: int, raw, x, r, M: int, K: int, rows=None):
    """Residual-add epilogue: y = x W^T + r (EdgeRunner, section 9.1 steps 13-14 and
    section 9.2: the O and down projections add into the residual stream)."""
    y, S = matmul_ref(fmt, raw, x, M, K, rows=rows)
    r64 = np.asarray(r, dtype=np.float64)
    if r64.ndim == 1:
        r64 = r64[None, :]
    if rows is not None:
        r64 = r64[:, rows]
    return y + r64, S


# ---------------------------------------------------------------- tolerances
def tol_linear(S):
    """Allowed |y_gpu - y_ref| for a linear output: 2e-3 * S + 1e-6."""
    return TOL_REL * np.asarray(S) + TOL_ABS


def tol_residual(S, y):
    """Allowed error of y = x W^T + r: the linear bound for the product plus the
    fp32 rounding of the final addition (one rounding, at most 2^-24 |y|; 2^-23 |y|
    is allowed)."""
    return tol_linear(S) + 2.0 ** -23 * np.abs(np.asarray(y))


SILU_SLOPE_MAX = 1.1   # max |silu'(z)| = 1.0998 near z = 2.40


def tol_swiglu(g, u, Sg, Su):
    """Allowed |h_gpu - h_ref| for h = silu(g) * u when g and u each obey tol_linear.

    With |g~ - g| <= Eg and |u~ - u| <= Eu:
      |silu(g~) u~ - silu(g) u| <= |silu(g~) - silu(g)| |u~| + |silu(g)| |u~ - u|
                                 <= 1.1 Eg (|u| + Eu) + |silu(g)| Eu,
    plus a relative 1e-6 |h| + 1e-6 for the fp32 epilogue itself.
    """
    Eg = tol_linear(Sg)
    Eu = tol_linear(Su)
    h = silu(g) * u
    return SILU_SLOPE_MAX * Eg * (np.abs(u) + Eu) + np.abs(silu(g)) * Eu + 1e-6 * np.abs(h) + 1e-6


def fp16_round(w):
    """Round float64 values to the nearest fp16 (ties to even), back to float64.

    Used to state what a prefill GEMM tile holds: fp16(d * q).
    """
    return np.asarray(w, dtype=np.float64).astype(np.float16).astype(np.float64)


# ----------------------------------------------------------- plain reference
def brute_force_matmul(fmt: int, raw: bytes, x_rows, M: int, K: int):
    """Exact rational y = x W^T with pure-Python loops (tiny shapes only).

    Decodes each block byte by byte from the format definition (no numpy) and
    accumulates with fractions.Fraction, so the result has no rounding at all.
    """
    from fractions import Fraction

    def f16(lo, hi):
        h = lo | (hi << 8)
        s = -1 if h >> 15 else 1
        e = (h >> 10) & 31
        m = h & 1023
        if e == 0:
            return s * Fraction(m, 1 << 24)
        if e == 31:
            raise ValueError("inf/nan scale")
        return s * Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15)

    raw = bytes(raw)
    rb = row_bytes(fmt, K)
    W = []
    for m in range(M):
        row = raw[m * rb:(m + 1) * rb]
        w = []
        if fmt == FMT_F16:
            for k in range(K):
                w.append(f16(row[2 * k], row[2 * k + 1]))
        else:
            bb = BLOCK_BYTES[fmt]
            for b in range(K // QK):
                blk = row[b * bb:(b + 1) * bb]
                d = f16(blk[0], blk[1])
                if fmt == FMT_Q8_0:
                    for i in range(32):
                        q = blk[2 + i]
                        w.append(d * (q - 256 if q >= 128 else q))
                    continue
                # Every other block format: [d][m if biased][qh if 5-bit][16 nibble bytes].
                biased = fmt in (FMT_Q4_1, FMT_Q5_1)
                five = fmt in (FMT_Q5_0, FMT_Q5_1)
                m = f16(blk[2], blk[3]) if biased else 0
                pos = 4 if biased else 2
                qh = 0
                if five:
                    qh = blk[pos] + 256 * blk[pos + 1] + 65536 * blk[pos + 2] + 16777216 * blk[pos + 3]
                    pos += 4
                codes = [0] * 32
                for j in range(16):
                    codes[j] = blk[pos + j] % 16
                    codes[j + 16] = blk[pos + j] // 16
                for e in range(32):
                    u = codes[e] + (16 if five and (qh // 2 ** e) % 2 else 0)
                    if fmt == FMT_Q4_0:
                        w.append(d * (u - 8))
                    elif fmt == FMT_Q5_0:
                        w.append(d * (u - 16))
                    else:
                        w.append(d * u + m)
        W.append(w)
    out = []
    for xr in x_rows:
        xf = [Fraction(float(v)) for v in xr]
        out.append([sum(W[m][k] * xf[k] for k in range(K)) for m in range(M)])
    return out
