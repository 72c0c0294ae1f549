"""GPU parity of the Q4_1, Q5_0 and Q5_1 paths against the float64 oracle.

* Element-wise decoders: qmm_dequant and qmm_get_rows must equal the oracle's exact
  weights rounded once to fp32, bit for bit (for the biased formats d*u + m needs more
  than 24 bits, so this pins a single rounding); qmm_expand_f16 must equal the exact
  weights rounded once to fp16 (the tiny-bias golden block would round differently
  through fp32).  Hand-computed golden blocks go through both.
* Decode products on the register-decode kernels:
  plain GEMV at shapes that cover the streaming kernel (a K slice of 128 blocks, a
  partial slice, many row groups, 1..4 tokens per pass and a second pass), its
  fallback for the final row when the matrix size is not a multiple of 16 bytes, and
  the sliced kernel when x does not fit in LDS (K = 65536); the gated, RMSNorm and
  residual products; x = e_k returning the decoded column exactly.
* MFMA products: the prefill GEMM on its tiled kernel (K % 256 == 0: 128- and
  256-token tiles, split K, the gated epilogue) and on the generic one (other K),
  with X = e_k returning fp16 of the exact weight bit for bit; the small-batch MFMA
  GEMV (2..32 tokens, split K) and its tiled hand-off above 32 tokens.
Outputs are poisoned with NaNs and followed by a guard band.
"""
import os

import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import (announce, check_linear, check_residual, check_swiglu, dev, guard_intact, poisoned,
                         sample_rows)
from test_oracle import GOLDEN_FILES, load_golden

pytestmark = pytest.mark.gpu
FMTS = [si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1]
FID = {si.FMT_Q4_1: "q4_1", si.FMT_Q5_0: "q5_0", si.FMT_Q5_1: "q5_1"}
VALU, MFMA = qmm.QMM_VARIANT_VALU, qmm.QMM_VARIANT_MFMA


def _bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


# ------------------------------------------------------------ element-wise
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("mode", ["uniform", "wide"])
@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (300, 576), (33, 4096)])
def test_dequant_bit_exact(fmt, mode, M, K):
    seed = 7000 + fmt * 100 + M + K
    raw = si.weights(fmt, M, K, seed, scale_mode=mode)
    announce(f"dequant fmt={fmt} mode={mode} M={M} K={K}")
    got = qmm.dequant(fmt, dev(raw), M, K).cpu().numpy()
    want = oracle.dequant(fmt, raw, M, K).astype(np.float32)
    assert np.array_equal(_bits32(got), _bits32(want))


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("mode", ["uniform", "wide", "gemm_wide"])
@pytest.mark.parametrize("M,K", [(1, 32), (5, 160), (257, 4096)])
def test_expand_f16_bit_exact(fmt, mode, M, K):
    seed = 7100 + fmt * 100 + M + K
    raw = si.weights(fmt, M, K, seed, scale_mode=mode)
    announce(f"expand_f16 fmt={fmt} mode={mode} M={M} K={K}")
    got = qmm.expand_f16(fmt, dev(raw), M, K).cpu().numpy()
    want = oracle.expand_f16_ref(fmt, raw, M, K)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


NEW_GOLDEN = [p for p in GOLDEN_FILES if load_golden(p)["fmt"] in FMTS]


@pytest.mark.parametrize("path", NEW_GOLDEN, ids=os.path.basename)
def test_golden_blocks_gpu(path):
    fx = load_golden(path)
    raw = np.frombuffer(fx["bytes"], np.uint8)
    announce(f"golden {os.path.basename(path)}")
    w = qmm.dequant(fx["fmt"], dev(raw), 1, 32).cpu().numpy()[0]
    h = qmm.expand_f16(fx["fmt"], dev(raw), 1, 32).cpu().numpy()[0]
    for k in range(32):
        exact = float(fx["w"].get(k, 0))
        assert w[k] == np.float32(exact), (k, w[k], exact)
        want_h = float(fx.get("h", {}).get(k, fx["w"].get(k, 0)))
        assert float(h[k]) == want_h, (k, float(h[k]), want_h)


def test_golden_count():
    assert {load_golden(p)["fmt"] for p in NEW_GOLDEN} == set(FMTS)


def _special_blocks(fmt):
    """Blocks whose scale or bias is inf, -inf, NaN or zero, or whose d * u + m overflows
    fp16: codes 0..15 (4-bit) or 0..31 (5-bit) repeated."""
    M, K = 3, 64
    d = np.array([[np.inf, -np.inf], [np.nan, 0.0], [1.0, 65504.0]], dtype=np.float16)
    m = np.array([[0.0, 1.0], [0.0, np.inf], [-np.inf, -65504.0]], dtype=np.float16)
    bits = 4 if fmt == si.FMT_Q4_1 else 5
    u = np.tile(np.arange(64, dtype=np.int64) % (1 << bits), (M, 1))
    if fmt == si.FMT_Q4_1:
        raw = oracle.pack_q4_1(u, d, m)
    elif fmt == si.FMT_Q5_0:
        raw = oracle.pack_q5_0(u, d)
    else:
        raw = oracle.pack_q5_1(u, d, m)
    return raw, M, K


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_special_scales_and_biases(fmt):
    """IEEE propagation through dequant, gather and fp16 expansion: inf * 0 and
    inf - inf give NaN, overflow gives inf, the rest are values rounded once."""
    raw, M, K = _special_blocks(fmt)
    announce(f"special scales fmt={fmt}")
    W = dev(raw)
    ref = oracle.dequant(fmt, raw, M, K)
    nan = np.isnan(ref)
    for got in (qmm.dequant(fmt, W, M, K).cpu().numpy(),
                qmm.get_rows(fmt, W, dev(np.arange(M, dtype=np.int32)), M, K).cpu().numpy()):
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(_bits32(got[~nan]), _bits32(ref[~nan].astype(np.float32)))
    h = qmm.expand_f16(fmt, W, M, K).cpu().numpy()
    href = oracle.expand_f16_ref(fmt, raw, M, K)
    hnan = np.isnan(href)
    assert np.array_equal(np.isnan(h), hnan)
    assert np.array_equal(h[~hnan].view(np.uint16), href[~hnan].view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_get_rows_bit_exact(fmt):
    M, K = 1000, 576
    raw = si.weights(fmt, M, K, 7200 + fmt, scale_mode="wide")
    ids = np.array([0, 999, 5, 5, 512, -1, 1000, 77], dtype=np.int32)
    announce(f"get_rows fmt={fmt}")
    got = qmm.get_rows(fmt, dev(raw), dev(ids), M, K).cpu().numpy()
    want = oracle.get_rows_ref(fmt, raw, M, K, ids).astype(np.float32)
    ok = (ids >= 0) & (ids < M)
    assert np.array_equal(_bits32(got[ok]), _bits32(want[ok]))
    assert np.isnan(got[~ok]).all()


# ------------------------------------------------------------ decode GEMV
GEMV_CASES = [
    (3, 32, 1),        # one block; 3 rows of 20-24 bytes: the last row goes to the sliced kernel
    (257, 576, 1),     # 18 blocks per row (a partial K slice)
    (257, 576, 3),
    (1000, 4096, 2),   # one 128-block slice per row
    (4099, 4096, 1),   # many row groups, ragged
    (300, 14336, 4),   # 4 tokens, x 35 KB per token
    (129, 2048, 6),    # two passes (4 + 2 tokens)
    (40, 65536, 1),    # x does not fit in LDS: the sliced kernel
    (20000, 1024, 1),  # 2-row tasks (M >= 16384)
]


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", GEMV_CASES)
def test_gemv(fmt, M, K, N):
    seed = 7300 + fmt * 1000 + M + K + N
    raw = si.weights(fmt, M, K, seed)
    x = si.activations(N, K, seed + 1)
    announce(f"gemv fmt={fmt} M={M} K={K} N={N} seed={seed}")
    buf = poisoned(N * M)
    qmm.qmm_gemv(fmt, dev(raw), dev(x), buf, M, K, N)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * M)
    got = buf[:N * M].cpu().numpy().reshape(N, M)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(got, y_ref, S, f"gemv fmt={fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_gemv_wide_scales(fmt):
    """Scales and biases drawn from every finite fp16 pattern (subnormals, both signs)."""
    M, K, N = 515, 2304, 2
    raw = si.weights(fmt, M, K, 7400 + fmt, scale_mode="wide")
    x = si.activations(N, K, 7401 + fmt)
    announce(f"gemv wide fmt={fmt}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K).cpu().numpy()
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(y, y_ref, S, f"gemv wide fmt={fmt}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("K", [4096, 65536])
def test_gemv_one_hot_exact(fmt, K):
    """x = e_k returns the decoded column rounded once to fp32 (both kernels).  Compared
    as values: a zero weight of negative scale is -0 in the column, while the sum over
    k of w_k x_k (with +0 terms) is +0."""
    M = 301
    raw = si.weights(fmt, M, K, 7500 + fmt, scale_mode="gemm_wide")
    cols = [0, 31, 2047, K - 1]
    x = si.one_hot(len(cols), K, cols)
    announce(f"gemv one-hot fmt={fmt} K={K}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=VALU).cpu().numpy()
    W = oracle.dequant(fmt, raw, M, K).astype(np.float32)
    for n, c in enumerate(cols):
        assert np.array_equal(y[n], W[:, c]), (n, c)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,N", [(3, 32, 1), (1536, 576, 1), (1000, 4096, 2), (129, 14336, 1)])
def test_gate_up_silu(fmt, I, K, N):
    seed = 7600 + fmt * 100 + I + K + N
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    x = si.activations(N, K, seed + 2)
    announce(f"gate_up_silu fmt={fmt} I={I} K={K} N={N}")
    buf = poisoned(N * I)
    qmm.qmm_gate_up_silu(fmt, dev(rg), dev(ru), dev(x), buf, I, K, N)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    check_swiglu(buf[:N * I].cpu().numpy().reshape(N, I), h_ref, g, u, Sg, Su, "gate_up_silu")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(257, 576, 1), (4100, 4096, 2)])
def test_rmsnorm_gemv(fmt, M, K, N):
    seed = 7700 + fmt * 100 + M + K + N
    raw = si.weights(fmt, M, K, seed)
    x = si.activations(N, K, seed + 1)
    gamma = (1.0 + 0.25 * si.activations(1, K, seed + 2)[0]).astype(np.float32)
    announce(f"rmsnorm_gemv fmt={fmt} M={M} K={K} N={N}")
    y = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), 1e-5, M, K)
    torch.cuda.synchronize()
    y_ref, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, 1e-5, M, K)
    check_linear(y.cpu().numpy(), y_ref, S, "rmsnorm_gemv")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(576, 1536, 1), (4096, 14336, 1), (4099, 4096, 3)])
@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
def test_gemv_add(fmt, M, K, N, inplace):
    seed = 7800 + fmt * 100 + M + K + N
    raw = si.weights(fmt, M, K, seed)
    x = si.activations(N, K, seed + 1)
    r = (si.activations(N, M, seed + 2) * 100.0).astype(np.float32)
    rd = dev(r)
    announce(f"gemv_add fmt={fmt} M={M} K={K} N={N} inplace={inplace}")
    y = qmm.gemv_add(fmt, dev(raw), dev(x), rd, M, K, out=rd if inplace else None)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_add_ref(fmt, raw, x, r, M, K)
    check_residual(y.cpu().numpy(), y_ref, S, "gemv_add")
    if not inplace:
        assert np.array_equal(rd.cpu().numpy(), r), "the residual input must not change"


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_gemv_llama3_8b_down_sampled(fmt):
    """The 8B down projection (4096 x 14336) at its full size; sampled rows against the oracle."""
    M, K = 4096, 14336
    raw = si.weights(fmt, M, K, 7900 + fmt)
    x = si.activations(1, K, 7901 + fmt)
    announce(f"gemv 8B down fmt={fmt}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K).cpu().numpy()
    rows = sample_rows(M, 64, 7902 + fmt)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
    check_linear(y[:, rows], y_ref, S, f"gemv 8B down fmt={fmt}")


# ------------------------------------------------------------ MFMA products
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,T", [(1, 32, 1), (300, 256, 40), (256, 4096, 256), (513, 96, 300), (64, 4160, 17),
                                   (130, 4096, 129), (300, 2816, 40), (64, 14336, 130)])
def test_gemm(fmt, M, K, T):
    """K % 256 == 0: the tiled kernel (2816 and 14336 split K over workgroups); other K:
    the generic kernel."""
    seed = 8000 + fmt * 1000 + M + K + T
    mode = "gemm_wide" if T % 2 else "uniform"
    raw = si.weights(fmt, M, K, seed, scale_mode=mode)
    X = si.activations(T, K, seed + 1, dtype=np.float16)
    announce(f"qmm_gemm fmt={fmt} M={M} K={K} T={T} seed={seed} mode={mode}")
    buf = poisoned(T * M)
    qmm.qmm_gemm(fmt, dev(raw), dev(X), buf, M, K, T)
    torch.cuda.synchronize()
    assert guard_intact(buf, T * M)
    y_ref, S = oracle.matmul_ref(fmt, raw, X, M, K)
    check_linear(buf[:T * M].cpu().numpy().reshape(T, M), y_ref, S, f"gemm fmt={fmt} M={M} K={K} T={T}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("K", [4096, 4160])
def test_gemm_one_hot_fp16(fmt, K):
    """X = e_k gives the exact weight rounded once to fp16 (what qmm_expand_f16 writes),
    on the tiled kernel (K = 4096) and the generic one (K = 4160)."""
    M = 300
    raw = si.weights(fmt, M, K, 8100 + fmt, scale_mode="gemm_wide")
    cols = list(range(0, K, 97)) + [K - 1]
    X = si.one_hot(len(cols), K, cols, dtype=np.float16)
    announce(f"gemm one-hot fmt={fmt} K={K}")
    Y = qmm.gemm(fmt, dev(raw), dev(X), M, K)
    torch.cuda.synchronize()
    H = oracle.expand_f16_ref(fmt, raw, M, K).astype(np.float64)
    Yc = Y.cpu().numpy().astype(np.float64)
    for t, c in enumerate(cols):
        assert np.array_equal(Yc[t], H[:, c]), (t, c)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,T", [(128, 256, 64), (200, 4096, 300), (64, 96, 7), (130, 4096, 9)])
def test_gemm_gate_up_silu(fmt, I, K, T):
    seed = 8200 + fmt * 100 + I + K + T
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    X = si.activations(T, K, seed + 2, dtype=np.float16)
    announce(f"qmm_gemm_gate_up_silu fmt={fmt} I={I} K={K} T={T}")
    buf = poisoned(T * I)
    qmm.qmm_gemm_gate_up_silu(fmt, dev(rg), dev(ru), dev(X), buf, I, K, T)
    torch.cuda.synchronize()
    assert guard_intact(buf, T * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, X, I, K)
    check_swiglu(buf[:T * I].cpu().numpy().reshape(T, I), h_ref, g, u, Sg, Su, f"gemm gate_up fmt={fmt}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(300, 2048, 5), (1000, 4096, 17), (33, 256, 32), (513, 14336, 9),
                                   (257, 2048, 128)])
def test_gemv_mfma(fmt, M, K, N):
    """2..32 tokens: the weight-streaming MFMA GEMV; 128: the tiled GEMM on fp32 x."""
    seed = 8300 + fmt * 100 + M + K + N
    raw = si.weights(fmt, M, K, seed, scale_mode="gemm_wide")
    x = si.activations(N, K, seed + 1)
    announce(f"gemv mfma fmt={fmt} M={M} K={K} N={N} seed={seed}")
    buf = poisoned(N * M)
    qmm.qmm_gemv_variant(fmt, dev(raw), dev(x), buf, M, K, N, MFMA)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * M)
    # The oracle takes the caller's fp32 x; the kernels scale and round it to fp16 themselves.
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(buf[:N * M].cpu().numpy().reshape(N, M), y_ref, S, f"gemv mfma fmt={fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,N", [(300, 4096, 3), (1000, 4096, 8)])
def test_gate_up_silu_mfma(fmt, I, K, N):
    seed = 8400 + fmt * 100 + I + K + N
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    x = si.activations(N, K, seed + 2)
    announce(f"gate_up_silu mfma fmt={fmt} I={I} K={K} N={N}")
    buf = poisoned(N * I)
    qmm.qmm_gate_up_silu_variant(fmt, dev(rg), dev(ru), dev(x), buf, I, K, N, MFMA)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    check_swiglu(buf[:N * I].cpu().numpy().reshape(N, I), h_ref, g, u, Sg, Su, "gate_up_silu mfma")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_gemv_llama3_8b_lm_head_sampled(fmt):
    """The 128256 x 4096 LM head (2-row DMA tasks) at its full size, one token; sampled
    rows against the oracle, and every output finite."""
    M, K = 128256, 4096
    raw = si.weights(fmt, M, K, 7950 + fmt)
    x = si.activations(1, K, 7951 + fmt)
    announce(f"gemv 8B LM head fmt={fmt}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K).cpu().numpy()
    assert np.isfinite(y).all()
    rows = sample_rows(M, 96, 7952 + fmt)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
    check_linear(y[:, rows], y_ref, S, f"gemv 8B LM head fmt={fmt}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_gate_up_llama3_8b_sampled(fmt):
    """Gate+up + SwiGLU at 2 x 14336 x 4096, one token; sampled outputs."""
    I, K = 14336, 4096
    rg, ru = si.weights(fmt, I, K, 7960 + fmt), si.weights(fmt, I, K, 7961 + fmt)
    x = si.activations(1, K, 7962 + fmt)
    announce(f"gate_up 8B fmt={fmt}")
    h = qmm.gate_up_silu(fmt, dev(rg), dev(ru), dev(x), I, K).cpu().numpy()
    assert np.isfinite(h).all()
    rows = sample_rows(I, 96, 7963 + fmt)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K, rows=rows)
    check_swiglu(h[:, rows], h_ref, g, u, Sg, Su, f"gate_up 8B fmt={fmt}")
