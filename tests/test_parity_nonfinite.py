"""GPU: inf and NaN block scales (and biases) through the products.

The fp16 scale of a block is decoded as IEEE binary16 ("EdgeRunner Core
Architecture", section 1.3 and sections 3.1-3.2), so an inf or NaN scale gives
non-finite weights, and a product over a row holding one is non-finite too.  Whether
it comes out as inf or as NaN depends on the order of the sums (the oracle adds
w_k x_k element by element, the kernels factor each block's scale out of its sum),
so the check is: every output of such a row is non-finite, in the oracle and on the
GPU, and every other row stays within the usual bound.  Outputs start as a finite
sentinel, so an element a kernel failed to write fails the check.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_swiglu, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")]  # the oracle's NaN rows
BLOCK_FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1]
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_Q4_1: "q4_1", si.FMT_Q5_0: "q5_0", si.FMT_Q5_1: "q5_1"}
BIASED = (si.FMT_Q4_1, si.FMT_Q5_1)
SPECIAL = (0x7C00, 0xFC00, 0x7E00)  # +inf, -inf, NaN (fp16 bits)
SENTINEL = 777.0
VALU, MFMA = qmm.QMM_VARIANT_VALU, qmm.QMM_VARIANT_MFMA


def _with_specials(fmt, M, K, seed, nrows=7):
    """Seeded weights with an inf / NaN scale in one block of a few rows (and, for the
    biased formats, a NaN bias in one more row).  Returns (raw, rows)."""
    raw = si.weights(fmt, M, K, seed).copy()
    bb = oracle.BLOCK_BYTES[fmt]
    nb = K // 32
    blocks = raw.reshape(M, nb, bb)
    g = np.random.Generator(np.random.PCG64(seed + 17))
    rows = sorted(set([0, M - 1, M // 2] + g.choice(M, size=nrows, replace=False).tolist()))
    for i, r in enumerate(rows):
        b = int(g.integers(0, nb))
        at = 2 if (fmt in BIASED and i == len(rows) - 1) else 0  # the last row: a NaN bias
        bits = 0x7E00 if at == 2 else SPECIAL[i % len(SPECIAL)]
        blocks[r, b, at:at + 2] = np.array([bits & 0xFF, bits >> 8], dtype=np.uint8)
    return raw, np.array(rows)


def _filled(shape):
    return torch.full(shape, SENTINEL, dtype=torch.float32, device="cuda")


def _check(got, y_ref, S, rows, what):
    got = np.asarray(got, dtype=np.float64)
    keep = np.ones(got.shape[-1], dtype=bool)
    keep[rows] = False
    assert not np.isfinite(y_ref[:, rows]).any(), f"{what}: oracle rows with special blocks are finite"
    assert np.isfinite(y_ref[:, keep]).all()
    assert not np.isfinite(got[:, rows]).any(), f"{what}: a row with an inf/NaN block came out finite"
    check_linear(got[:, keep], y_ref[:, keep], S[:, keep], what)


# (M, K, N, variant): the register-staged kernel on a small matrix, the DMA-fed kernel
# (more than 2048 rows, K % 256 == 0) at 1 and 3 tokens, a partial K slice, and the
# small-batch MFMA kernel.
GEMV_CASES = [(300, 4096, 1, VALU), (3000, 4096, 1, VALU), (3000, 4096, 3, VALU), (257, 576, 2, VALU),
              (3000, 4096, 8, MFMA)]


@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N,variant", GEMV_CASES)
def test_gemv_nonfinite_rows(fmt, M, K, N, variant):
    seed = 9100 + 100 * fmt + N
    raw, rows = _with_specials(fmt, M, K, seed)
    x = si.activations(N, K, seed + 1)
    what = f"gemv nonfinite fmt={fmt} M={M} K={K} N={N} variant={variant}"
    announce(what)
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, out=_filled((N, M)), variant=variant)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    _check(y.cpu().numpy(), y_ref, S, rows, what)


@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=FID.get)
@pytest.mark.parametrize("N,variant", [(1, VALU), (8, MFMA)])
def test_gate_up_nonfinite_rows(fmt, N, variant):
    """Special blocks in some gate rows and in other up rows: h is non-finite exactly there."""
    I, K = 1000, 4096
    seed = 9300 + 100 * fmt + N
    raw_g, rows_g = _with_specials(fmt, I, K, seed, nrows=4)
    raw_u, rows_u = _with_specials(fmt, I, K, seed + 50, nrows=4)
    x = si.activations(N, K, seed + 1)
    what = f"gate_up nonfinite fmt={fmt} N={N} variant={variant}"
    announce(what)
    h = qmm.gate_up_silu(fmt, dev(raw_g), dev(raw_u), dev(x), I, K, out=_filled((N, I)), variant=variant)
    torch.cuda.synchronize()
    h = h.cpu().numpy().astype(np.float64)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, raw_g, raw_u, x, I, K)
    rows = np.union1d(rows_g, rows_u)
    keep = np.ones(I, dtype=bool)
    keep[rows] = False
    assert not np.isfinite(h_ref[:, rows]).any() and np.isfinite(h_ref[:, keep]).all()
    assert not np.isfinite(h[:, rows]).any(), what
    check_swiglu(h[:, keep], h_ref[:, keep], g[:, keep], u[:, keep], Sg[:, keep], Su[:, keep], what)


# (M, K, T): the tiled kernel (K % 256 == 0) and the generic one.
@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,T", [(600, 4096, 64), (300, 576, 40)])
def test_gemm_nonfinite_rows(fmt, M, K, T):
    seed = 9500 + 100 * fmt + T
    raw, rows = _with_specials(fmt, M, K, seed)
    X = si.activations(T, K, seed + 1, dtype=np.float16)
    what = f"gemm nonfinite fmt={fmt} M={M} K={K} T={T}"
    announce(what)
    Y = qmm.gemm(fmt, dev(raw), dev(X), M, K, out=_filled((T, M)))
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_ref(fmt, raw, X, M, K)
    _check(Y.cpu().numpy(), y_ref, S, rows, what)


@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=FID.get)
def test_gemm_gate_up_nonfinite_rows(fmt):
    I, K, T = 600, 4096, 64
    seed = 9700 + 100 * fmt
    raw_g, rows_g = _with_specials(fmt, I, K, seed, nrows=4)
    raw_u, rows_u = _with_specials(fmt, I, K, seed + 50, nrows=4)
    X = si.activations(T, K, seed + 1, dtype=np.float16)
    what = f"gemm gate_up nonfinite fmt={fmt}"
    announce(what)
    H = qmm.gemm_gate_up_silu(fmt, dev(raw_g), dev(raw_u), dev(X), I, K, out=_filled((T, I)))
    torch.cuda.synchronize()
    H = H.cpu().numpy().astype(np.float64)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, raw_g, raw_u, X, I, K)
    rows = np.union1d(rows_g, rows_u)
    keep = np.ones(I, dtype=bool)
    keep[rows] = False
    assert not np.isfinite(h_ref[:, rows]).any() and np.isfinite(h_ref[:, keep]).all()
    assert not np.isfinite(H[:, rows]).any(), what
    check_swiglu(H[:, keep], h_ref[:, keep], g[:, keep], u[:, keep], Sg[:, keep], Su[:, keep], what)
