"""GPU parity of the register-decode GEMVs on inputs that stress their arithmetic.

* Near-offset blocks (tests/near_offset.py): every weight at its format's zero code
  but one unit step per block, x = 1 except a small eps at those steps.  sum |w x| is
  tiny against sum |x|, so any offset carried through the sums (or a bias factored
  out of them) misses the bound; the exact-code dot products must meet it.  Every
  block format, 1..4 tokens, on the DMA-fed kernel (16-byte aligned rows, more than
  2048 rows), on the register-staged kernel (small matrices; 2-byte aligned rows at
  K = 576, whose final row goes to the sliced kernel), and through every entry point
  that runs them: qmm_gemv, qmm_gate_up_silu, qmm_rmsnorm_gemv,
  qmm_rmsnorm_gate_up_silu and qmm_gemv_add.
* Wide blocks: x blocks whose dynamic range exceeds what block floating point in
  fp16 keeps (a 1e20 beside ones, a single 1e15 outlier), which switch the kernels
  to fp32 x: re-staged in LDS where it fits, else read from global memory (two
  tokens at K = 14336); and x far outside the fp16 range in either direction (1e30,
  1e-35, fp32 subnormals), which block scaling alone handles.
Checked against the float64 oracle with |y - y_ref| <= 2e-3 sum |w x| + 1e-6
(the fused outputs with their propagated bounds); outputs start as NaN.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import near_offset
import oracle
import seeded_inputs as si
from parity_util import (announce, check_linear, check_residual, check_swiglu, dev, guard_intact, poisoned,
                         sample_rows)

pytestmark = pytest.mark.gpu
ALL_FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1]
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_Q4_1: "q4_1", si.FMT_Q5_0: "q5_0", si.FMT_Q5_1: "q5_1"}
VALU = qmm.QMM_VARIANT_VALU
# (M, K): DMA-fed kernel; register-staged kernel; register-staged with 2-byte aligned rows.
SHAPES = [(2304, 4096), (300, 4096), (301, 576)]


def _gemv(fmt, raw, x, M, K, variant):
    N = x.shape[0]
    buf = poisoned(N * M)
    qmm.qmm_gemv_variant(fmt, dev(raw), dev(x), buf, M, K, N, variant)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * M)
    return buf[:N * M].cpu().numpy().reshape(N, M)


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 4])
def test_near_offset_gemv(fmt, M, K, N):
    raw = near_offset.weights(fmt, M, K)
    x = near_offset.activations(N, K)
    announce(f"near-offset gemv fmt={fmt} M={M} K={K} N={N}")
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(_gemv(fmt, raw, x, M, K, VALU), y_ref, S, f"near-offset gemv fmt={fmt} M={M} K={K} N={N}")
    check_linear(_gemv(fmt, raw, x, M, K, qmm.QMM_VARIANT_AUTO), y_ref, S, "near-offset gemv (auto)")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K", [(2304, 4096), (300, 576)])
@pytest.mark.parametrize("N", [1, 4])
def test_near_offset_gate_up_silu(fmt, I, K, N):
    rg = near_offset.weights(fmt, I, K)
    ru = np.roll(rg.reshape(I, -1), 1, axis=0).reshape(-1)  # up row r = gate row r - 1
    x = near_offset.activations(N, K)
    announce(f"near-offset gate_up_silu fmt={fmt} I={I} K={K} N={N}")
    buf = poisoned(N * I)
    qmm.qmm_gate_up_silu_variant(fmt, dev(rg), dev(ru), dev(x), buf, I, K, N, VALU)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    check_swiglu(buf[:N * I].cpu().numpy().reshape(N, I), h_ref, g, u, Sg, Su, "near-offset gate_up_silu")


def _gamma(K, seed):
    return np.random.default_rng(seed).uniform(0.5, 1.5, K).astype(np.float32)


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 3])
def test_near_offset_rmsnorm_gemv(fmt, M, K, N):
    raw = near_offset.weights(fmt, M, K)
    x = near_offset.activations(N, K)
    gamma = _gamma(K, 3)
    announce(f"near-offset rmsnorm_gemv fmt={fmt} M={M} K={K} N={N}")
    y = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), 1e-5, M, K)
    torch.cuda.synchronize()
    y_ref, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, 1e-5, M, K)
    check_linear(y.cpu().numpy(), y_ref, S, "near-offset rmsnorm_gemv")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("N", [1, 2])
def test_near_offset_rmsnorm_gate_up_silu(fmt, N):
    I, K = 2304, 4096
    rg = near_offset.weights(fmt, I, K)
    ru = np.roll(rg.reshape(I, -1), 3, axis=0).reshape(-1)
    x = near_offset.activations(N, K)
    gamma = _gamma(K, 4)
    announce(f"near-offset rmsnorm_gate_up_silu fmt={fmt} N={N}")
    h = qmm.rmsnorm_gate_up_silu(fmt, dev(rg), dev(ru), dev(x), dev(gamma), 1e-5, I, K)
    torch.cuda.synchronize()
    h_ref, g, u, Sg, Su = oracle.rmsnorm_gate_up_silu_ref(fmt, rg, ru, x, gamma, 1e-5, I, K)
    check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, "near-offset rmsnorm_gate_up_silu")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 4])
def test_near_offset_gemv_add(fmt, M, K, N):
    raw = near_offset.weights(fmt, M, K)
    x = near_offset.activations(N, K)
    r = si.activations(N, M, 9)
    announce(f"near-offset gemv_add fmt={fmt} M={M} K={K} N={N}")
    y = qmm.gemv_add(fmt, dev(raw), dev(x), dev(r), M, K)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_add_ref(fmt, raw, x, r, M, K)
    check_residual(y.cpu().numpy(), y_ref, S, "near-offset gemv_add")


# ---------------------------------------------------------------- wide blocks
def _wide_near(N, K):
    """Near-offset x with 1e20 at position 1 of every block (a zero weight there):
    the eps and the ones fall 2^52+ below their block's largest."""
    x = near_offset.activations(N, K)
    x[:, 1::32] = 1e20
    return x


def _wide_tiny(N, K):
    """Near-offset x with 1e-30 at position 1 of every block (a zero weight there):
    every block is wide while the RMS of x stays near 1."""
    x = near_offset.activations(N, K)
    x[:, 1::32] = 1e-30
    return x


def _outlier(N, K, seed):
    """N(0, 1) x with one 1e15 in block 3 of the last token: one wide block."""
    x = si.activations(N, K, seed)
    x[-1, 3 * 32 + 7] = 1e15
    return x


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 4])
def test_wide_blocks_gemv(fmt, M, K, N):
    raw = near_offset.weights(fmt, M, K)
    x = _wide_near(N, K)
    announce(f"wide near-offset gemv fmt={fmt} M={M} K={K} N={N}")
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(_gemv(fmt, raw, x, M, K, VALU), y_ref, S, "wide near-offset gemv")
    raw2 = si.weights(fmt, M, K, 77)
    x2 = _outlier(N, K, 78)
    announce(f"one-outlier gemv fmt={fmt} M={M} K={K} N={N}")
    y_ref, S = oracle.matmul_ref(fmt, raw2, x2, M, K)
    check_linear(_gemv(fmt, raw2, x2, M, K, VALU), y_ref, S, "one-outlier gemv")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("N", [1, 3])
def test_wide_blocks_fused(fmt, N):
    """The exact path under every epilogue: gated, norm, norm + gated, residual."""
    M, K = 2304, 4096
    raw = near_offset.weights(fmt, M, K)
    ru = np.roll(raw.reshape(M, -1), 1, axis=0).reshape(-1)
    x = _wide_tiny(N, K)
    gamma = _gamma(K, 5)
    r = si.activations(N, M, 11)
    announce(f"wide fused fmt={fmt} N={N}")
    h = qmm.gate_up_silu(fmt, dev(raw), dev(ru), dev(x), M, K, variant=VALU)
    yn = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), 1e-5, M, K)
    hn = qmm.rmsnorm_gate_up_silu(fmt, dev(raw), dev(ru), dev(x), dev(gamma), 1e-5, M, K)
    ya = qmm.gemv_add(fmt, dev(raw), dev(x), dev(r), M, K)
    torch.cuda.synchronize()
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, raw, ru, x, M, K)
    check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, "wide gate_up_silu")
    y_ref, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, 1e-5, M, K)
    check_linear(yn.cpu().numpy(), y_ref, S, "wide rmsnorm_gemv")
    h_ref, g, u, Sg, Su = oracle.rmsnorm_gate_up_silu_ref(fmt, raw, ru, x, gamma, 1e-5, M, K)
    check_swiglu(hn.cpu().numpy(), h_ref, g, u, Sg, Su, "wide rmsnorm_gate_up_silu")
    y_ref, S = oracle.matmul_add_ref(fmt, raw, x, r, M, K)
    check_residual(ya.cpu().numpy(), y_ref, S, "wide gemv_add")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("scale", [1e30, 1e-35, 1e-42], ids=["huge", "tiny", "fp32-subnormal"])
@pytest.mark.parametrize("M,K", [(2304, 4096), (300, 576)])
def test_x_range_gemv(fmt, scale, M, K):
    raw = si.weights(fmt, M, K, 80)
    x = (si.activations(3, K, 81).astype(np.float64) * scale).astype(np.float32)
    announce(f"x range gemv fmt={fmt} scale={scale} M={M} K={K}")
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(_gemv(fmt, raw, x, M, K, VALU), y_ref, S, f"x range gemv scale={scale}")


# Two tokens of wide x at K = 14336, whose fp32 copy takes 2 x 448 blocks x 144 bytes.
# 4096 rows run on the DMA-fed kernel, where it does not fit beside the weight ring: every
# workgroup takes the exact path that reads x and the weights from global memory.  1000
# rows run on the register-staged kernel with 4-wave workgroups, whose small ring leaves
# room for fp32 x in LDS.  The gated product (register-staged, 8 waves, gate and up rows
# in every task) does not have that room and takes the global path.
@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M", [4096, 1000])
def test_wide_blocks_k14336(fmt, M):
    K, N = 14336, 2
    rows = sample_rows(M, 40, 90 + fmt)
    raw = near_offset.weights(fmt, M, K)
    x = _wide_near(N, K)
    announce(f"wide near-offset gemv fmt={fmt} M={M} K={K} N={N}")
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
    check_linear(_gemv(fmt, raw, x, M, K, VALU)[:, rows], y_ref, S, "wide gemv at K = 14336")
    raw2 = si.weights(fmt, M, K, 91)
    x2 = _outlier(N, K, 92)
    announce(f"one-outlier gemv fmt={fmt} M={M} K={K} N={N}")
    y_ref, S = oracle.matmul_ref(fmt, raw2, x2, M, K, rows=rows)
    check_linear(_gemv(fmt, raw2, x2, M, K, VALU)[:, rows], y_ref, S, "one-outlier gemv at K = 14336")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
def test_wide_blocks_k14336_gated(fmt):
    I, K, N = 1536, 14336, 2
    rows = sample_rows(I, 40, 95 + fmt)
    rg = near_offset.weights(fmt, I, K)
    ru = np.roll(rg.reshape(I, -1), 1, axis=0).reshape(-1)
    x = _wide_tiny(N, K)
    announce(f"wide gate_up_silu (global exact path) fmt={fmt} I={I} K={K} N={N}")
    buf = poisoned(N * I)
    qmm.qmm_gate_up_silu_variant(fmt, dev(rg), dev(ru), dev(x), buf, I, K, N, VALU)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K, rows=rows)
    check_swiglu(buf[:N * I].cpu().numpy().reshape(N, I)[:, rows], h_ref, g, u, Sg, Su,
                 "wide gate_up_silu, global exact path")
