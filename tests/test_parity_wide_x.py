"""GPU parity of the decode GEMVs when x holds wide blocks, on the DMA-fed kernel.

A block of x is wide when one of its nonzero values lies more than about 2^28 below
the block's largest, so that block floating point in fp16 cannot hold it; a
workgroup that meets one runs its rows on fp32 x.  Such x is what the gate+up
product hands to the down projection when its gate values reach -60 or so (silu
then returns about 1e-25 next to values of order 10).  These cases cover that
switch at the shapes that run the DMA-fed kernel (more than 2048 rows, K a multiple
of 256):
* 1-4 tokens at K = 4096 (x staged in one round, its fp32 copy written from the
  staging registers), and at K = 14336 one token (one round) and more (x staged over
  several rounds and read again, the exact path when fp32 x does not fit, or another
  kernel when block-scaled x does not);
* 12-wave workgroups (49160 rows, sampled);
* the plain product, the RMSNorm prologue, the residual epilogue and gate+up;
* every block format.
The oracle takes the fp32 x the caller passed; the bound is the usual
2e-3 * sum |w x| + 1e-6 (SwiGLU: its propagated form).
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_residual, check_swiglu, dev, sample_rows

pytestmark = pytest.mark.gpu
BLOCK_FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1]
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_Q4_1: "q4_1", si.FMT_Q5_0: "q5_0",
       si.FMT_Q5_1: "q5_1"}


def _wide_x(N, K, seed, kind):
    """fp32 tokens with wide blocks: 'swiglu' = silu(27 g) u (g, u standard normal),
    'sparse' = standard normal with about one value in 200 replaced by 1e-30 times a
    standard normal."""
    g = np.random.default_rng(seed)
    if kind == "swiglu":
        a = 27.0 * g.standard_normal((N, K))
        x = a / (1.0 + np.exp(-a)) * g.standard_normal((N, K))
    else:
        x = g.standard_normal((N, K))
        tiny = g.random((N, K)) < 0.005
        x = np.where(tiny, 1e-30 * g.standard_normal((N, K)), x)
    x = x.astype(np.float32)
    m = np.max(np.abs(x.reshape(N, K // 32, 32)), axis=2, keepdims=True)
    small = (np.abs(x.reshape(N, K // 32, 32)) < m * 2.0 ** -29) & (x.reshape(N, K // 32, 32) != 0)
    assert small.any(), "the draw must hold a wide block"
    return x


CASES = [(2100, 4096, 1), (2100, 4096, 2), (2100, 4096, 3), (2100, 4096, 4), (2056, 14336, 1),
         (2056, 14336, 2), (2056, 14336, 4)]


def _rows(M, K, seed):
    """All rows at K = 4096; sampled rows (first, last and 150 more) beyond."""
    return None if K <= 4096 else sample_rows(M, 150, seed)


def _take(y, rows):
    return y if rows is None else y[:, rows]


@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", CASES)
@pytest.mark.parametrize("kind", ["swiglu", "sparse"])
def test_gemv_wide_x(fmt, M, K, N, kind):
    seed = 9500 + M + K + N + (7 if kind == "sparse" else 0)
    raw = si.weights(fmt, M, K, seed)
    x = _wide_x(N, K, seed + 1, kind)
    announce(f"qmm_gemv (VALU) wide x fmt={fmt} M={M} K={K} N={N} kind={kind}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=qmm.QMM_VARIANT_VALU)
    torch.cuda.synchronize()
    rows = _rows(M, K, seed)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
    check_linear(_take(y.cpu().numpy(), rows), y_ref, S, f"gemv wide x ({kind})")


@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(2100, 4096, 1), (2100, 4096, 3), (2056, 14336, 2)])
def test_fused_wide_x(fmt, M, K, N):
    seed = 9600 + M + K + N
    raw = si.weights(fmt, M, K, seed)
    x = _wide_x(N, K, seed + 1, "swiglu")
    gamma = (1.0 + 0.25 * si.activations(1, K, seed + 2)[0]).astype(np.float32)
    announce(f"qmm_rmsnorm_gemv wide x fmt={fmt} M={M} K={K} N={N}")
    y = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), 1e-5, M, K)
    torch.cuda.synchronize()
    rows = _rows(M, K, seed)
    y_ref, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, 1e-5, M, K, rows=rows)
    check_linear(_take(y.cpu().numpy(), rows), y_ref, S, "rmsnorm_gemv wide x")
    r = (si.activations(N, M, seed + 3) * 10.0).astype(np.float32)
    announce(f"qmm_gemv_add wide x fmt={fmt} M={M} K={K} N={N}")
    y = qmm.gemv_add(fmt, dev(raw), dev(x), dev(r), M, K)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_add_ref(fmt, raw, x, r, M, K, rows=rows)
    check_residual(_take(y.cpu().numpy(), rows), y_ref, S, "gemv_add wide x")


@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=FID.get)
@pytest.mark.parametrize("N", [1, 2, 4])
def test_gate_up_wide_x(fmt, N):
    I, K = 2100, 4096
    seed = 9700 + N
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    x = _wide_x(N, K, seed + 2, "sparse")
    announce(f"qmm_gate_up_silu (VALU) wide x fmt={fmt} I={I} K={K} N={N}")
    h = qmm.gate_up_silu(fmt, dev(rg), dev(ru), dev(x), I, K, variant=qmm.QMM_VARIANT_VALU)
    torch.cuda.synchronize()
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, "gate_up wide x")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("N", [1, 2, 4])
def test_gemv_wide_x_twelve_waves(fmt, N):
    """49160 rows: the 12-wave workgroups (Q4_0 at 1-4 tokens, Q8_0 at 2-4)."""
    M, K = 49160, 4096
    seed = 9800 + N + fmt
    raw = si.weights(fmt, M, K, seed)
    x = _wide_x(N, K, seed + 1, "swiglu")
    announce(f"qmm_gemv (VALU) wide x fmt={fmt} M={M} K={K} N={N}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=qmm.QMM_VARIANT_VALU).cpu().numpy()
    rows = sample_rows(M, 300, seed)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
    check_linear(y[:, rows], y_ref, S, "gemv wide x, 12 waves")
