"""GPU parity over a seeded random sweep of shapes, formats, token counts and entry points.

The fixed-shape suites pick shapes by hand; this one draws them, so that the kernel
selection (register-staged or DMA-fed VALU kernels, 8- or 12-wave workgroups, 1- or
2-row tasks, gated products on either kernel, the MFMA GEMV with and without a K
split, the tiled GEMM) is exercised on shapes nobody chose.  Each draw takes M from
one of three ranges (up to 1024 rows, 2049..6000, 49152..60000), K as 32 k (any) or
256 k (the DMA- and MFMA-eligible rows), N from 1..40, one of the block formats or
F16, and one entry point; weights and x are seeded synthetic data, the oracle checks
every row of small outputs and 160 sampled rows of large ones.  The draws are fixed by
the seed: the same cases run every time.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_residual, check_swiglu, dev, sample_rows

pytestmark = pytest.mark.gpu

FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1, si.FMT_F16]
OPS = ["gemv", "gate_up", "rmsnorm_gemv", "gemv_add", "gemm"]
MAX_WEIGHTS = 48 << 20  # M K per draw, so that generating the weights stays quick


def _draw(i):
    g = np.random.default_rng(910000 + i)
    fmt = FMTS[g.integers(len(FMTS))]
    op = OPS[g.integers(len(OPS))]
    band = g.integers(3)
    M = int(g.integers(1, 1025) if band == 0 else g.integers(2049, 6001) if band == 1 else g.integers(49152, 60001))
    if g.random() < 0.6:
        K = 256 * int(g.integers(1, 17))
    else:
        K = 32 * int(g.integers(1, 129))
    while M * K > MAX_WEIGHTS:
        K = max(32, (K // 2) // 32 * 32)
    N = int(g.choice([1, 1, 2, 3, 4, 5, 8, 16, 17, 32, 33, 40]))
    if op == "gate_up" and M * K * 2 > MAX_WEIGHTS:
        M = max(1, MAX_WEIGHTS // (2 * K))
    return fmt, op, M, K, N


# Hand-picked draws for routes that the drawn shapes may miss: the gated product on the
# DMA-fed kernel (Q8_0 at 1-4 tokens, Q4_0 at 2-4, rows past 2048, K % 256 == 0), and
# the 12-wave, 2-row multi-token GEMV of Q8_0 and Q4_0 from 49152 rows.
ROUTES = [(si.FMT_Q4_0, "gate_up", 3000, 1024, n) for n in (2, 3, 4)] + \
         [(si.FMT_Q8_0, "gate_up", 2500, 768, n) for n in (1, 4)] + \
         [(si.FMT_Q8_0, "gemv", 50001, 512, n) for n in (2, 3, 4)] + \
         [(si.FMT_Q4_0, "gemv", 49153, 1024, 3), (si.FMT_Q8_0, "rmsnorm_gemv", 49160, 768, 2),
          (si.FMT_Q4_0, "rmsnorm_gemv", 2600, 512, 3)]
CASES = [_draw(i) for i in range(120)] + ROUTES


@pytest.mark.parametrize("fmt,op,M,K,N", CASES, ids=[f"{c[1]}-f{c[0]}-{c[2]}x{c[3]}-n{c[4]}" for c in CASES])
def test_random_sweep(fmt, op, M, K, N):
    seed = 920000 + 7 * M + 3 * K + N + fmt
    rows = np.arange(M) if M <= 4096 else sample_rows(M, 160, seed)
    raw = si.weights(fmt, M, K, seed)
    announce(f"random sweep op={op} fmt={fmt} M={M} K={K} N={N} seed={seed}")
    if op == "gemm":
        X = si.activations(N, K, seed + 1, dtype=np.float16)
        y = qmm.gemm(fmt, dev(raw), dev(X), M, K)
        torch.cuda.synchronize()
        r, S = oracle.matmul_ref(fmt, raw, X, M, K, rows=rows)
        check_linear(y.cpu().numpy()[:, rows], r, S, f"gemm {fmt} {M}x{K} T={N}")
        return
    x = si.activations(N, K, seed + 1)
    if op == "gemv":
        y = qmm.gemv(fmt, dev(raw), dev(x), M, K)
        torch.cuda.synchronize()
        r, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
        check_linear(y.cpu().numpy()[:, rows], r, S, f"gemv {fmt} {M}x{K} N={N}")
    elif op == "gate_up":
        ru = si.weights(fmt, M, K, seed + 2)
        h = qmm.gate_up_silu(fmt, dev(raw), dev(ru), dev(x), M, K)
        torch.cuda.synchronize()
        hr, gg, uu, Sg, Su = oracle.gate_up_silu_ref(fmt, raw, ru, x, M, K, rows=rows)
        check_swiglu(h.cpu().numpy()[:, rows], hr, gg, uu, Sg, Su, f"gate_up {fmt} {M}x{K} N={N}")
    elif op == "rmsnorm_gemv":
        gamma = (1.0 + 0.1 * si.activations(1, K, seed + 3)[0]).astype(np.float32)
        y = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), 1e-5, M, K)
        torch.cuda.synchronize()
        r, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, 1e-5, M, K, rows=rows)
        check_linear(y.cpu().numpy()[:, rows], r, S, f"rmsnorm_gemv {fmt} {M}x{K} N={N}")
    else:
        res = si.activations(N, M, seed + 4)
        y = qmm.gemv_add(fmt, dev(raw), dev(x), dev(res), M, K)
        torch.cuda.synchronize()
        r, S = oracle.matmul_add_ref(fmt, raw, x, res, M, K, rows=rows)
        check_residual(y.cpu().numpy()[:, rows], r, S, f"gemv_add {fmt} {M}x{K} N={N}")
