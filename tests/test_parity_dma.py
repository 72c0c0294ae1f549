"""GPU parity of the DMA-fed decode GEMV (block-format rows that are 16-byte aligned,
K % 256 == 0, 1..4 tokens per weight pass) against the float64 oracle.

The shapes walk the kernel's geometry:
* a partial last K slice (64 blocks per Q8_0 slice, 128 per slice of the nibble
  formats) and a single partial slice;
* fewer tasks per wave than ring slots, and many more (the ring wraps);
* row counts that are not multiples of the rows per task (the nibble formats run
  2-row tasks when those spread the rows as evenly over the waves as 1-row tasks:
  here at 20000, 65537 and 65600 rows, and 8192 rows in the residual mode), and
  more row groups than waves;
* x sizes up to 35 KB per token (K = 14336) and 4 tokens of K = 4096;
* the RMSNorm and residual modes, including the residual with more row groups per
  wave than the kernel reads ahead (another kernel takes those);
* the gated (SwiGLU) product at the same shapes (served by the register-staged
  kernel, which measured faster for it).
Matrices of up to 2048 rows run on the register-staged kernel (its small workgroups
win there), so every case here has more rows.  Each output is poisoned with NaNs and
followed by a guard band.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import (announce, check_linear, check_residual, check_swiglu, dev, guard_intact, poisoned)

pytestmark = pytest.mark.gpu
FMTS = [si.FMT_Q8_0, si.FMT_Q4_0]
ALL_FMTS = FMTS + [si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1]  # 3072-byte slots for the last three
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_Q4_1: "q4_1", si.FMT_Q5_0: "q5_0", si.FMT_Q5_1: "q5_1"}
VALU = qmm.QMM_VARIANT_VALU

GEMV_CASES = [
    (2051, 256, 1),    # one partial slice, fewer tasks than slots
    (2305, 768, 1),    # partial slice, ragged M
    (2305, 768, 4),    # 4 tokens per pass
    (3048, 2304, 2),   # Q8_0: 64 + 8 blocks; Q4_0: one 72-block slice
    (4100, 4352, 1),   # more row groups than waves; Q8_0 3 slices, Q4_0 128 + 8
    (16385, 2304, 1),  # many row groups per wave
    (20000, 4352, 3),  # ring wraps many times, 3 tokens (nibble formats: 2-row tasks)
    (65537, 512, 1),   # nibble formats: 2-row tasks with a lone last row
    (65600, 256, 4),   # nibble formats: 2-row tasks, 4 tokens
    (4096, 14336, 1),  # nibble formats: 2-row tasks, x 35 KB
    (2561, 14336, 1),  # x 35 KB per token
    (2348, 4096, 4),   # 4 tokens, x 40 KB
    (2057, 4096, 6),   # two passes (4 + 2 tokens)
]


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", GEMV_CASES)
def test_dma_gemv(fmt, M, K, N):
    seed = 5000 + M + K + N
    raw = si.weights(fmt, M, K, seed, scale_mode="uniform", q8_low=-128)
    x = si.activations(N, K, seed + 1)
    announce(f"dma gemv fmt={fmt} M={M} K={K} N={N} seed={seed}")
    buf = poisoned(N * M)
    qmm.qmm_gemv_variant(fmt, dev(raw), dev(x), buf, M, K, N, VALU)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * M)
    got = buf[:N * M].cpu().numpy().reshape(N, M)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(got, y_ref, S, f"dma gemv fmt={fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
def test_dma_gemv_one_hot_exact(fmt):
    """x = e_k returns the decoded column rounded once to fp32 (exact for Q8_0 / Q4_0 /
    Q5_0; d * u + m of the biased formats may need more bits), across slices and ring
    slots."""
    M, K = 4100, 4352
    raw = si.weights(fmt, M, K, 61, scale_mode="gemm_wide", q8_low=-128)
    cols = [0, 31, 2047, 4351]
    x = si.one_hot(len(cols), K, cols)
    announce(f"dma gemv one-hot fmt={fmt} M={M} K={K}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=VALU).cpu().numpy().astype(np.float64)
    W = oracle.dequant(fmt, raw, M, K).astype(np.float32).astype(np.float64)
    for n, c in enumerate(cols):
        assert np.array_equal(y[n], W[:, c]), (n, c)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,N", [(3, 256, 1), (1000, 2304, 2), (5000, 4352, 1), (700, 14336, 1), (129, 4096, 4)])
def test_dma_gate_up_silu(fmt, I, K, N):
    seed = 5100 + I + K + N
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    x = si.activations(N, K, seed + 2)
    announce(f"dma gate_up_silu fmt={fmt} I={I} K={K} N={N}")
    buf = poisoned(N * I)
    qmm.qmm_gate_up_silu_variant(fmt, dev(rg), dev(ru), dev(x), buf, I, K, N, VALU)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    check_swiglu(buf[:N * I].cpu().numpy().reshape(N, I), h_ref, g, u, Sg, Su, "dma gate_up_silu")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(2305, 768, 1), (4100, 4352, 2), (20000, 2304, 1), (2561, 14336, 1),
                                   (50000, 512, 1)])  # one token: nibble formats on 12-wave workgroups
def test_dma_rmsnorm_gemv(fmt, M, K, N):
    seed = 5200 + M + K + N
    raw = si.weights(fmt, M, K, seed)
    x = si.activations(N, K, seed + 1)
    gamma = (1.0 + 0.25 * si.activations(1, K, seed + 2)[0]).astype(np.float32)
    announce(f"dma rmsnorm_gemv fmt={fmt} M={M} K={K} N={N}")
    y = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), 1e-5, M, K)
    torch.cuda.synchronize()
    y_ref, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, 1e-5, M, K)
    check_linear(y.cpu().numpy(), y_ref, S, "dma rmsnorm_gemv")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(2305, 768, 1), (4100, 4352, 1), (8192, 2304, 2), (20000, 2304, 1),
                                   (50001, 256, 1)])
@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
def test_dma_gemv_add(fmt, M, K, N, inplace):
    """8192 rows: two row groups per wave (read ahead); 20000 and 50001: more row
    groups per wave than the DMA kernel reads residuals for ahead of its loop (the
    register-staged kernel takes them; 50001: a lone last row)."""
    seed = 5300 + M + K + N
    raw = si.weights(fmt, M, K, seed)
    x = si.activations(N, K, seed + 1)
    r = (si.activations(N, M, seed + 2) * 100.0).astype(np.float32)
    rd = dev(r)
    announce(f"dma gemv_add fmt={fmt} M={M} K={K} N={N} inplace={inplace}")
    y = qmm.gemv_add(fmt, dev(raw), dev(x), rd, M, K, out=rd if inplace else None)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_add_ref(fmt, raw, x, r, M, K)
    check_residual(y.cpu().numpy(), y_ref, S, "dma gemv_add")
    if not inplace:
        assert np.array_equal(rd.cpu().numpy(), r), "the residual input must not change"


@pytest.mark.parametrize("fmt", FMTS + [si.FMT_Q5_0], ids=FID.get)
@pytest.mark.parametrize("N", [1, 3])
def test_dma_zero_codes_give_zero(fmt, N):
    """Codes equal to the zero code (q = 0, nibble 8, 5-bit code 16) give exactly zero:
    the offset is removed in fp16 before the dot products, so such codes enter them as
    exact zeros."""
    M, K = 2348, 4352
    d = np.full((M, K // 32), 0.75, dtype=np.float16)
    if fmt == si.FMT_Q8_0:
        raw = oracle.pack_q8_0(np.zeros((M, K), dtype=np.int8), d)
    elif fmt == si.FMT_Q5_0:
        raw = oracle.pack_q5_0(np.full((M, K), 16, dtype=np.int64), d)
    else:
        raw = oracle.pack_q4_0(np.full((M, K), 8, dtype=np.uint8), d)
    x = (si.activations(N, K, 17) * np.float32(1e3)).astype(np.float32)
    announce(f"dma zero codes fmt={fmt} N={N}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=VALU)
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == 0).all()
