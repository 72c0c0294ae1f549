"""GPU parity of the decode GEMVs with fused neighbours: RMSNorm prologue (fused QKV,
final norm + LM head, FFN norm + gate+up+SwiGLU) and residual-add epilogue (O, down).

Each is compared with the float64 oracle's composition of the plain steps.
Covered:
* every format;
* 1..9 tokens (several 4-token weight passes and a remainder);
* ragged K;
* a final row left to the sliced kernel;
* per-token input scales spanning 1e-3..1e3 and a zero token;
* eps = 0 and large eps;
* in-place residual;
* the full Llama-3-8B projection shapes (sampled rows).
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_residual, check_swiglu, dev, sample_rows

pytestmark = pytest.mark.gpu
FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_F16]
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_F16: "f16"}
L8 = si.LLAMA3_8B

SHAPES = [(1, 32, 1), (17, 96, 2), (576, 576, 1), (300, 4096, 3), (70, 4128, 5), (33, 2048, 9), (960, 576, 4),
          (100, 14336, 1)]


def _x(N, K, seed, zero_token=False):
    """Tokens of N(0,1) times a per-token scale 10^a, a in [-3, 3]."""
    x = si.activations(N, K, seed)
    a = np.random.default_rng(seed).uniform(-3, 3, size=(N, 1))
    x = (x * 10.0 ** a).astype(np.float32)
    if zero_token and N > 1:
        x[1] = 0
    return x


def _gamma(K, seed):
    return (1.0 + 0.25 * si.activations(1, K, seed)[0]).astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_rmsnorm_gemv(fmt, M, K, N):
    seed = 9000 + M + K + N
    raw = si.weights(fmt, M, K, seed, scale_mode="uniform", q8_low=-128)
    x, gamma = _x(N, K, seed + 1, zero_token=True), _gamma(K, seed + 2)
    for eps in (1e-5, 0.0 if N == 1 else 1e-6, 4.0):
        announce(f"qmm_rmsnorm_gemv fmt={fmt} M={M} K={K} N={N} eps={eps}")
        y = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), eps, M, K)
        torch.cuda.synchronize()
        y_ref, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, eps, M, K)
        check_linear(y.cpu().numpy(), y_ref, S, f"rmsnorm_gemv eps={eps}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,N", [(64, 64, 1), (130, 576, 2), (300, 4096, 5), (77, 4128, 1), (200, 2816, 4)])
def test_rmsnorm_gate_up_silu(fmt, I, K, N):
    seed = 9100 + I + K + N
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    x, gamma = _x(N, K, seed + 2, zero_token=True), _gamma(K, seed + 3)
    eps = 1e-5
    announce(f"qmm_rmsnorm_gate_up_silu fmt={fmt} I={I} K={K} N={N}")
    h = qmm.rmsnorm_gate_up_silu(fmt, dev(rg), dev(ru), dev(x), dev(gamma), eps, I, K)
    torch.cuda.synchronize()
    h_ref, g, u, Sg, Su = oracle.rmsnorm_gate_up_silu_ref(fmt, rg, ru, x, gamma, eps, I, K)
    check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, "rmsnorm_gate_up_silu")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
def test_gemv_add(fmt, M, K, N, inplace):
    seed = 9200 + M + K + N
    raw = si.weights(fmt, M, K, seed, scale_mode="uniform", q8_low=-128)
    x = si.activations(N, K, seed + 1)
    r = (si.activations(N, M, seed + 2) * 100.0).astype(np.float32)
    rd = dev(r)
    announce(f"qmm_gemv_add fmt={fmt} M={M} K={K} N={N} inplace={inplace}")
    y = qmm.gemv_add(fmt, dev(raw), dev(x), rd, M, K, out=rd if inplace else None)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_add_ref(fmt, raw, x, r, M, K)
    check_residual(y.cpu().numpy(), y_ref, S, "gemv_add")
    if not inplace:
        assert np.array_equal(rd.cpu().numpy(), r), "the residual input must not change"


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_llama8b_fused_decode_projections_sampled(fmt):
    """One Llama-3-8B decode layer's fused calls plus the final norm + LM head,
    full sizes, N = 1, sampled rows."""
    H, I, V = L8["hidden"], L8["intermediate"], L8["vocab"]
    seed = 9300 + fmt
    x = _x(1, H, seed)
    gamma = _gamma(H, seed + 1)
    eps = 1e-5
    for name, M in (("qkv", si.qkv_rows(L8)), ("lm_head", V)):
        raw = si.weights(fmt, M, H, seed + M % 101)
        announce(f"llama8b rmsnorm + {name} fmt={fmt}")
        y = qmm.rmsnorm_gemv(fmt, dev(raw), dev(x), dev(gamma), eps, M, H).cpu().numpy()
        rows = sample_rows(M, 200, seed)
        y_ref, S = oracle.rmsnorm_matmul_ref(fmt, raw, x, gamma, eps, M, H, rows=rows)
        check_linear(y[:, rows], y_ref, S, f"rmsnorm {name}")
    rg, ru = si.weights(fmt, I, H, seed + 7), si.weights(fmt, I, H, seed + 8)
    announce(f"llama8b rmsnorm + gate_up fmt={fmt}")
    h = qmm.rmsnorm_gate_up_silu(fmt, dev(rg), dev(ru), dev(x), dev(gamma), eps, I, H).cpu().numpy()
    rows = sample_rows(I, 200, seed + 1)
    h_ref, g, u, Sg, Su = oracle.rmsnorm_gate_up_silu_ref(fmt, rg, ru, x, gamma, eps, I, H, rows=rows)
    check_swiglu(h[:, rows], h_ref, g, u, Sg, Su, "rmsnorm gate_up")
    for name, M, K in (("o", H, H), ("down", H, I)):
        raw = si.weights(fmt, M, K, seed + K % 103)
        xin = si.activations(1, K, seed + 9)
        r = si.activations(1, M, seed + 10)
        rd = dev(r)
        announce(f"llama8b {name} + residual (in place) fmt={fmt}")
        qmm.gemv_add(fmt, dev(raw), dev(xin), rd, M, K, out=rd)
        y = rd.cpu().numpy()
        rows = sample_rows(M, 200, seed + 2)
        y_ref, S = oracle.matmul_add_ref(fmt, raw, xin, r, M, K, rows=rows)
        check_residual(y[:, rows], y_ref, S, f"{name} + residual")
