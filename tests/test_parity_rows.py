"""GPU parity of the element-wise weight kernels: quantised row gather and fp16 expansion.

* qmm_get_rows: bit-exact against the oracle's row gather (repeats, first and last
  rows, ragged K, full SmolLM2-135M and Llama-3-8B embedding tables), NaN rows for
  ids outside [0, M), an empty gather, inf/NaN scales.
* qmm_expand_f16: bit-exact fp16 bits against the oracle's round-to-nearest-even
  expansion (subnormal and overflowing products included), and expand-then-GEMM
  (qmm_expand_f16 followed by the F16 qmm_gemm) bitwise equal to the fused qmm_gemm.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_swiglu, dev, guard_intact, poisoned, sample_rows

pytestmark = pytest.mark.gpu
FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_F16]
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_F16: "f16"}


def _ids(M, n, seed):
    g = np.random.default_rng(seed)
    ids = g.integers(0, M, size=n).astype(np.int32)
    ids[: min(n, 2)] = [0, M - 1][: min(n, 2)]
    if n > 4:
        ids[-1] = ids[2]  # a repeat
    return ids


def _gather(fmt, raw, M, K, ids):
    n = len(ids)
    buf = poisoned(n * K)
    qmm.qmm_get_rows(fmt, dev(raw), dev(ids), buf, M, K, n)
    torch.cuda.synchronize()
    assert guard_intact(buf, n * K), "write past the end of out"
    return buf[: n * K].cpu().numpy().reshape(n, K).astype(np.float64)


def _same_bits(got, ref):
    assert got.shape == ref.shape
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------------------ row gather
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,n,mode", [(1, 32, 1, "uniform"), (7, 96, 9, "wide"), (1000, 4096, 37, "wide"),
                                        (300, 4128, 64, "uniform"), (5, 14336, 3, "wide")])
def test_get_rows_bit_exact(fmt, M, K, n, mode):
    seed = 8000 + M + K + n
    raw = si.weights(fmt, M, K, seed, scale_mode=mode, q8_low=-128)
    ids = _ids(M, n, seed)
    announce(f"qmm_get_rows fmt={fmt} M={M} K={K} n={n} mode={mode}")
    _same_bits(_gather(fmt, raw, M, K, ids), oracle.get_rows_ref(fmt, raw, M, K, ids))


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_get_rows_invalid_ids_give_nan_rows(fmt):
    M, K = 50, 256
    raw = si.weights(fmt, M, K, 8101, q8_low=-128)
    ids = np.array([3, -1, M, 0, 2**31 - 1, -2**31, M - 1, 3], dtype=np.int32)
    announce(f"qmm_get_rows invalid ids fmt={fmt}")
    got = _gather(fmt, raw, M, K, ids)
    ref = oracle.get_rows_ref(fmt, raw, M, K, ids)
    assert np.isnan(got[[1, 2, 4, 5]]).all()
    _same_bits(got, ref)


def test_get_rows_empty_is_a_no_op():
    M, K = 4, 64
    raw = si.weights(si.FMT_Q8_0, M, K, 8102)
    buf = poisoned(0)
    announce("qmm_get_rows n=0")
    out = qmm.get_rows(si.FMT_Q8_0, dev(raw), torch.empty(0, dtype=torch.int32, device="cuda"), M, K, out=buf)
    torch.cuda.synchronize()
    assert out is buf and guard_intact(buf, 0)


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_get_rows_inf_nan_scales(fmt):
    M, K = 2, 64
    d = np.array([[np.inf, -np.inf], [np.nan, 0.0]], dtype=np.float16)
    if fmt == si.FMT_Q8_0:
        raw = oracle.pack_q8_0(np.tile(np.arange(-32, 32, dtype=np.int8), (M, 1)), d)
    else:
        raw = oracle.pack_q4_0(np.tile(np.arange(64, dtype=np.uint8) % 16, (M, 1)), d)
    ids = np.array([1, 0, 1], dtype=np.int32)
    announce(f"qmm_get_rows inf/nan scales fmt={fmt}")
    _same_bits(_gather(fmt, raw, M, K, ids), oracle.get_rows_ref(fmt, raw, M, K, ids))


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("model", ["smollm2_135m", "llama3_8b"])
def test_get_rows_full_embedding_table(fmt, model):
    cfg = si.SMOLLM2_135M if model == "smollm2_135m" else si.LLAMA3_8B
    V, H = cfg["vocab"], cfg["hidden"]
    seed = 8200 + V % 1009 + fmt
    raw = si.weights(fmt, V, H, seed)
    ids = _ids(V, 512, seed)
    announce(f"qmm_get_rows {model} token table fmt={fmt} V={V} H={H} n=512")
    _same_bits(_gather(fmt, raw, V, H, ids), oracle.get_rows_ref(fmt, raw, V, H, ids))


# ------------------------------------------------------------- fp16 expansion
def _expand(fmt, raw, M, K):
    guard = 64
    buf = torch.full((M * K + guard,), 0x7E01, dtype=torch.int16, device="cuda")  # NaN bits + guard
    qmm.qmm_expand_f16(fmt, dev(raw), buf, M, K)
    torch.cuda.synchronize()
    assert bool((buf[M * K:] == 0x7E01).all().item()), "write past the end of out"
    return buf[: M * K].cpu().numpy().view(np.uint16).reshape(M, K)


def _ref_bits(fmt, raw, M, K):
    with np.errstate(over="ignore", invalid="ignore"):
        return oracle.expand_f16_ref(fmt, raw, M, K).view(np.uint16)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,mode", [(1, 32, "uniform"), (7, 96, "wide"), (33, 576, "gemm_wide"),
                                      (5, 4096, "wide"), (3, 4128, "wide"), (130, 2816, "uniform")])
def test_expand_f16_bit_exact(fmt, M, K, mode):
    seed = 8300 + M + K
    raw = si.weights(fmt, M, K, seed, scale_mode=mode, q8_low=-128)
    announce(f"qmm_expand_f16 fmt={fmt} M={M} K={K} mode={mode}")
    got = _expand(fmt, raw, M, K)
    assert np.array_equal(got, _ref_bits(fmt, raw, M, K))


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_expand_f16_inf_nan_scales(fmt):
    M, K = 2, 64
    d = np.array([[np.inf, -np.inf], [np.nan, 0.0]], dtype=np.float16)
    if fmt == si.FMT_Q8_0:
        raw = oracle.pack_q8_0(np.tile(np.arange(-32, 32, dtype=np.int8), (M, 1)), d)
    else:
        raw = oracle.pack_q4_0(np.tile(np.arange(64, dtype=np.uint8) % 16, (M, 1)), d)
    announce(f"qmm_expand_f16 inf/nan scales fmt={fmt}")
    got = _expand(fmt, raw, M, K).view(np.float16)
    ref = _ref_bits(fmt, raw, M, K).view(np.float16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint16), ref[~nan].view(np.uint16))


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_expand_f16_llama_up_sampled(fmt):
    M, K = si.LLAMA3_8B["intermediate"], si.LLAMA3_8B["hidden"]
    seed = 8400 + fmt
    raw = si.weights(fmt, M, K, seed)
    announce(f"qmm_expand_f16 llama8b up fmt={fmt} M={M} K={K}")
    out = torch.empty((M, K), dtype=torch.float16, device="cuda")
    qmm.qmm_expand_f16(fmt, dev(raw), out, M, K)
    torch.cuda.synchronize()
    rows = sample_rows(M, 200, seed)
    got = out.cpu().numpy()[rows].view(np.uint16)
    rb = qmm.qmm_row_bytes(fmt, K)
    sel = raw.reshape(M, rb)[rows].reshape(-1)
    assert np.array_equal(got, _ref_bits(fmt, sel, len(rows), K))


# ---------------------------------------------------------- expand then GEMM
@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("M,K,T", [(300, 2816, 40), (600, 4096, 300), (257, 1280, 129)])
def test_expand_then_gemm_matches_fused(fmt, M, K, T):
    seed = 8500 + M + K + T
    raw = si.weights(fmt, M, K, seed, scale_mode="gemm_wide", q8_low=-128)
    X = si.activations(T, K, seed + 1, dtype=np.float16)
    Wd, Xd = dev(raw), dev(X)
    announce(f"expand-then-gemm vs fused fmt={fmt} M={M} K={K} T={T}")
    W16 = qmm.expand_f16(fmt, Wd, M, K)
    Y_exp = qmm.gemm(si.FMT_F16, W16, Xd, M, K)
    Y_fused = qmm.gemm(fmt, Wd, Xd, M, K)
    torch.cuda.synchronize()
    y_exp, y_fused = Y_exp.cpu().numpy(), Y_fused.cpu().numpy()
    y_ref, S = oracle.matmul_ref(fmt, raw, X, M, K)
    check_linear(y_exp, y_ref, S, "expand-then-gemm")
    assert np.array_equal(y_exp, y_fused), "expand-then-GEMM must feed the MFMAs the same fp16 weights"


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_expand_then_gate_up_matches_fused(fmt):
    I, K, T = 200, 4096, 130
    rg, ru = si.weights(fmt, I, K, 8601), si.weights(fmt, I, K, 8602)
    X = si.activations(T, K, 8603, dtype=np.float16)
    g_d, u_d, Xd = dev(rg), dev(ru), dev(X)
    announce(f"expand-then-gate_up vs fused fmt={fmt} I={I} K={K} T={T}")
    H_exp = qmm.gemm_gate_up_silu(si.FMT_F16, qmm.expand_f16(fmt, g_d, I, K), qmm.expand_f16(fmt, u_d, I, K),
                                  Xd, I, K)
    H_fused = qmm.gemm_gate_up_silu(fmt, g_d, u_d, Xd, I, K)
    torch.cuda.synchronize()
    h_exp = H_exp.cpu().numpy()
    h_ref, gg, uu, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, X, I, K)
    check_swiglu(h_exp, h_ref, gg, uu, Sg, Su, "expand-then-gate_up")
    assert np.array_equal(h_exp, H_fused.cpu().numpy())
