"""GPU parity at the measured workloads' full sizes, in the launch configuration the benchmark times.

* 576 x 576 Q8_0 GEMV, seed 0 (every output checked).
* SmolLM2-135M-shaped decode step, all 30 layers + LM head, Q8_0 and Q4_0 (every output).
* Llama-3-8B-shaped decode GEMVs (QKV, O, gate+up+SwiGLU, down, LM head), Q8_0 and Q4_0:
  the GPU computes the whole output; the oracle checks sampled rows.
* Batched decode N in {1, 2, 4, 8, 16}, F16 / Q8_0 / Q4_0, both GEMV variants (sampled rows).
* Prefill GEMM 4096->14336 and 14336->4096, T in {128, 2048, 4096}, Q8_0 / Q4_0 (sampled rows,
  all tokens), and the fused gate+up GEMM at 4096 -> 2 x 14336.
* One GPU's share of the Llama-3-8B decode projections under 8-way tensor parallelism (QKV,
  gate+up and LM head split by output rows, O and down by K), every block format, one token
  and (Q8_0, Q4_0) eight (every output; LM-head shard on sampled rows).
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_swiglu, dev, sample_rows

pytestmark = pytest.mark.gpu
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_F16: "f16"}
L8 = si.LLAMA3_8B
SM = si.SMOLLM2_135M


def test_single_q8_0_gemv_576_seed0():
    M = K = 576
    raw = si.weights(si.FMT_Q8_0, M, K, 0)
    x = si.activations(1, K, 1)
    announce("576x576 Q8_0 gemv seed 0")
    y = qmm.gemv(qmm.QMM_Q8_0, dev(raw), dev(x), M, K)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_ref(si.FMT_Q8_0, raw, x, M, K)
    check_linear(y.cpu().numpy(), y_ref, S, "576x576")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_smollm2_decode_step_all_layers(fmt):
    H, I, V = SM["hidden"], SM["intermediate"], SM["vocab"]
    Q = si.qkv_rows(SM)
    base = 2000 if fmt == si.FMT_Q8_0 else 2500
    for layer in range(SM["layers"]):
        s = base + 10 * layer
        w_qkv, w_o = si.weights(fmt, Q, H, s), si.weights(fmt, H, H, s + 1)
        w_g, w_u = si.weights(fmt, I, H, s + 2), si.weights(fmt, I, H, s + 3)
        w_d = si.weights(fmt, H, I, s + 4)
        x = si.activations(1, H, s + 5)
        announce(f"smollm2 layer {layer} fmt={fmt}")
        xd = dev(x)
        y_qkv = qmm.gemv(fmt, dev(w_qkv), xd, Q, H)
        y_o = qmm.gemv(fmt, dev(w_o), xd, H, H)
        h = qmm.gate_up_silu(fmt, dev(w_g), dev(w_u), xd, I, H)
        h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, w_g, w_u, x, I, H)
        x_down = h_ref.astype(np.float32)     # the oracle's h, rounded to fp32, feeds down on both sides
        y_d = qmm.gemv(fmt, dev(w_d), dev(x_down), H, I)
        torch.cuda.synchronize()
        r, S = oracle.matmul_ref(fmt, w_qkv, x, Q, H)
        check_linear(y_qkv.cpu().numpy(), r, S, f"L{layer} qkv")
        r, S = oracle.matmul_ref(fmt, w_o, x, H, H)
        check_linear(y_o.cpu().numpy(), r, S, f"L{layer} o")
        check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, f"L{layer} gate_up")
        r, S = oracle.matmul_ref(fmt, w_d, x_down, H, I)
        check_linear(y_d.cpu().numpy(), r, S, f"L{layer} down")
    w_lm = si.weights(fmt, V, H, base + 999)
    x = si.activations(1, H, base + 998)
    announce(f"smollm2 lm head fmt={fmt}")
    y = qmm.gemv(fmt, dev(w_lm), dev(x), V, H)
    torch.cuda.synchronize()
    r, S = oracle.matmul_ref(fmt, w_lm, x, V, H)
    check_linear(y.cpu().numpy(), r, S, "lm head")


LLAMA_GEMV = [("qkv", si.qkv_rows(L8), L8["hidden"]), ("o", L8["hidden"], L8["hidden"]),
              ("down", L8["hidden"], L8["intermediate"]), ("lm_head", L8["vocab"], L8["hidden"])]


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("name,M,K", LLAMA_GEMV, ids=[n for n, _, _ in LLAMA_GEMV])
def test_llama8b_gemv_sampled(fmt, name, M, K):
    seed = 3100 + M % 997 + K % 991 + fmt
    raw = si.weights(fmt, M, K, seed)
    x = si.activations(1, K, seed + 1)
    announce(f"llama8b {name} gemv fmt={fmt} M={M} K={K}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K).cpu().numpy()
    assert np.isfinite(y).all()
    rows = sample_rows(M, 200, seed)
    r, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
    check_linear(y[:, rows], r, S, f"llama {name}")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_llama8b_gate_up_sampled(fmt):
    I, K = L8["intermediate"], L8["hidden"]
    rg, ru = si.weights(fmt, I, K, 3300 + fmt), si.weights(fmt, I, K, 3301 + fmt)
    x = si.activations(1, K, 3302)
    announce(f"llama8b gate_up fmt={fmt}")
    h = qmm.gate_up_silu(fmt, dev(rg), dev(ru), dev(x), I, K).cpu().numpy()
    rows = sample_rows(I, 200, 5)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K, rows=rows)
    check_swiglu(h[:, rows], h_ref, g, u, Sg, Su, "llama gate_up")


@pytest.mark.parametrize("fmt", [si.FMT_F16, si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("name,M,K", [LLAMA_GEMV[0], LLAMA_GEMV[2]], ids=["qkv", "down"])
def test_llama8b_small_batch_sampled(fmt, name, M, K):
    seed = 3400 + M % 97 + fmt
    raw = si.weights(fmt, M, K, seed)
    Wd = dev(raw)
    rows = sample_rows(M, 64, seed)
    for N in (1, 2, 4, 8, 16):
        x = si.activations(N, K, seed + N)
        xd = dev(x)
        r, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
        for v in (qmm.QMM_VARIANT_VALU, qmm.QMM_VARIANT_MFMA):
            announce(f"llama8b {name} N={N} fmt={fmt} variant={v}")
            y = qmm.gemv(fmt, Wd, xd, M, K, variant=v).cpu().numpy()
            assert np.isfinite(y).all()
            check_linear(y[:, rows], r, S, f"{name} N={N} v={v}")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("M,K", [(14336, 4096), (4096, 14336)], ids=["up", "down"])
def test_prefill_gemm_sampled(fmt, M, K):
    seed = 3500 + M % 101 + fmt
    raw = si.weights(fmt, M, K, seed)
    Wd = dev(raw)
    rows = sample_rows(M, 40, seed)
    for T in (128, 2048, 4096):
        X = si.activations(T, K, seed + T, dtype=np.float16)
        announce(f"prefill gemm fmt={fmt} M={M} K={K} T={T}")
        Y = qmm.gemm(fmt, Wd, dev(X), M, K).cpu().numpy()
        assert np.isfinite(Y).all()
        r, S = oracle.matmul_ref(fmt, raw, X, M, K, rows=rows)
        check_linear(Y[:, rows], r, S, f"gemm M={M} K={K} T={T}")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_prefill_gate_up_gemm_sampled(fmt):
    I, K, T = L8["intermediate"], L8["hidden"], 128
    rg, ru = si.weights(fmt, I, K, 3600 + fmt), si.weights(fmt, I, K, 3601 + fmt)
    X = si.activations(T, K, 3602, dtype=np.float16)
    announce(f"prefill gate_up gemm fmt={fmt}")
    H = qmm.gemm_gate_up_silu(fmt, dev(rg), dev(ru), dev(X), I, K).cpu().numpy()
    rows = sample_rows(I, 40, 6)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, X, I, K, rows=rows)
    check_swiglu(H[:, rows], h_ref, g, u, Sg, Su, "gemm gate_up")


# One GPU's share at 8-way tensor parallelism: column-parallel QKV (768 of 6144 rows),
# gate+up (1792 of 14336) and LM head (16032 of 128256 rows); row-parallel O (K = 512 of
# 4096) and down (K = 1792 of 14336).
TP8 = [("qkv", si.qkv_rows(L8) // 8, L8["hidden"]), ("o", L8["hidden"], L8["hidden"] // 8),
       ("down", L8["hidden"], L8["intermediate"] // 8), ("lm_head", L8["vocab"] // 8, L8["hidden"])]
BLOCK_FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1]


@pytest.mark.parametrize("fmt", BLOCK_FMTS, ids=str)
def test_tp8_shard_decode(fmt):
    I8, H = L8["intermediate"] // 8, L8["hidden"]
    for k, (name, M, K) in enumerate(TP8):
        seed = 3900 + 10 * fmt + k
        raw = si.weights(fmt, M, K, seed)
        x = si.activations(1, K, seed + 1)
        announce(f"tp8 shard {name} fmt={fmt} M={M} K={K}")
        y = qmm.gemv(fmt, dev(raw), dev(x), M, K)
        torch.cuda.synchronize()
        rows = sample_rows(M, 300, seed) if M > 8192 else np.arange(M)
        r, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
        check_linear(y.cpu().numpy()[:, rows], r, S, f"tp8 {name} fmt={fmt}")
    rg, ru = si.weights(fmt, I8, H, 3950 + fmt), si.weights(fmt, I8, H, 3951 + fmt)
    x = si.activations(1, H, 3952)
    announce(f"tp8 shard gate_up fmt={fmt} I={I8}")
    h = qmm.gate_up_silu(fmt, dev(rg), dev(ru), dev(x), I8, H)
    torch.cuda.synchronize()
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I8, H)
    check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, f"tp8 gate_up fmt={fmt}")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("name,M,K", TP8[:3], ids=[n for n, _, _ in TP8[:3]])
def test_tp8_shard_eight_tokens(fmt, name, M, K):
    seed = 3960 + 10 * fmt + M % 7
    raw = si.weights(fmt, M, K, seed)
    x = si.activations(8, K, seed + 1)
    announce(f"tp8 shard {name} N=8 fmt={fmt} M={M} K={K}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K)
    torch.cuda.synchronize()
    r, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(y.cpu().numpy(), r, S, f"tp8 {name} N=8 fmt={fmt}")
