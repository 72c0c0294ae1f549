"""GPU parity far beyond the workloads' sizes, on weights drawn on the device.

* 2^27 + 3 rows of one block (Q4_0, Q5_1) and 2^26 + 1 rows (Q8_0): a grid of
  millions of workgroups, 64-bit row offsets, and a matrix size that is not a multiple of
  16 bytes (the final row goes to the sliced kernel).
* K = 2^20 weights per row: x (4 MB per token) is far beyond LDS, so the sliced kernel
  walks 512 or 256 K slices; also the gated product at that K.
* The prefill GEMM at K = 2^18 (split K over workgroups) and the small-batch MFMA GEMV at
  K = 2^18.
The checked rows' bytes are read back from the device and decoded by the oracle.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_swiglu, dev, sample_rows

pytestmark = pytest.mark.gpu
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_Q5_1: "q5_1", si.FMT_F16: "f16"}


def _rows_bytes(W, fmt, K, rows):
    rb = si.layout_bytes(fmt, K)
    idx = torch.as_tensor(np.asarray(rows), device=W.device)
    return W.view(-1, rb).index_select(0, idx).cpu().numpy().reshape(-1)


@pytest.mark.parametrize("fmt,M", [(si.FMT_Q4_0, 2**27 + 3), (si.FMT_Q5_1, 2**27 + 3), (si.FMT_Q8_0, 2**26 + 1)],
                         ids=lambda v: FID.get(v, str(v)))
def test_gemv_many_rows(fmt, M):
    K, N = 32, 2
    announce(f"gemv many rows fmt={fmt} M={M} K={K} N={N}")
    W = si.device_weights(fmt, M, K, 8800 + fmt, "cuda")
    x = si.activations(N, K, 8801)
    y = qmm.gemv(fmt, W, dev(x), M, K)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(M, 200, 8802), [M - 1, M - 2, M - 3, M // 2]]))
    got = y[:, torch.as_tensor(rows, device="cuda")].cpu().numpy()
    raw = _rows_bytes(W, fmt, K, rows)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, len(rows), K)
    check_linear(got, y_ref, S, f"gemv many rows fmt={fmt}")
    del W, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q5_1, si.FMT_F16], ids=FID.get)
def test_gemv_long_k(fmt):
    M, K, N = 5, 2**20, 2
    announce(f"gemv long K fmt={fmt} M={M} K={K} N={N}")
    W = si.device_weights(fmt, M, K, 8900 + fmt, "cuda")
    x = si.activations(N, K, 8901)
    y = qmm.gemv(fmt, W, dev(x), M, K).cpu().numpy()
    raw = W.cpu().numpy()
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(y, y_ref, S, f"gemv long K fmt={fmt}")


def test_gate_up_long_k():
    fmt, I, K = si.FMT_Q4_0, 3, 2**20
    announce(f"gate_up long K I={I} K={K}")
    Wg, Wu = si.device_weights(fmt, I, K, 8950, "cuda"), si.device_weights(fmt, I, K, 8951, "cuda")
    x = si.activations(1, K, 8952)
    h = qmm.gate_up_silu(fmt, Wg, Wu, dev(x), I, K).cpu().numpy()
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, Wg.cpu().numpy(), Wu.cpu().numpy(), x, I, K)
    check_swiglu(h, h_ref, g, u, Sg, Su, "gate_up long K")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q5_1], ids=FID.get)
def test_gemm_long_k(fmt):
    M, K, T = 300, 2**18, 40
    announce(f"gemm long K fmt={fmt} M={M} K={K} T={T}")
    W = si.device_weights(fmt, M, K, 9000 + fmt, "cuda")
    X = si.activations(T, K, 9001, dtype=np.float16)
    Y = qmm.gemm(fmt, W, dev(X), M, K).cpu().numpy()
    rows = sample_rows(M, 40, 9002)
    raw = _rows_bytes(W, fmt, K, rows)
    y_ref, S = oracle.matmul_ref(fmt, raw, X, len(rows), K)
    check_linear(Y[:, rows], y_ref, S, f"gemm long K fmt={fmt}")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q5_1], ids=FID.get)
def test_gemv_mfma_long_k(fmt):
    M, K, N = 300, 2**18, 8
    announce(f"gemv mfma long K fmt={fmt} M={M} K={K} N={N}")
    W = si.device_weights(fmt, M, K, 9100 + fmt, "cuda")
    x = si.activations(N, K, 9101)
    y = qmm.gemv(fmt, W, dev(x), M, K, variant=qmm.QMM_VARIANT_MFMA).cpu().numpy()
    rows = sample_rows(M, 40, 9102)
    raw = _rows_bytes(W, fmt, K, rows)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, len(rows), K)
    check_linear(y[:, rows], y_ref, S, f"gemv mfma long K fmt={fmt}")
