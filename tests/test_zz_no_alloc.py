"""qmm_gemm_noalloc, the GEMM that allocates nothing, against qmm_gemm with a workspace.

Two calls in a row through the C ABI, the second on a smaller input; both shapes split
K, so their partial sums pass through the library's fixed scratch array (the second
call finds the first call's partials there).  Each result must equal qmm_gemm's bit for
bit (the same kernels, the same fixed-order reduction) and meet the oracle's bound on
sampled rows.  Outputs start as NaN.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, dev, sample_rows

pytestmark = pytest.mark.gpu

# (fmt, M, K, T): a Llama-3-8B down projection at 128 tokens (16 row tiles, K split 16
# ways, 33.5 MB of partials), then a smaller Q4_0 matrix at 40 tokens.
CASES = [(si.FMT_Q8_0, 4096, 14336, 128), (si.FMT_Q4_0, 1000, 4096, 40)]


def test_gemm_noalloc_matches_gemm_twice():
    for i, (fmt, M, K, T) in enumerate(CASES):
        need = qmm.qmm_workspace_size(qmm.QMM_OP_GEMM, fmt, M, K, T)
        assert 0 < need <= qmm.QMM_NOALLOC_SCRATCH_BYTES, "the shape splits K and fits the scratch"
        seed = 9100 + 10 * i
        raw = si.weights(fmt, M, K, seed)
        X = si.activations(T, K, seed + 1, dtype=np.float16)
        Wd, Xd = dev(raw), dev(X)
        announce(f"gemm_noalloc call {i}: fmt={fmt} M={M} K={K} T={T} (workspace {need} bytes)")
        Y_ws = torch.full((T, M), float("nan"), device="cuda")
        qmm.qmm_gemm(fmt, Wd, Xd, Y_ws, M, K, T, torch.empty(need, dtype=torch.uint8, device="cuda"))
        Y = torch.full((T, M), float("nan"), device="cuda")
        qmm.qmm_gemm_noalloc(fmt, Wd, Xd, Y, M, K, T)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ws), f"call {i}: differs from qmm_gemm"
        rows = sample_rows(M, 24, seed + 2)
        y_ref, S = oracle.matmul_ref(fmt, raw, X, M, K, rows=rows)
        check_linear(Y.cpu().numpy()[:, rows], y_ref, S, f"gemm_noalloc call {i}")
