"""Calls captured into a HIP graph and replayed.

The calls run the same kernels eagerly and under capture.  Those captured here use a
caller workspace (allocated before the capture): the small-batch MFMA GEMV (tokens
scaled to fp16 there, split-K partials) and the tiled GEMM on few tiles (split-K
partials); the test asserts that each shape does split K.  Each graph is replayed
several times with eager work (on a workspace of its own) and synchronisations in
between, and every replay is checked against the oracle and against the first replay.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_residual, check_swiglu, dev

pytestmark = pytest.mark.gpu

MFMA = qmm.QMM_VARIANT_MFMA


def _replays(g, out, eager_noise):
    got = []
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        got.append(out.cpu().numpy().copy())
        eager_noise()  # unrelated eager work between replays
        torch.cuda.synchronize()
    for r in range(1, 3):
        assert np.array_equal(got[r], got[0]), f"replay {r} differs from replay 0"
    return got[0]


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q4_1, si.FMT_Q5_0, si.FMT_Q5_1],
                         ids=["q8_0", "q4_0", "q4_1", "q5_0", "q5_1"])
def test_graph_gemv_small_batch_and_n1(fmt):
    M, K = 1024, 4096
    raw = si.weights(fmt, M, K, 7001, scale_mode="gemm_wide", q8_low=-128)
    x16 = si.activations(16, K, 7002)
    x1 = si.activations(1, K, 7003)
    Wd, x16d, x1d = dev(raw), dev(x16), dev(x1)
    y16 = torch.empty((16, M), device="cuda")
    y1 = torch.empty((1, M), device="cuda")
    scratch = torch.empty((16, M), device="cuda")
    need = qmm.qmm_workspace_size(qmm.QMM_OP_GEMV, fmt, M, K, 16, MFMA)
    assert need > 16 * K * 2 + 256, "this shape splits K (partials in the workspace)"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_noise = torch.empty(need, dtype=torch.uint8, device="cuda")
    announce(f"graph capture: gemv N=16 (mfma) + N=1, fmt={fmt} M={M} K={K}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmm.qmm_gemv_variant(fmt, Wd, x16d, y16, M, K, 16, MFMA, ws)
        qmm.qmm_gemv(fmt, Wd, x1d, y1, M, K, 1)
    torch.cuda.synchronize()

    def noise():
        qmm.qmm_gemv_variant(fmt, Wd, x16d, scratch, M, K, 16, MFMA, ws_noise)

    got16 = _replays(g, y16, noise)
    y_ref, S = oracle.matmul_ref(fmt, raw, x16, M, K)
    check_linear(got16, y_ref, S, f"graph gemv mfma fmt={fmt}")
    y_ref1, S1 = oracle.matmul_ref(fmt, raw, x1, M, K)
    check_linear(y1.cpu().numpy(), y_ref1, S1, f"graph gemv N=1 fmt={fmt}")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_F16, si.FMT_Q5_0, si.FMT_Q5_1],
                         ids=["q8_0", "q4_0", "f16", "q5_0", "q5_1"])
def test_graph_gemm_few_tiles(fmt):
    M, K, T = 300, 2816, 40  # 2 tiles: split-K outside of capture
    raw = si.weights(fmt, M, K, 7101, scale_mode="gemm_wide", q8_low=-128)
    X = si.activations(T, K, 7102, dtype=np.float16)
    Wd, Xd = dev(raw), dev(X)
    Y = torch.empty((T, M), device="cuda")
    scratch = torch.empty((T, M), device="cuda")
    need = qmm.qmm_workspace_size(qmm.QMM_OP_GEMM, fmt, M, K, T)
    assert need >= 2 * T * M * 4, "this shape splits K"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_noise = torch.empty(need, dtype=torch.uint8, device="cuda")
    announce(f"graph capture: gemm split-K shape fmt={fmt} M={M} K={K} T={T}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmm.qmm_gemm(fmt, Wd, Xd, Y, M, K, T, ws)
    torch.cuda.synchronize()

    def noise():
        qmm.qmm_gemm(fmt, Wd, Xd, scratch, M, K, T, ws_noise)

    got = _replays(g, Y, noise)
    y_ref, S = oracle.matmul_ref(fmt, raw, X, M, K)
    check_linear(got, y_ref, S, f"graph gemm fmt={fmt}")


def test_graph_gemm_gate_up_few_tiles():
    fmt, I, K, T = si.FMT_Q8_0, 200, 2816, 24
    rg, ru = si.weights(fmt, I, K, 7201), si.weights(fmt, I, K, 7202)
    X = si.activations(T, K, 7203, dtype=np.float16)
    g_d, u_d, Xd = dev(rg), dev(ru), dev(X)
    H = torch.empty((T, I), device="cuda")
    need = qmm.qmm_workspace_size(qmm.QMM_OP_GEMM_GATE_UP_SILU, fmt, I, K, T)
    assert need >= 2 * T * 2 * I * 4, "this shape splits K"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_noise = torch.empty(need, dtype=torch.uint8, device="cuda")
    announce(f"graph capture: gemm gate_up split-K shape I={I} K={K} T={T}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmm.qmm_gemm_gate_up_silu(fmt, g_d, u_d, Xd, H, I, K, T, ws)
    torch.cuda.synchronize()
    got = _replays(g, H, lambda: qmm.qmm_gemm_gate_up_silu(fmt, g_d, u_d, Xd, torch.empty_like(H), I, K, T,
                                                            ws_noise))
    h_ref, gg, uu, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, X, I, K)
    check_swiglu(got, h_ref, gg, uu, Sg, Su, "graph gemm gate_up")


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q5_1], ids=["q8_0", "q4_0", "q5_1"])
def test_graph_decode_chain(fmt):
    """One decode layer's projections as a replayed graph, on the kernels the 8B step uses:
    RMSNorm + GEMV on the DMA-fed kernel (3072 rows), RMSNorm + gate/up on the gated
    kernel, and the down projection with the residual added, fed by the gate/up output of
    the same graph (DMA-fed, 4096 rows).  Every replay equals the eager calls bit for bit,
    and the chain matches the oracle."""
    H, Q, I = 4096, 3072, 3072
    eps = 1e-5
    rq = si.weights(fmt, Q, H, 7201)
    rg = si.weights(fmt, I, H, 7202)
    ru = si.weights(fmt, I, H, 7203)
    rd = si.weights(fmt, H, I, 7204)
    x = si.activations(1, H, 7205)
    gamma = (1.0 + 0.1 * si.activations(1, H, 7206)[0]).astype(np.float32)
    Wq, Wg, Wu, Wd, xd, gd = dev(rq), dev(rg), dev(ru), dev(rd), dev(x), dev(gamma)
    a = torch.empty((1, Q), device="cuda")
    h = torch.empty((1, I), device="cuda")
    y = torch.empty((1, H), device="cuda")

    def chain():
        qmm.qmm_rmsnorm_gemv(fmt, Wq, xd, gd, eps, a, Q, H, 1)
        qmm.qmm_rmsnorm_gate_up_silu(fmt, Wg, Wu, xd, gd, eps, h, I, H, 1)
        qmm.qmm_gemv_add(fmt, Wd, h, xd, y, H, I, 1)

    announce(f"graph capture: decode chain fmt={fmt} H={H} Q={Q} I={I}")
    chain()
    torch.cuda.synchronize()
    eager = [t.cpu().numpy().copy() for t in (a, h, y)]
    for t in (a, h, y):
        t.fill_(float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        chain()
    torch.cuda.synchronize()
    scratch = torch.empty((1, Q), device="cuda")

    def noise():
        qmm.qmm_gemv(fmt, Wq, xd, scratch, Q, H, 1)

    for r in range(3):
        for t in (a, h, y):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip("ahy", (a, h, y), eager):
            assert np.array_equal(t.cpu().numpy(), e), f"replay {r}: {name} differs from the eager call"
        noise()
        torch.cuda.synchronize()

    a_ref, S = oracle.rmsnorm_matmul_ref(fmt, rq, x, gamma, eps, Q, H)
    check_linear(eager[0], a_ref, S, f"graph chain rmsnorm gemv fmt={fmt}")
    h_ref, gg, uu, Sg, Su = oracle.rmsnorm_gate_up_silu_ref(fmt, rg, ru, x, gamma, eps, I, H)
    check_swiglu(eager[1], h_ref, gg, uu, Sg, Su, f"graph chain gate_up fmt={fmt}")
    yd, Sd = oracle.matmul_ref(fmt, rd, eager[1], H, I)  # on the h the GPU produced
    check_residual(eager[2], yd + x.astype(np.float64), Sd, f"graph chain down + residual fmt={fmt}")
