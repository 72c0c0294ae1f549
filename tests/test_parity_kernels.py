"""GPU parity of every C-ABI entry point against the float64 oracle (small and ragged shapes).

Each case poisons its output with NaNs (unwritten elements fail), keeps a guard
band after the output (stray writes fail), and compares element by element:
dequantisation bit-exact, products within 2e-3 * sum|w x| + 1e-6, the SwiGLU
output within the propagated bound.  Invariants with exact answers (one-hot x,
all-zero Q4_0 codes, doubled scales) are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_gguf_amd as qmm
import oracle
import seeded_inputs as si
from parity_util import announce, check_linear, check_swiglu, dev, guard_intact, poisoned

pytestmark = pytest.mark.gpu

FMTS = [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_F16]
FID = {si.FMT_Q8_0: "q8_0", si.FMT_Q4_0: "q4_0", si.FMT_F16: "f16"}
AUTO, VALU, MFMA = qmm.QMM_VARIANT_AUTO, qmm.QMM_VARIANT_VALU, qmm.QMM_VARIANT_MFMA


def _seed(*parts):
    return abs(hash(parts)) % (2**31)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,mode", [(1, 32, "uniform"), (7, 96, "wide"), (33, 576, "uniform"),
                                      (5, 4096, "wide"), (3, 4128, "wide")])
def test_dequant_bit_exact(fmt, M, K, mode):
    seed = 11 + M + K
    raw = si.weights(fmt, M, K, seed, scale_mode=mode, q8_low=-128)
    announce(f"qmm_dequant fmt={fmt} M={M} K={K} mode={mode} seed={seed}")
    buf = poisoned(M * K)
    qmm.qmm_dequant(fmt, dev(raw), buf, M, K)
    torch.cuda.synchronize()
    got = buf[:M * K].cpu().numpy().reshape(M, K).astype(np.float64)
    ref = oracle.dequant(fmt, raw, M, K)
    assert guard_intact(buf, M * K)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_dequant_inf_nan_scales(fmt):
    M, K = 2, 64
    d = np.array([[np.inf, -np.inf], [np.nan, 0.0]], dtype=np.float16)
    if fmt == si.FMT_Q8_0:
        q = np.tile(np.arange(-32, 32, dtype=np.int8), (M, 1))
        raw = oracle.pack_q8_0(q, d)
    else:
        n = np.tile(np.arange(64, dtype=np.uint8) % 16, (M, 1))
        raw = oracle.pack_q4_0(n, d)
    announce(f"qmm_dequant inf/nan scales fmt={fmt}")
    out = qmm.dequant(fmt, dev(raw), M, K)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.dequant(fmt, raw, M, K)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


# ------------------------------------------------------------------ GEMV
GEMV_SHAPES = [(1, 32, 1), (3, 64, 2), (17, 96, 1), (576, 576, 1), (100, 1536, 3), (70, 4096, 4),
               (33, 4128, 1), (20, 4160, 5), (64, 2048, 16), (9, 14336, 2)]


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", GEMV_SHAPES)
@pytest.mark.parametrize("variant", [VALU, MFMA], ids=["valu", "mfma"])
def test_gemv(fmt, M, K, N, variant):
    seed = 1000 + M * 3 + K + N
    mode = "gemm_wide" if (M + K) % 3 == 0 else "uniform"
    raw = si.weights(fmt, M, K, seed, scale_mode=mode, q8_low=-128)
    x = si.activations(N, K, seed + 1)
    announce(f"qmm_gemv_variant fmt={fmt} M={M} K={K} N={N} variant={variant} seed={seed} mode={mode}")
    buf = poisoned(N * M)
    qmm.qmm_gemv_variant(fmt, dev(raw), dev(x), buf, M, K, N, variant)
    torch.cuda.synchronize()
    got = buf[:N * M].cpu().numpy().reshape(N, M)
    assert guard_intact(buf, N * M)
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(got, y_ref, S, f"gemv fmt={fmt} M={M} K={K} N={N} v={variant}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K", [(40, 96), (130, 4160), (5, 14336)])
def test_gemv_one_hot_bit_exact(fmt, M, K):
    """x = e_k gives the decoded column exactly (VALU) or its fp16 rounding (MFMA)."""
    raw = si.weights(fmt, M, K, 77 + K, scale_mode="gemm_wide", q8_low=-128)
    cols = [0, 1, 31, 32, K // 2 + 17, K - 1]
    x = si.one_hot(len(cols), K, cols)
    W = oracle.dequant(fmt, raw, M, K)
    announce(f"one-hot gemv fmt={fmt} M={M} K={K} N={len(cols)}")
    y_valu = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=VALU)
    y_mfma = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=MFMA)
    torch.cuda.synchronize()
    yv = y_valu.cpu().numpy().astype(np.float64)
    ym = y_mfma.cpu().numpy().astype(np.float64)
    for n, c in enumerate(cols):
        assert np.array_equal(yv[n], W[:, c]), (n, c)
        assert np.array_equal(ym[n], oracle.fp16_round(W[:, c])), (n, c)


def test_q4_0_zero_codes_give_zero():
    M, K, N = 37, 576, 3
    d = np.full((M, K // 32), 0.75, dtype=np.float16)
    raw = oracle.pack_q4_0(np.full((M, K), 8, dtype=np.uint8), d)
    x = si.activations(N, K, 5)
    announce("q4_0 all-0x88 gemv")
    for v in (VALU, MFMA):
        y = qmm.gemv(si.FMT_Q4_0, dev(raw), dev(x), M, K, variant=v)
        torch.cuda.synchronize()
        assert (y.cpu().numpy() == 0).all()


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
def test_doubled_scales_double_output(fmt):
    """Scaling every d by 2 scales every product and partial sum by 2 exactly."""
    M, K, N = 300, 4096, 2
    blk_t = si.Q8_0_BLOCK if fmt == si.FMT_Q8_0 else si.Q4_0_BLOCK
    raw = si.weights(fmt, M, K, 31)
    raw2 = raw.copy()
    b2 = raw2.view(blk_t)
    b2["d"] = (b2["d"].astype(np.float32) * 2).astype(np.float16)
    x = si.activations(N, K, 32)
    announce(f"doubled scales fmt={fmt}")
    y1 = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=VALU)
    y2 = qmm.gemv(fmt, dev(raw2), dev(x), M, K, variant=VALU)
    torch.cuda.synchronize()
    assert torch.equal(y2, 2 * y1)


def test_gemv_row_permutation():
    fmt, M, K = si.FMT_Q8_0, 64, 576
    raw = si.weights(fmt, M, K, 8)
    perm = np.random.default_rng(3).permutation(M)
    rawp = raw.reshape(M, -1)[perm].reshape(-1)
    x = si.activations(1, K, 9)
    announce("row permutation gemv")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=VALU)
    yp = qmm.gemv(fmt, dev(rawp), dev(x), M, K, variant=VALU)
    torch.cuda.synchronize()
    assert torch.equal(yp[0], y[0][torch.from_numpy(perm).cuda()])


def test_gemv_auto_matches_choice():
    fmt, M, K = si.FMT_Q4_0, 96, 576
    raw = si.weights(fmt, M, K, 12)
    for N in (1, 4, 8, 16):
        x = si.activations(N, K, 13 + N)
        announce(f"qmm_gemv auto N={N}")
        buf = poisoned(N * M)
        qmm.qmm_gemv(fmt, dev(raw), dev(x), buf, M, K, N)
        torch.cuda.synchronize()
        y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
        check_linear(buf[:N * M].cpu().numpy().reshape(N, M), y_ref, S, f"auto N={N}")
        assert guard_intact(buf, N * M)


# The MFMA variant for a handful of tokens (N <= 32, K % 256 == 0) streams the weights
# once and runs the dot products on the matrix cores; shapes cover one and two token
# fragments, ragged M, a single weight stage (K = 256), long K (split over workgroups)
# and the partial last split.
@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0], ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(300, 2048, 5), (1000, 4096, 17), (33, 256, 32), (513, 14336, 9),
                                   (257, 1280, 2), (4096, 768, 16)])
def test_gemv_mfma_small_batch(fmt, M, K, N):
    seed = 2500 + M + K + N
    raw = si.weights(fmt, M, K, seed, scale_mode="gemm_wide", q8_low=-128)  # fp16(d*q) stays finite
    x = si.activations(N, K, seed + 1)
    announce(f"qmm_gemv_variant mfma small-batch fmt={fmt} M={M} K={K} N={N} seed={seed}")
    buf = poisoned(N * M)
    qmm.qmm_gemv_variant(fmt, dev(raw), dev(x), buf, M, K, N, MFMA)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * M)
    # The oracle takes the caller's fp32 x; the kernel's own fp16 scaling must meet the bound.
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(buf[:N * M].cpu().numpy().reshape(N, M), y_ref, S, f"gemv mfma fmt={fmt} M={M} K={K} N={N}")


# -------------------------------------------------------------- gate + up
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,N", [(1, 32, 1), (96, 128, 2), (1536, 576, 1), (300, 4096, 3), (64, 576, 8),
                                   (50, 4160, 4), (130, 96, 20), (200, 4096, 16), (130, 256, 3), (200, 2816, 24)])
@pytest.mark.parametrize("variant", [AUTO, VALU, MFMA], ids=["auto", "valu", "mfma"])
def test_gate_up_silu(fmt, I, K, N, variant):
    seed = 2000 + I + K + N
    rg = si.weights(fmt, I, K, seed)
    ru = si.weights(fmt, I, K, seed + 1)
    x = si.activations(N, K, seed + 2) * 2.0
    announce(f"qmm_gate_up_silu_variant fmt={fmt} I={I} K={K} N={N} variant={variant} seed={seed}")
    buf = poisoned(N * I)
    qmm.qmm_gate_up_silu_variant(fmt, dev(rg), dev(ru), dev(x), buf, I, K, N, variant)
    torch.cuda.synchronize()
    assert guard_intact(buf, N * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    check_swiglu(buf[:N * I].cpu().numpy().reshape(N, I), h_ref, g, u, Sg, Su, f"gate_up fmt={fmt}")


def test_gate_up_concatenated_buffer():
    """A [gate; up] buffer passed as (base, base + I * row_bytes)."""
    fmt, I, K, N = si.FMT_Q8_0, 192, 576, 1
    rg, ru = si.weights(fmt, I, K, 41), si.weights(fmt, I, K, 42)
    cat = dev(np.concatenate([rg, ru]))
    x = si.activations(N, K, 43)
    rb = qmm.qmm_row_bytes(fmt, K)
    h = torch.empty((N, I), dtype=torch.float32, device="cuda")
    announce("gate_up concatenated buffer")
    qmm.qmm_gate_up_silu(fmt, cat.data_ptr(), cat.data_ptr() + I * rb, dev(x), h, I, K, N)
    torch.cuda.synchronize()
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, "gate_up concat")


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,T", [(1, 32, 1), (300, 256, 40), (256, 4096, 256), (513, 96, 300), (64, 4160, 17),
                                   (1000, 576, 513), (520, 1024, 128), (520, 1024, 129)])
def test_gemm(fmt, M, K, T):
    seed = 3000 + M + K + T
    mode = "gemm_wide" if T % 2 else "uniform"
    raw = si.weights(fmt, M, K, seed, scale_mode=mode, q8_low=-128)
    X = si.activations(T, K, seed + 1, dtype=np.float16)
    announce(f"qmm_gemm fmt={fmt} M={M} K={K} T={T} seed={seed} mode={mode}")
    buf = poisoned(T * M)
    qmm.qmm_gemm(fmt, dev(raw), dev(X), buf, M, K, T)
    torch.cuda.synchronize()
    assert guard_intact(buf, T * M)
    y_ref, S = oracle.matmul_ref(fmt, raw, X, M, K)
    check_linear(buf[:T * M].cpu().numpy().reshape(T, M), y_ref, S, f"gemm fmt={fmt} M={M} K={K} T={T}")


# The MFMA GEMV variant above 32 tokens runs the tiled GEMM on fp32 x (converted to
# fp16 while staged); up to 128 tokens with 128-token tiles, beyond with 256.
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,N", [(300, 1024, 40), (257, 2048, 128), (130, 1024, 150)])
def test_gemv_mfma_tile_fp32_x(fmt, M, K, N):
    seed = 3300 + M + K + N
    raw = si.weights(fmt, M, K, seed, scale_mode="gemm_wide", q8_low=-128)
    x = si.activations(N, K, seed + 1)
    announce(f"gemv mfma (tile, fp32 x) fmt={fmt} M={M} K={K} N={N}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=MFMA)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(y.cpu().numpy(), y_ref, S, f"gemv mfma tile fmt={fmt} N={N}")


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
def test_gemm_one_hot_fp16_tile(fmt):
    """X = e_k gives fp16(W[:, k]) exactly: the tile holds d*q rounded to nearest even."""
    M, K = 300, 4160
    raw = si.weights(fmt, M, K, 91, scale_mode="gemm_wide", q8_low=-128)
    cols = list(range(0, K, 97)) + [K - 1]
    X = si.one_hot(len(cols), K, cols, dtype=np.float16)
    announce(f"gemm one-hot fmt={fmt}")
    Y = qmm.gemm(fmt, dev(raw), dev(X), M, K)
    torch.cuda.synchronize()
    W = oracle.dequant(fmt, raw, M, K)
    Yc = Y.cpu().numpy().astype(np.float64)
    for t, c in enumerate(cols):
        assert np.array_equal(Yc[t], oracle.fp16_round(W[:, c])), (t, c)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,T", [(128, 256, 64), (200, 4096, 300), (64, 96, 7)])
def test_gemm_gate_up_silu(fmt, I, K, T):
    seed = 4000 + I + K + T
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    X = si.activations(T, K, seed + 2, dtype=np.float16)
    announce(f"qmm_gemm_gate_up_silu fmt={fmt} I={I} K={K} T={T}")
    buf = poisoned(T * I)
    qmm.qmm_gemm_gate_up_silu(fmt, dev(rg), dev(ru), dev(X), buf, I, K, T)
    torch.cuda.synchronize()
    assert guard_intact(buf, T * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, X, I, K)
    check_swiglu(buf[:T * I].cpu().numpy().reshape(T, I), h_ref, g, u, Sg, Su, f"gemm gate_up fmt={fmt}")


# Split-K: few tiles and a long K make the tiled GEMM split the K loop over several
# workgroups and add the partial sums in a second pass.  Shapes cover uneven splits,
# an F16 K whose step count is odd (last split shorter than the rest), M % 4 != 0
# (scalar reduce path) and the gated epilogue applied after the reduction.
@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("M,K,T", [(300, 2816, 40), (301, 2816, 3), (64, 14336, 130)])
def test_gemm_split_k(fmt, M, K, T):
    if fmt == si.FMT_F16:
        K += 64  # odd number of 64-wide steps
    seed = 5000 + M + K + T
    raw = si.weights(fmt, M, K, seed, scale_mode="gemm_wide", q8_low=-128)
    X = si.activations(T, K, seed + 1, dtype=np.float16)
    announce(f"qmm_gemm split-K fmt={fmt} M={M} K={K} T={T} seed={seed}")
    buf = poisoned(T * M)
    Wd, Xd = dev(raw), dev(X)
    qmm.qmm_gemm(fmt, Wd, Xd, buf, M, K, T)
    torch.cuda.synchronize()
    assert guard_intact(buf, T * M)
    y_ref, S = oracle.matmul_ref(fmt, raw, X, M, K)
    got = buf[:T * M].cpu().numpy().reshape(T, M)
    check_linear(got, y_ref, S, f"gemm split-K fmt={fmt} M={M} K={K} T={T}")
    # The partials are added in a fixed order: a second call gives the same bits.
    buf2 = poisoned(T * M)
    qmm.qmm_gemm(fmt, Wd, Xd, buf2, M, K, T)
    torch.cuda.synchronize()
    assert np.array_equal(buf2[:T * M].cpu().numpy().reshape(T, M), got)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("I,K,T", [(200, 2816, 70), (130, 4096, 9)])
def test_gemm_gate_up_split_k(fmt, I, K, T):
    seed = 6000 + I + K + T
    rg, ru = si.weights(fmt, I, K, seed), si.weights(fmt, I, K, seed + 1)
    X = si.activations(T, K, seed + 2, dtype=np.float16)
    announce(f"qmm_gemm_gate_up_silu split-K fmt={fmt} I={I} K={K} T={T}")
    buf = poisoned(T * I)
    qmm.qmm_gemm_gate_up_silu(fmt, dev(rg), dev(ru), dev(X), buf, I, K, T)
    torch.cuda.synchronize()
    assert guard_intact(buf, T * I)
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, X, I, K)
    check_swiglu(buf[:T * I].cpu().numpy().reshape(T, I), h_ref, g, u, Sg, Su, f"gemm gate_up split-K fmt={fmt}")


def test_stream_argument():
    """Work goes to the stream passed in; results match the default-stream run."""
    fmt, M, K, N = si.FMT_Q8_0, 256, 1536, 2
    raw, x = si.weights(fmt, M, K, 55), si.activations(N, K, 56)
    s = torch.cuda.Stream()
    Wd, xd = dev(raw), dev(x)
    torch.cuda.synchronize()
    announce("explicit stream gemv")
    with torch.cuda.stream(s):
        y1 = torch.empty((N, M), dtype=torch.float32, device="cuda")
        qmm.qmm_gemv(fmt, Wd, xd, y1, M, K, N, stream=s)
    s.synchronize()
    y0 = qmm.gemv(fmt, Wd, xd, M, K)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("fmt", FMTS, ids=FID.get)
@pytest.mark.parametrize("scale", [1e6, 1e30, 1e-35, 1e-42], ids=["1e6", "1e30", "1e-35", "fp32-subnormal"])
@pytest.mark.parametrize("M,K,N", [(300, 1024, 8), (257, 2048, 48)])
def test_mfma_x_beyond_fp16_range(fmt, scale, M, K, N):
    """The MFMA variant scales each token by a power of two before rounding it to fp16,
    so x far outside fp16's range (or inside its subnormals) keeps the bound; every
    token here also has its own magnitude (tokens spread over 1e-6 .. 1 of the scale,
    so that the exact outputs stay inside fp32's range).  8 tokens: the
    weight-streaming MFMA GEMV; 48: the tiled GEMM."""
    seed = 3400 + M + K + N
    raw = si.weights(fmt, M, K, seed, scale_mode="gemm_wide", q8_low=-128)
    spread = np.logspace(-6, 0, N).astype(np.float64)[:, None]
    x = (si.activations(N, K, seed + 1).astype(np.float64) * scale * spread).astype(np.float32)
    announce(f"mfma x range fmt={fmt} scale={scale} M={M} K={K} N={N}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=MFMA)
    torch.cuda.synchronize()
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K)
    check_linear(y.cpu().numpy(), y_ref, S, f"mfma x range fmt={fmt} scale={scale} N={N}")
    rg, ru = raw, si.weights(fmt, M, K, seed + 2, scale_mode="gemm_wide", q8_low=-128)
    xs = (x.astype(np.float64) / max(scale, 1.0)).astype(np.float32)  # keep silu's argument finite
    h = qmm.gate_up_silu(fmt, dev(rg), dev(ru), dev(xs), M, K, variant=MFMA)
    torch.cuda.synchronize()
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, xs, M, K)
    check_swiglu(h.cpu().numpy(), h_ref, g, u, Sg, Su, f"mfma gate_up x range fmt={fmt} scale={scale}")


def _stage_profiles(N, K, seed, big=1e7, high=1e20):
    """fp32 tokens whose magnitude changes along K, so that the weight-streaming MFMA
    GEMV's running per-token scale (one power of two per 128-wide stage and
    workgroup) moves from stage to stage: growing and shrinking ramps over 2^-20 ..
    2^20, a zero prefix, a single element `big` in the last stage, a step from 1e-30
    to `high` half way, an all-zero token, and plain Gaussian tokens.

    The spike stays within about 2^24 of its token's other values: an element more
    than 2^28 below the largest |x| read before it keeps only an absolute error of
    2^-39 times that largest, and where the spike meets a zero weight (a Q4_0 code
    of 8) the bound's sum |w x| does not contain the spike."""
    g = si.activations(N, K, seed).astype(np.float64)
    ramp = np.linspace(-20.0, 20.0, K)
    x = np.empty((N, K), np.float64)
    for n in range(N):
        kind = n % 7
        if kind == 0:
            x[n] = g[n] * np.exp2(ramp)
        elif kind == 1:
            x[n] = g[n] * np.exp2(-ramp)
        elif kind == 2:
            x[n] = np.where(np.arange(K) < K // 2, 0.0, g[n])
        elif kind == 3:
            x[n] = g[n]
            x[n, K - 1 - (n % 128)] = big
        elif kind == 4:
            x[n] = np.where(np.arange(K) < K // 2, 1e-30, high) * g[n]
        elif kind == 5:
            x[n] = 0.0
        else:
            x[n] = g[n]
    return x.astype(np.float32)


# The shapes: split K (2 or 4 stages per workgroup, partials at the tokens' true scale
# summed by the reduce kernel) and unsplit K (129 row tiles or more: 8 stages in one
# workgroup, the epilogue descales); one and two token fragments.  Large matrices are
# checked on their first and last rows.
@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_Q5_1], ids=str)
@pytest.mark.parametrize("M,K,N", [(300, 2048, 8), (8192, 4096, 7), (33024, 1024, 20), (33024, 1024, 3)])
def test_mfma_running_token_scale(fmt, M, K, N):
    seed = 3600 + M + K + N + fmt
    raw = si.weights(fmt, M, K, seed, scale_mode="gemm_wide", q8_low=-128)
    x = _stage_profiles(N, K, seed + 1)
    announce(f"mfma running scale fmt={fmt} M={M} K={K} N={N} seed={seed}")
    y = qmm.gemv(fmt, dev(raw), dev(x), M, K, variant=MFMA)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 512 else np.r_[0:256, M - 256:M]
    y_ref, S = oracle.matmul_ref(fmt, raw, x, M, K, rows=rows)
    got = y.cpu().numpy().reshape(N, M)[:, rows]
    check_linear(got, y_ref, S, f"mfma running scale fmt={fmt} M={M} K={K} N={N}")
    if N > 5:
        assert np.all(got[5::7] == 0.0)  # the all-zero tokens


@pytest.mark.parametrize("fmt", [si.FMT_Q8_0, si.FMT_Q4_1], ids=str)
@pytest.mark.parametrize("I,K,N", [(200, 2048, 8), (16512, 1024, 20)])
def test_mfma_running_token_scale_gate_up(fmt, I, K, N):
    """The gated instance of the same: 200 outputs split K; 16512 outputs (129 tiles
    of 128) keep K whole.  The spike and the step's high side are 1e6, so that
    silu(gate) * up stays inside fp32's range."""
    seed = 3700 + I + K + N + fmt
    rg = si.weights(fmt, I, K, seed, scale_mode="gemm_wide", q8_low=-128)
    ru = si.weights(fmt, I, K, seed + 2, scale_mode="gemm_wide", q8_low=-128)
    x = _stage_profiles(N, K, seed + 1, big=1e6, high=1e6)
    announce(f"mfma running scale gate_up fmt={fmt} I={I} K={K} N={N} seed={seed}")
    h = qmm.gate_up_silu(fmt, dev(rg), dev(ru), dev(x), I, K, variant=MFMA)
    torch.cuda.synchronize()
    rows = np.arange(I) if I <= 512 else np.r_[0:256, I - 256:I]
    h_ref, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rg, ru, x, I, K, rows=rows)
    check_swiglu(h.cpu().numpy().reshape(N, I)[:, rows], h_ref, g, u, Sg, Su,
                 f"mfma running scale gate_up fmt={fmt} I={I} K={K} N={N}")


# ------------------------------------------------------------- streaming-read reference
@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 8191, 16 * 8193, (1 << 20) + 48, (64 << 20) + 16 * 12345])
def test_stream_read_fold(nbytes):
    """qmm_stream_read's per-workgroup XOR folds, bit for bit: the ranges of 16-byte
    units, ceil(units / blocks) long, including sizes that leave trailing workgroups
    with empty ranges (their word is 0) and ragged last ranges."""
    g = np.random.default_rng(nbytes % 1000)
    buf = g.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    B = qmm.QMM_STREAM_READ_BLOCKS
    sink = torch.full((B,), 0xDEADBEEF & 0x7FFFFFFF, dtype=torch.int32, device="cuda")
    announce(f"stream_read fold bytes={nbytes}")
    qmm.qmm_stream_read(torch.from_numpy(buf.view(np.int32)).cuda(), nbytes, sink)
    torch.cuda.synchronize()
    n = nbytes // 16
    per = -(-n // B)
    words = buf.reshape(n, 4)
    want = np.zeros(B, dtype=np.uint32)
    for b in range(B):
        lo, hi = min(b * per, n), min((b + 1) * per, n)
        if hi > lo:
            want[b] = np.bitwise_xor.reduce(words[lo:hi].reshape(-1))
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
