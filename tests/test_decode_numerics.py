"""CPU model of the decode kernels' arithmetic and its error bound.

The register-decode GEMV kernels (gemv_dma.hip, gemv_stream.hpp, via block_dot in
gemv_block.hpp) hold x in block floating point and form their products with
v_dot2_f32_f16.  This file models that arithmetic step by step in numpy (each dot2
step is the exact sum rounded once to fp32; the hardware is within an fp32 ulp of
that) and checks it against the float64 oracle:

* the construction of tests/near_offset.py breaks the 2e-3 * S + 1e-6 bound under
  the earlier offset-code form (p = sum v x~ and c = sum v0 x~ rounded separately,
  and the biased formats' d sum u x + m sum x), which is what the construction is
  for;
* the exact-code form the kernels use now (the offset removed in fp16 before the
  dot2 steps, and the biased blocks split around their integer centre) meets the
  stated worst-case bound (2^-11 + 3 (25 + K/2048) 2^-23)(1 + 2^-11) S there, on
  random blocks and on random near-offset blocks;
* the wide-block test (an unsigned key of |x| against the key of 2^(-14 - s))
  flags exactly the blocks holding a nonzero element that would not be a normal
  fp16 after scaling.

The oracle is the reference; the model here is test code, not part of either side.
The bound follows the "alpaca.swift" page's Numerical validation (each
reduced-precision step checked against a derived element-wise bound).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import near_offset

F32 = np.float32


def _stage(xb: np.ndarray):
    """One block of x: (x~ as float64 [32], 2^-s), as block_scale / stage_block."""
    m = np.float32(np.max(np.abs(xb)))
    e = int((np.array(m, dtype=np.float32).view(np.uint32) >> 23) & 0xFF) - 127
    se = min(126, 14 - e)
    xt = (xb.astype(np.float64) * 2.0 ** se).astype(np.float16).astype(np.float64)
    return xt, 2.0 ** -se


def _chain(codes: np.ndarray, xt: np.ndarray) -> np.float32:
    """16 dot2 steps over consecutive pairs: acc = fp32(acc + c0 x0 + c1 x1)."""
    a = 0.0
    for i in range(0, 32, 2):
        a = float(F32(a + codes[i] * xt[i] + codes[i + 1] * xt[i + 1]))
    return F32(a)


def _split(fmt, c, d16, m16):
    """Per block: d (fp32), m (fp32 or 0) and the integer codes u (biased: raw code)."""
    d = d16.astype(np.float32)
    m = m16.astype(np.float32) if m16 is not None else np.zeros_like(d)
    return d, m


def model_new(fmt, c, d16, m16, x):
    """The exact-code arithmetic of block_dot: y[n][r] in fp32."""
    M, K = c.shape
    nb = K // 32
    N = x.shape[0]
    d, m = _split(fmt, c, d16, m16)
    F = 64.0 if fmt in (oracle.FMT_Q5_0, oracle.FMT_Q5_1) else 1.0
    unit = 1.0 / F
    y = np.zeros((N, M), dtype=np.float32)
    for n in range(N):
        staged = [_stage(x[n, 32 * b:32 * b + 32]) for b in range(nb)]
        for r in range(M):
            acc = F32(0.0)
            for b in range(nb):
                xt, inv = staged[b]
                u = c[r, 32 * b:32 * b + 32].astype(np.float64)
                db, mb = d[r, b], m[r, b]
                if fmt in (oracle.FMT_Q4_1, oracle.FMT_Q5_1):
                    t = -float(mb) / float(db) if db != 0 else float("nan")
                    cen = int(min(max(t + 0.5, 0.0), 31.0)) if t <= 62.0 else 0
                    rr = F32(float(mb) + cen * float(db))   # fmaf(c, d, m)
                    X = _chain(np.ones(32), xt)
                    p = _chain((u - cen) * unit, xt)
                    blk = F32(float(rr) * float(X) + float(F32(float(p) * float(F32(db * F)))))
                else:
                    p = _chain((u - near_offset.ZERO[fmt]) * unit, xt)
                    blk = F32(float(p) * float(F32(db * F)))
                acc = F32(float(blk) * inv + float(acc))
            y[n, r] = acc
    return y


def model_old(fmt, c, d16, m16, x):
    """The earlier offset-code arithmetic: p = sum v x~ and c = sum v0 x~ as two dot2
    chains, a block adding (p - c) d F 2^-s; the biased formats' bias term m sum x~."""
    M, K = c.shape
    nb = K // 32
    N = x.shape[0]
    d, m = _split(fmt, c, d16, m16)
    if fmt == oracle.FMT_Q8_0:
        v = lambda u: 1024.0 + (u + 128.0)
        v0, F = 1152.0, 1.0
    elif fmt == oracle.FMT_Q4_0:
        v = lambda u: 1.0 + u / 64.0
        v0, F = 1.125, 64.0
    else:  # Q4_1 / Q5_1
        v = lambda u: 1.0 + u / 64.0
        v0, F = 1.0, 64.0
    y = np.zeros((N, M), dtype=np.float32)
    for n in range(N):
        staged = [_stage(x[n, 32 * b:32 * b + 32]) for b in range(nb)]
        for r in range(M):
            acc = F32(0.0)
            for b in range(nb):
                xt, inv = staged[b]
                u = c[r, 32 * b:32 * b + 32].astype(np.float64)
                p = _chain(v(u), xt)
                cc = _chain(np.full(32, v0), xt)
                pc = F32(float(p) - float(cc))
                t = F32(float(pc) * float(F32(d[r, b] * F)))
                if fmt in (oracle.FMT_Q4_1, oracle.FMT_Q5_1):
                    t = F32(float(m[r, b]) * float(cc) + float(t))
                acc = F32(float(t) * inv + float(acc))
            y[n, r] = acc
    return y


def proven_bound(S, K):
    return (2.0 ** -11 + 3 * (25 + K / 2048) * 2.0 ** -23) * (1 + 2.0 ** -11) * S


def _ref(fmt, raw, x, M, K):
    return oracle.matmul_ref(fmt, raw, x, M, K)


@pytest.mark.parametrize("fmt", [oracle.FMT_Q8_0, oracle.FMT_Q4_0, oracle.FMT_Q4_1])
def test_offset_code_form_breaks_bound_on_near_offset_blocks(fmt):
    """The construction is sharp: the earlier arithmetic misses the bound on it."""
    M, K = 6, 4096
    c, d16, m16 = near_offset.codes(fmt, M, K)
    raw = near_offset.weights(fmt, M, K)
    x = near_offset.activations(4, K)
    y_ref, S = _ref(fmt, raw, x, M, K)
    y = model_old(fmt, c, d16, m16, x)
    ratio = np.abs(y.astype(np.float64) - y_ref) / oracle.tol_linear(S)
    assert ratio.max() > 5.0, ratio.max()


@pytest.mark.parametrize("fmt", [oracle.FMT_Q8_0, oracle.FMT_Q4_0, oracle.FMT_Q4_1, oracle.FMT_Q5_0,
                                 oracle.FMT_Q5_1])
def test_exact_code_form_meets_bound_on_near_offset_blocks(fmt):
    M, K = 6, 4096
    c, d16, m16 = near_offset.codes(fmt, M, K)
    raw = near_offset.weights(fmt, M, K)
    x = near_offset.activations(4, K)
    y_ref, S = _ref(fmt, raw, x, M, K)
    y = model_new(fmt, c, d16, m16, x)
    err = np.abs(y.astype(np.float64) - y_ref)
    assert (err <= proven_bound(S, K)).all(), (err / S).max()
    assert (err <= oracle.tol_linear(S)).all()


def _random_codes(fmt, g, M, K, near):
    nb = K // 32
    if fmt == oracle.FMT_Q8_0:
        c = g.integers(-1, 2, (M, K)) if near else g.integers(-128, 128, (M, K))
    else:
        top = 16 if fmt in (oracle.FMT_Q4_0, oracle.FMT_Q4_1) else 32
        z = near_offset.ZERO[fmt]
        c = z + g.integers(-1, 2, (M, K)) if near else g.integers(0, top, (M, K))
    d16 = g.uniform(1e-3, 1e-2, (M, nb)).astype(np.float16) * np.where(g.random((M, nb)) < 0.5, -1, 1).astype(np.float16)
    m16 = None
    if fmt in (oracle.FMT_Q4_1, oracle.FMT_Q5_1):
        # Biases anywhere from far below to far above the code range (the centre clamps).
        m16 = (d16.astype(np.float64) * g.uniform(-90, 8, (M, nb))).astype(np.float16)
    return c, d16, m16


def _pack(fmt, c, d16, m16):
    if fmt == oracle.FMT_Q8_0:
        return oracle.pack_q8_0(c, d16)
    if fmt == oracle.FMT_Q4_0:
        return oracle.pack_q4_0(c, d16)
    if fmt == oracle.FMT_Q4_1:
        return oracle.pack_q4_1(c, d16, m16)
    if fmt == oracle.FMT_Q5_0:
        return oracle.pack_q5_0(c, d16)
    return oracle.pack_q5_1(c, d16, m16)


@pytest.mark.parametrize("near", [False, True])
@pytest.mark.parametrize("fmt", [oracle.FMT_Q8_0, oracle.FMT_Q4_0, oracle.FMT_Q4_1, oracle.FMT_Q5_0,
                                 oracle.FMT_Q5_1])
def test_exact_code_form_meets_bound_on_random_blocks(fmt, near):
    """Random codes (or codes within one step of the zero code) with x that mixes
    N(0, 1) values and values down to 1e-6 of them in the same blocks."""
    g = np.random.default_rng(100 + fmt + 10 * near)
    M, K = 5, 512
    c, d16, m16 = _random_codes(fmt, g, M, K, near)
    raw = _pack(fmt, c, d16, m16)
    x = si.activations(3, K, 7)
    x[1] *= np.float32(1e-6) ** g.random(K).astype(np.float32)
    x[2, ::3] = 0.0
    y_ref, S = _ref(fmt, raw, x, M, K)
    y = model_new(fmt, c, d16, m16, x)
    err = np.abs(y.astype(np.float64) - y_ref)
    assert (err <= proven_bound(S, K) + 1e-30).all(), (err / np.maximum(S, 1e-300)).max()


def _key(v: np.ndarray) -> np.ndarray:
    """mag_key: 2 * bits(|v|) - 2 as uint32 (zeros wrap to the top)."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b << 1) - 2) & 0xFFFFFFFF


def _wide_flag(xb: np.ndarray) -> bool:
    m = np.float32(np.max(np.abs(xb)))
    e = int((np.array(m, dtype=np.float32).view(np.uint32) >> 23) & 0xFF) - 127
    se = min(126, 14 - e)
    thr = np.float32(2.0 ** (-14 - se))
    return bool(_key(xb).min() < _key(np.array([thr]))[0])


def test_wide_key_flags_exactly_the_subnormal_elements():
    """The staging kernels' wide test against its definition: some nonzero element
    x with 2^s |x| below 2^-14, the smallest normal fp16."""
    g = np.random.default_rng(5)
    seen = {True: 0, False: 0}
    for trial in range(4000):
        xb = g.standard_normal(32).astype(np.float32)
        k = g.integers(0, 32)
        xb[k] = np.float32(xb[k] * 2.0 ** -float(g.uniform(20, 36)))  # dynamic range around 2^28
        if trial % 7 == 0:
            xb[g.integers(0, 32)] = 0.0
        if trial % 11 == 0:
            xb[:] = 0.0
        if trial % 13 == 0:
            xb *= np.float32(2.0 ** float(g.integers(-140, 120)))
        m = float(np.max(np.abs(xb.astype(np.float64))))
        e = int((np.array(np.float32(m), dtype=np.float32).view(np.uint32) >> 23) & 0xFF) - 127
        se = min(126, 14 - e)
        scaled = np.abs(xb.astype(np.float64)) * 2.0 ** se
        want = bool(((scaled < 2.0 ** -14) & (xb != 0)).any())
        assert _wide_flag(xb) == want, (trial, xb)
        seen[want] += 1
    assert seen[True] > 100 and seen[False] > 100, seen


@pytest.mark.parametrize("fmt", [oracle.FMT_Q4_1, oracle.FMT_Q5_1])
def test_exact_code_form_one_hot_returns_the_rounded_weight(fmt):
    """x = e_k gives d u + m rounded once to fp32 for every bias, because the block's
    r = m + c d is exact: biases from -100 d to +10 d cross every branch of the centre
    (inside the code range, clamped at 31 up to -62 d, and c = 0 beyond), with scales
    of both signs over a wide range of exponents."""
    g = np.random.default_rng(fmt)
    M, K = 64, 64
    nb = K // 32
    top = 16 if fmt == oracle.FMT_Q4_1 else 32
    c = g.integers(0, top, (M, K))
    d16 = (g.uniform(0.5, 1.0, (M, nb)) * 2.0 ** g.integers(-20, 8, (M, nb))).astype(np.float16)
    d16 *= np.where(g.random((M, nb)) < 0.5, -1, 1).astype(np.float16)
    m16 = (d16.astype(np.float64) * g.uniform(-100, 10, (M, nb))).astype(np.float16)
    cols = [0, 5, 17, 31, 32, 63]
    x = si.one_hot(len(cols), K, cols)
    y = model_new(fmt, c, d16, m16, x)
    W32 = oracle.dequant(fmt, _pack(fmt, c, d16, m16), M, K).astype(np.float32)
    for n, k in enumerate(cols):
        assert np.array_equal(y[n], W32[:, k]), (n, k)
