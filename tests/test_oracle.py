"""Pins of the float64 oracle to facts outside itself (CPU only).

Each check is written as a function taking the oracle's pieces as arguments, so
that the mutation tests at the bottom can hand it a deliberately wrong variant
(wrong nibble order, missing offset, unsigned codes, swapped scale, transposed
operand, dropped term) and show that some pin rejects it.
"""
import glob
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from oracle import qmm_oracle as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMT_BY_NAME = {"Q8_0": Q.FMT_Q8_0, "Q4_0": Q.FMT_Q4_0, "F16": Q.FMT_F16, "Q4_1": Q.FMT_Q4_1,
               "Q5_0": Q.FMT_Q5_0, "Q5_1": Q.FMT_Q5_1}
BIAS_FMTS = [Q.FMT_Q4_1, Q.FMT_Q5_0, Q.FMT_Q5_1]


# ----------------------------------------------------------------- fixtures
def load_golden(path):
    fx = {"w": {}, "x": {}}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "fmt":
            fx["fmt"] = FMT_BY_NAME[rest[0]]
        elif key == "bytes":
            fx["bytes"] = bytes(int(b, 16) for b in rest)
        elif key == "w":
            fx["w"][int(rest[0])] = Fraction(rest[1])
            if rest[1].startswith("-") and Fraction(rest[1]) == 0:
                fx.setdefault("negzero", []).append(int(rest[0]))
        elif key == "x":
            fx["x"][int(rest[0])] = Fraction(rest[1])
        elif key == "h":
            fx.setdefault("h", {})[int(rest[0])] = Fraction(rest[1])
        elif key == "xramp":
            fx["x"] = {k: Fraction(k) for k in range(32)}
        elif key == "xones":
            fx["x"] = {k: Fraction(1) for k in range(32)}
        elif key == "dot":
            fx["dot"] = Fraction(rest[0])
    return fx


GOLDEN_FILES = sorted(glob.glob(os.path.join(GOLDEN, "*.txt")))


def check_golden(fx, dequant, matmul):
    K = 32
    w = dequant(fx["fmt"], np.frombuffer(fx["bytes"], np.uint8), 1, K)[0]
    want = np.zeros(K)
    for k, v in fx["w"].items():
        want[k] = float(v)
    if not all(Fraction(float(a)) == Fraction(float(b)) for a, b in zip(w, want)):
        return False
    for k in fx.get("negzero", []):
        if math.copysign(1.0, w[k]) != -1.0:
            return False
    x = np.zeros((1, K), np.float32)
    for k, v in fx["x"].items():
        x[0, k] = float(v)
    y, _ = matmul(fx["fmt"], np.frombuffer(fx["bytes"], np.uint8), x, 1, K)
    return Fraction(float(y[0, 0])) == fx["dot"]


@pytest.mark.parametrize("path", GOLDEN_FILES, ids=os.path.basename)
def test_golden_blocks(path):
    fx = load_golden(path)
    assert check_golden(fx, Q.dequant, Q.matmul_ref)


@pytest.mark.parametrize("path", GOLDEN_FILES, ids=os.path.basename)
def test_golden_blocks_brute_force(path):
    """The byte-by-byte rational decoder agrees with the stored hand values too."""
    fx = load_golden(path)
    xr = [float(fx["x"].get(k, 0)) for k in range(32)]
    (row,) = Q.brute_force_matmul(fx["fmt"], fx["bytes"], [xr], 1, 32)
    assert row[0] == fx["dot"]


def test_golden_fixture_count():
    assert len(GOLDEN_FILES) >= 10
    fmts = {load_golden(p)["fmt"] for p in GOLDEN_FILES}
    assert set(FMT_BY_NAME.values()) <= fmts


# --------------------------------------------- row gather and fp16 expansion
def _golden_by_fmt():
    by = {}
    for p in GOLDEN_FILES:
        fx = load_golden(p)
        by.setdefault(fx["fmt"], []).append(fx)
    return by


def _hand_block(fx):
    want = np.zeros(32)
    for k, v in fx["w"].items():
        want[k] = float(v)
    return want


def check_get_rows(get_rows):
    """A matrix whose rows are strings of golden blocks; gathered rows must show
    those blocks' hand values in order, repeats included, and NaN for bad ids."""
    for fmt, fxs in _golden_by_fmt().items():
        blocks = [(fx["bytes"], _hand_block(fx)) for fx in fxs]
        if len(blocks) == 1:  # a lone fixture: pair it with an all-zero block
            blocks.append((bytes(len(blocks[0][0])), np.zeros(32)))
        nb, M, L = 3, 4, len(blocks)
        K = 32 * nb
        # row r spells r + 1 in base L over its blocks: rows differ, none is a palindrome of row 0
        pick = [[((r + 1) // L ** (nb - 1 - b)) % L for b in range(nb)] for r in range(M)]
        raw = np.frombuffer(b"".join(blocks[i][0] for r in range(M) for i in pick[r]), np.uint8)
        hand = [np.concatenate([blocks[i][1] for i in pick[r]]) for r in range(M)]
        ids = [3, 0, 3, 1, -1, M, 2]
        got = get_rows(fmt, raw, M, K, ids)
        if got.shape != (len(ids), K):
            return False
        for i, r in enumerate(ids):
            if 0 <= r < M:
                if not np.array_equal(got[i], hand[r]):
                    return False
            elif not np.isnan(got[i]).all():
                return False
        if get_rows(fmt, raw, M, K, []).shape != (0, K):
            return False
    return True


def test_get_rows_golden():
    assert check_get_rows(Q.get_rows_ref)


def test_get_rows_pin_catches_mistakes():
    # a wrapped id, an off-by-one row, a zero fill for bad ids, blocks reversed
    wrap = lambda f, raw, M, K, ids: Q.get_rows_ref(f, raw, M, K, np.mod(np.asarray(ids, np.int64), M))
    off1 = lambda f, raw, M, K, ids: Q.get_rows_ref(f, raw, M, K, [i + 1 if 0 <= i < M - 1 else i for i in ids])
    zero = lambda f, raw, M, K, ids: np.nan_to_num(Q.get_rows_ref(f, raw, M, K, ids), nan=0.0)
    rev = lambda f, raw, M, K, ids: Q.get_rows_ref(f, raw, M, K, ids).reshape(len(ids), K // 32, 32)[:, ::-1].reshape(
        len(ids), K)
    for bad in (wrap, off1, zero, rev):
        assert not check_get_rows(bad)


def check_expand(expand):
    n = 0
    for p in GOLDEN_FILES:
        fx = load_golden(p)
        if "h" not in fx:
            continue
        got = expand(fx["fmt"], np.frombuffer(fx["bytes"], np.uint8), 1, 32)
        if got.dtype != np.float16:
            return False
        for k in range(32):
            want = float(fx["h"].get(k, fx["w"].get(k, 0)))
            if Fraction(float(got[0, k])) != Fraction(want):
                return False
        n += 1
    return n >= 1


def test_expand_f16_golden_ties():
    assert check_expand(Q.expand_f16_ref)


def test_expand_pin_catches_truncation():
    # truncation toward zero, and rounding ties away from zero, both differ on the fixture
    def trunc(f, raw, M, K):
        w = Q.dequant(f, raw, M, K)
        h = w.astype(np.float16)
        back = h.astype(np.float64)
        over = np.abs(back) > np.abs(w)
        h[over] = np.nextafter(h[over], np.float16(0))
        return h

    def away(f, raw, M, K):
        w = Q.dequant(f, raw, M, K)
        h = w.astype(np.float16)
        lo = np.nextafter(h, np.float16(0))
        hi = np.nextafter(h, np.where(h < 0, np.float16(-np.inf), np.float16(np.inf)))
        for c in (lo, hi):
            tie = np.abs(c.astype(np.float64) - w) == np.abs(h.astype(np.float64) - w)
            pick = tie & (np.abs(c) > np.abs(h))
            h[pick] = c[pick]
        return h

    def via_fp32(f, raw, M, K):  # two roundings: exact -> fp32 -> fp16
        return Q.dequant(f, raw, M, K).astype(np.float32).astype(np.float16)

    assert not check_expand(trunc)
    assert not check_expand(away)
    assert not check_expand(via_fp32)


# ------------------------------------------------------ RMSNorm and residual
def check_rmsnorm(rmsnorm):
    """Closed forms of x / sqrt(mean(x^2) + eps) * gamma."""
    def close(a, b):
        return np.allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=1e-15, atol=0)

    # mean of (9, 16, 0, 0) is 25/4: rms 2.5
    if not close(rmsnorm([[3, 4, 0, 0]], [1, 2, 3, 4], 0.0), [[1.2, 3.2, 0, 0]]):
        return False
    # eps inside the root: sqrt(1 + 3) = 2
    if not close(rmsnorm([[1, 1, 1, 1]], [2, 4, 6, 8], 3.0), [[1, 2, 3, 4]]):
        return False
    # the mean is over K, whatever K is: a constant row normalises to gamma
    for K in (1, 5, 64):
        if not close(rmsnorm([[2.0] * K], np.arange(K), 0.0), [np.arange(K)]):
            return False
    # token rows are normalised independently
    if not close(rmsnorm([[3, 4, 0, 0], [1, 1, 1, 1]], [1, 1, 1, 1], 0.0), [[1.2, 1.6, 0, 0], [1, 1, 1, 1]]):
        return False
    # a zero row stays zero (eps > 0) and odd symmetry holds
    if not close(rmsnorm([[0.0] * 8], np.ones(8), 1e-5), [[0.0] * 8]):
        return False
    x = np.random.default_rng(1).standard_normal((3, 40))
    g = np.random.default_rng(2).standard_normal(40)
    if not np.allclose(rmsnorm(-x, g, 1e-5), -rmsnorm(x, g, 1e-5), rtol=1e-15, atol=0):
        return False
    return True


def test_rmsnorm_closed_forms():
    assert check_rmsnorm(Q.rmsnorm_ref)


def test_rmsnorm_pin_catches_mistakes():
    def g64(g):
        return np.asarray(g, np.float64)[None, :]

    def x64(x):
        return np.atleast_2d(np.asarray(x, np.float64))

    sum_sq = lambda x, g, e: x64(x) / np.sqrt((x64(x) ** 2).sum(1, keepdims=True) + e) * g64(g)
    eps_out = lambda x, g, e: x64(x) / (np.sqrt((x64(x) ** 2).mean(1, keepdims=True)) + e) * g64(g)
    tok_axis = lambda x, g, e: x64(x) / np.sqrt((x64(x) ** 2).mean(0, keepdims=True) + e) * g64(g)
    no_gamma = lambda x, g, e: x64(x) / np.sqrt((x64(x) ** 2).mean(1, keepdims=True) + e)
    with np.errstate(all="ignore"):
        for bad in (sum_sq, eps_out, tok_axis, no_gamma):
            assert not check_rmsnorm(bad)


@pytest.mark.parametrize("path", GOLDEN_FILES, ids=os.path.basename)
def test_rmsnorm_matmul_golden(path):
    """A constant input row of 2s normalises to exactly gamma; with gamma set to the
    fixture's x the fused product must give the fixture's hand-computed dot."""
    fx = load_golden(path)
    gamma = np.array([float(fx["x"].get(k, 0)) for k in range(32)])
    y, S = Q.rmsnorm_matmul_ref(fx["fmt"], np.frombuffer(fx["bytes"], np.uint8), np.full((1, 32), 2.0), gamma,
                                0.0, 1, 32)
    assert Fraction(float(y[0, 0])) == fx["dot"]
    # eps = 12 with a row of 2s: sqrt(4 + 12) = 4, so gamma is halved
    y2, _ = Q.rmsnorm_matmul_ref(fx["fmt"], np.frombuffer(fx["bytes"], np.uint8), np.full((1, 32), 2.0),
                                 2 * gamma, 12.0, 1, 32)
    assert Fraction(float(y2[0, 0])) == fx["dot"]


@pytest.mark.parametrize("path", GOLDEN_FILES, ids=os.path.basename)
def test_matmul_add_golden(path):
    fx = load_golden(path)
    x = np.array([[float(fx["x"].get(k, 0)) for k in range(32)]])
    y, _ = Q.matmul_add_ref(fx["fmt"], np.frombuffer(fx["bytes"], np.uint8), x, np.array([[0.25]]), 1, 32)
    assert Fraction(float(y[0, 0])) == fx["dot"] + Fraction(1, 4)


def test_rmsnorm_gate_up_is_gate_up_of_the_norm():
    """With a constant input row the norm is gamma itself: the fused FFN reference
    must equal the plain gate+up reference applied to gamma."""
    fmt, I, K = Q.FMT_Q8_0, 5, 64
    rg, ru = si.weights(fmt, I, K, 41), si.weights(fmt, I, K, 42)
    gamma = si.activations(1, K, 43)[0].astype(np.float64)
    h, g, u, Sg, Su = Q.rmsnorm_gate_up_silu_ref(fmt, rg, ru, np.full((1, K), -3.0), gamma, 0.0, I, K)
    h2, g2, u2, _, _ = Q.gate_up_silu_ref(fmt, rg, ru, -gamma[None, :], I, K)
    assert np.array_equal(h, h2) and np.array_equal(g, g2) and np.array_equal(u, u2)


def test_tol_residual_covers_fp32_addition():
    g = np.random.default_rng(5)
    y = g.standard_normal(10000) * 10.0 ** g.integers(-3, 4, 10000)
    r = g.standard_normal(10000) * 10.0 ** g.integers(-3, 4, 10000)
    y32, r32 = y.astype(np.float32), r.astype(np.float32)
    s32 = (y32 + r32).astype(np.float64)
    exact = y32.astype(np.float64) + r32.astype(np.float64)
    assert (np.abs(s32 - exact) <= Q.tol_residual(np.zeros_like(exact), exact)).all()


# ------------------------------------------------------------ fp16 decoding
def manual_f16(h):
    """IEEE binary16 from sign, exponent and mantissa fields with math.ldexp."""
    s = -1.0 if h >> 15 else 1.0
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    if e == 0:
        return s * math.ldexp(m, -24)
    if e == 31:
        return s * math.inf if m == 0 else math.nan
    return s * math.ldexp(1024 + m, e - 25)


def test_fp16_all_patterns_q8_0():
    """Every fp16 scale pattern times codes {-128,-1,0,1,127} decodes as manual IEEE."""
    codes = np.array([-128, -1, 0, 1, 127] + [0] * 27, dtype=np.int8)
    hs = np.arange(65536, dtype=np.uint32)
    raw = np.zeros((65536, 34), np.uint8)
    raw[:, 0] = hs & 0xFF
    raw[:, 1] = hs >> 8
    raw[:, 2:34] = codes.view(np.uint8)
    W = Q.unpack_q8_0(raw.reshape(-1), 65536, 32)
    for h in range(65536):
        d = manual_f16(h)
        for i, c in enumerate(codes[:5]):
            want = d * float(c)
            got = W[h, i]
            if math.isnan(want):
                assert math.isnan(got), (h, c)
            else:
                assert got == want, (h, c, got, want)
                if want == 0:
                    assert math.copysign(1, got) == math.copysign(1, want), (h, c)


def test_fp16_subnormal_example():
    raw = bytes([0x01, 0x00, 0x80] + [0] * 31)
    assert Q.unpack_q8_0(np.frombuffer(raw, np.uint8), 1, 32)[0, 0] == -7.62939453125e-06


# ------------------------------------------------------------ round trips
def test_roundtrip_q8_0():
    g = np.random.default_rng(11)
    M, K = 7, 96
    q = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    q[0, 0], q[0, 1] = -128, 127
    d = g.uniform(-4, 4, size=(M, K // 32)).astype(np.float16)
    raw = Q.pack_q8_0(q, d)
    assert raw.size == M * K // 32 * 34
    W = Q.unpack_q8_0(raw, M, K)
    assert np.array_equal(W, np.repeat(d.astype(np.float64), 32, axis=1) * q)
    assert np.array_equal(Q.pack_q8_0(q, d), raw)


def test_roundtrip_q4_0():
    g = np.random.default_rng(12)
    M, K = 5, 128
    n = g.integers(0, 16, size=(M, K), dtype=np.uint8)
    n[0, :2] = (0, 15)
    d = g.uniform(-4, 4, size=(M, K // 32)).astype(np.float16)
    raw = Q.pack_q4_0(n, d)
    assert raw.size == M * K // 32 * 18
    W = Q.unpack_q4_0(raw, M, K)
    assert np.array_equal(W, np.repeat(d.astype(np.float64), 32, axis=1) * (n.astype(np.float64) - 8))


def _codes_and_scales(g, M, K, bits):
    u = g.integers(0, 1 << bits, size=(M, K), dtype=np.int64)
    u[0, :4] = (0, (1 << bits) - 1, 1 << (bits - 1), 1)
    d = g.uniform(-4, 4, size=(M, K // 32)).astype(np.float16)
    m = g.uniform(-30, 30, size=(M, K // 32)).astype(np.float16)
    return u, d, m


def test_roundtrip_bias_formats():
    """pack -> unpack gives d*u + m (or d*(u-16)) element for element, and the byte
    counts are the pages' 20 / 22 / 24 per block."""
    g = np.random.default_rng(13)
    M, K = 6, 96
    for fmt, bits, bb in ((Q.FMT_Q4_1, 4, 20), (Q.FMT_Q5_0, 5, 22), (Q.FMT_Q5_1, 5, 24)):
        u, d, m = _codes_and_scales(g, M, K, bits)
        if fmt == Q.FMT_Q4_1:
            raw = Q.pack_q4_1(u, d, m)
        elif fmt == Q.FMT_Q5_0:
            raw = Q.pack_q5_0(u, d)
        else:
            raw = Q.pack_q5_1(u, d, m)
        assert raw.size == M * K // 32 * bb
        d64 = np.repeat(d.astype(np.float64), 32, axis=1)
        m64 = np.repeat(m.astype(np.float64), 32, axis=1)
        want = d64 * (u - 16) if fmt == Q.FMT_Q5_0 else d64 * u + m64
        assert np.array_equal(Q.dequant(fmt, raw, M, K), want), fmt


def test_bias_formats_reduce_to_q4_0():
    """Identities between the formats under the adopted layouts, each tying a new
    decoder to the pinned Q4_0 decoder or to another new one:
    Q4_1 with m = -8d is Q4_0; Q5_0 with every fifth bit clear is Q4_0 shifted by
    -8d; Q5_1 with every fifth bit clear is Q4_1; Q5_1 with m = -16d is Q5_0."""
    g = np.random.default_rng(14)
    M, K = 5, 128
    n = g.integers(0, 16, size=(M, K), dtype=np.int64)
    d = g.uniform(-4, 4, size=(M, K // 32)).astype(np.float16)
    m8 = (np.float16(-8) * d).astype(np.float16)       # exact: a power-of-two multiple
    m16 = (np.float16(-16) * d).astype(np.float16)
    q40 = Q.unpack_q4_0(Q.pack_q4_0(n.astype(np.uint8), d), M, K)
    assert np.array_equal(Q.unpack_q4_1(Q.pack_q4_1(n, d, m8), M, K), q40)
    d64 = np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.array_equal(Q.unpack_q5_0(Q.pack_q5_0(n, d), M, K), q40 - 8 * d64)
    m = g.uniform(-9, 9, size=(M, K // 32)).astype(np.float16)
    assert np.array_equal(Q.unpack_q5_1(Q.pack_q5_1(n, d, m), M, K), Q.unpack_q4_1(Q.pack_q4_1(n, d, m), M, K))
    u = g.integers(0, 32, size=(M, K), dtype=np.int64)
    assert np.array_equal(Q.unpack_q5_1(Q.pack_q5_1(u, d, m16), M, K), Q.unpack_q5_0(Q.pack_q5_0(u, d), M, K))


def test_fifth_bits_are_one_word():
    """Setting only bit e of the 32-bit word moves exactly element e up by 16 scales."""
    M, K = 1, 32
    d = np.full((1, 1), 0.5, np.float16)
    base = Q.unpack_q5_0(Q.pack_q5_0(np.zeros((M, K), np.int64), d), M, K)[0]
    for e in (0, 7, 8, 15, 16, 23, 24, 31):
        u = np.zeros((M, K), np.int64)
        u[0, e] = 16
        raw = Q.pack_q5_0(u, d)
        word = int.from_bytes(bytes(raw[2:6]), "little")
        assert word == 1 << e
        diff = Q.unpack_q5_0(raw, M, K)[0] - base
        assert np.flatnonzero(diff).tolist() == [e] and diff[e] == 8.0


def test_bias_exact_in_float64():
    """d*u + m with the extreme fp16 exponents is still exact in float64 (the
    reading's claim): largest d with u = 31 plus the smallest subnormal bias."""
    d = np.full((1, 1), 65504.0, np.float16)
    m = np.full((1, 1), 2.0 ** -24, np.float16)
    u = np.full((1, 32), 31, np.int64)
    w = Q.unpack_q5_1(Q.pack_q5_1(u, d, m), 1, 32)[0, 0]
    assert Fraction(float(w)) == Fraction(65504 * 31) + Fraction(1, 2 ** 24)


def test_row_bytes():
    assert Q.row_bytes(Q.FMT_Q4_1, 4096) == 128 * 20
    assert Q.row_bytes(Q.FMT_Q5_0, 4096) == 128 * 22
    assert Q.row_bytes(Q.FMT_Q5_1, 4096) == 128 * 24
    assert Q.row_bytes(Q.FMT_Q8_0, 576) == 612
    assert Q.row_bytes(Q.FMT_Q4_0, 576) == 324
    assert Q.row_bytes(Q.FMT_F16, 576) == 1152
    assert Q.row_bytes(Q.FMT_Q8_0, 4096) == 4352
    assert Q.row_bytes(Q.FMT_Q4_0, 14336) == 8064
    with pytest.raises(ValueError):
        Q.row_bytes(Q.FMT_Q8_0, 100)


# ------------------------------------------------------------ brute force
def check_brute_force(fmt, M, K, N, seed, matmul, scale_mode="uniform"):
    raw = si.weights(fmt, M, K, seed, scale_mode=scale_mode, q8_low=-128)
    x = si.activations(N, K, seed + 1)
    y, S = matmul(fmt, raw, x, M, K)
    exact = Q.brute_force_matmul(fmt, raw.tobytes(), x.tolist(), M, K)
    for n in range(N):
        for m in range(M):
            err = abs(Fraction(float(y[n, m])) - exact[n][m])
            if err > Fraction(1e-12) * Fraction(float(S[n, m])) + Fraction(1, 10**300):
                return False
    return True


@pytest.mark.parametrize("fmt", [Q.FMT_Q8_0, Q.FMT_Q4_0, Q.FMT_F16] + BIAS_FMTS)
@pytest.mark.parametrize("shape", [(1, 32, 1), (3, 64, 2), (4, 64, 3), (2, 96, 1)])
def test_brute_force(fmt, shape):
    M, K, N = shape
    assert check_brute_force(fmt, M, K, N, 100 + M * 7 + K + N, Q.matmul_ref)


def test_brute_force_square_catches_transpose():
    # Square shapes make a transposed operand type-check, so they are included.
    assert check_brute_force(Q.FMT_Q8_0, 32, 32, 2, 5, Q.matmul_ref)


def test_sampled_rows_match_full():
    fmt, M, K = Q.FMT_Q4_0, 300, 128
    raw = si.weights(fmt, M, K, 3)
    x = si.activations(2, K, 4)
    y, S = Q.matmul_ref(fmt, raw, x, M, K, chunk_rows=64)
    rows = [0, 7, 63, 64, 299]
    ys, Ss = Q.matmul_ref(fmt, raw, x, M, K, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(Ss, S[:, rows])


# --------------------------------------------------------------- SwiGLU
def test_silu_closed_forms():
    assert Q.silu(0.0) == 0.0
    h = 1e-6
    assert abs((Q.silu(h) - Q.silu(-h)) / (2 * h) - 0.5) < 1e-9      # silu'(0) = 1/2
    z = np.linspace(-30, 30, 601)
    assert np.allclose(Q.silu(z) - Q.silu(-z), z, rtol=0, atol=1e-12)  # silu(z) - silu(-z) = z
    assert Q.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert abs(Q.silu(-800.0)) == 0.0
    assert Q.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


def test_silu_slope_bound():
    z = np.linspace(-20, 20, 400001)
    s = 1 / (1 + np.exp(-z))
    slope = s * (1 + z * (1 - s))
    assert np.abs(slope).max() <= Q.SILU_SLOPE_MAX
    assert np.abs(slope).max() > 1.09


def test_swiglu_tolerance_sound():
    """Random g~, u~ inside their linear bounds stay inside tol_swiglu."""
    g0 = np.random.default_rng(7)
    n = 200000
    g = g0.normal(0, 3, n)
    u = g0.normal(0, 3, n)
    Sg = np.abs(g) * g0.uniform(1, 50, n)
    Su = np.abs(u) * g0.uniform(1, 50, n)
    Eg, Eu = Q.tol_linear(Sg), Q.tol_linear(Su)
    gt = g + Eg * g0.uniform(-1, 1, n)
    ut = u + Eu * g0.uniform(-1, 1, n)
    err = np.abs(Q.silu(gt) * ut - Q.silu(g) * u)
    assert (err <= Q.tol_swiglu(g, u, Sg, Su)).all()


def test_gate_up_ref_definition():
    fmt, I, K = Q.FMT_Q8_0, 16, 64
    rg, ru = si.weights(fmt, I, K, 1), si.weights(fmt, I, K, 2)
    x = si.activations(2, K, 3)
    h, g, u, Sg, Su = Q.gate_up_silu_ref(fmt, rg, ru, x, I, K)
    Wg, Wu = Q.dequant(fmt, rg, I, K), Q.dequant(fmt, ru, I, K)
    x64 = x.astype(np.float64)
    assert np.allclose(g, x64 @ Wg.T, rtol=1e-14, atol=0)
    assert np.allclose(h, (x64 @ Wg.T) / (1 + np.exp(-(x64 @ Wg.T))) * (x64 @ Wu.T), rtol=1e-13, atol=0)


def test_fp16_round_ties_even():
    assert Q.fp16_round(2049.0) == 2048.0     # tie -> even mantissa
    assert Q.fp16_round(2051.0) == 2052.0
    assert Q.fp16_round(1.0 + 2 ** -11) == 1.0


# ------------------------------------------------------------ generators
def test_generator_ranges_and_determinism():
    M, K = 64, 256
    a = si.weights(si.FMT_Q8_0, M, K, 9)
    assert np.array_equal(a, si.weights(si.FMT_Q8_0, M, K, 9))
    blk = a.view(si.Q8_0_BLOCK)
    assert blk["qs"].min() >= -127 and blk["qs"].max() <= 127
    d = blk["d"].astype(np.float64)
    assert d.min() >= np.float16(1e-3) and d.max() <= np.float16(1e-2)
    b = si.weights(si.FMT_Q4_0, M, K, 9).view(si.Q4_0_BLOCK)
    nib = np.concatenate([b["qs"] & 15, b["qs"] >> 4])
    counts = np.bincount(nib.reshape(-1), minlength=16)
    assert counts.min() > 0.8 * counts.mean()
    f = si.weights(si.FMT_F16, 256, 256, 9).view(np.float16).astype(np.float64)
    assert abs(f.std() - 0.02) < 0.001


def test_generator_chunking_is_part_of_recipe():
    # Rows beyond one chunk continue the same stream deterministically.
    M, K = si._CHUNK_ROWS + 3, 32
    a = si.weights(si.FMT_Q4_0, M, K, 1)
    assert a.size == M * 18
    assert np.array_equal(a, si.weights(si.FMT_Q4_0, M, K, 1))


# ------------------------------------------------------------ mutation tests
def _mut_q4_interleaved(raw, M, K):
    blk = Q._blocks(raw, Q.FMT_Q4_0, M, K)
    d = Q._scale64(blk)
    b = blk[..., 2:18].astype(np.int64)
    q = np.stack([(b & 15) - 8, (b >> 4) - 8], axis=-1).reshape(M, K // 32, 32)
    return (d[..., None] * q).reshape(M, K)


def _mut_q4_no_offset(raw, M, K):
    blk = Q._blocks(raw, Q.FMT_Q4_0, M, K)
    d = Q._scale64(blk)
    b = blk[..., 2:18].astype(np.int64)
    q = np.concatenate([b & 15, b >> 4], axis=-1)
    return (d[..., None] * q).reshape(M, K)


def _mut_q8_unsigned(raw, M, K):
    blk = Q._blocks(raw, Q.FMT_Q8_0, M, K)
    d = Q._scale64(blk)
    return (d[..., None] * blk[..., 2:34].astype(np.float64)).reshape(M, K)


def _mut_q8_scale_last(raw, M, K):
    blk = Q._blocks(raw, Q.FMT_Q8_0, M, K)
    d = np.ascontiguousarray(blk[..., 32:34]).view("<f2")[..., 0].astype(np.float64)
    q = np.ascontiguousarray(blk[..., 0:32]).view(np.int8)
    return (d[..., None] * q).reshape(M, K)


def _mut_q8_big_endian_scale(raw, M, K):
    blk = Q._blocks(raw, Q.FMT_Q8_0, M, K)
    d = np.ascontiguousarray(blk[..., 0:2]).view(">f2")[..., 0].astype(np.float64)
    q = np.ascontiguousarray(blk[..., 2:34]).view(np.int8)
    return (d[..., None] * q).reshape(M, K)


def _bias_fields(raw, fmt, M, K):
    """Fields of a biased/5-bit block as the adopted reading places them."""
    blk = Q._blocks(raw, fmt, M, K)
    biased = fmt in (Q.FMT_Q4_1, Q.FMT_Q5_1)
    at = 4 if biased else 2
    qh = blk[..., at:at + 4] if fmt != Q.FMT_Q4_1 else None
    qs = blk[..., (at + 4 if qh is not None else at):][..., :16]
    return blk, qh, qs


def _mut_q4_1_swapped(raw, M, K):
    blk, _, qs = _bias_fields(raw, Q.FMT_Q4_1, M, K)
    d, m = Q._scale64(blk, 2), Q._scale64(blk, 0)
    return (d[..., None] * Q._nibbles(qs) + m[..., None]).reshape(M, K)


def _mut_q4_1_minus_bias(raw, M, K):
    blk, _, qs = _bias_fields(raw, Q.FMT_Q4_1, M, K)
    d, m = Q._scale64(blk, 0), Q._scale64(blk, 2)
    return (d[..., None] * Q._nibbles(qs) - m[..., None]).reshape(M, K)


def _mut_q5_0_no_offset(raw, M, K):
    blk, qh, qs = _bias_fields(raw, Q.FMT_Q5_0, M, K)
    u = Q._nibbles(qs) + 16 * Q._high_bits(qh)
    return (Q._scale64(blk)[..., None] * u).reshape(M, K)


def _mut_q5_0_reversed_bits(raw, M, K):
    blk, qh, qs = _bias_fields(raw, Q.FMT_Q5_0, M, K)
    u = Q._nibbles(qs) + 16 * Q._high_bits(qh)[..., ::-1]
    return (Q._scale64(blk)[..., None] * (u - 16)).reshape(M, K)


def _mut_q5_0_big_endian_word(raw, M, K):
    blk, qh, qs = _bias_fields(raw, Q.FMT_Q5_0, M, K)
    u = Q._nibbles(qs) + 16 * Q._high_bits(np.ascontiguousarray(qh[..., ::-1]))
    return (Q._scale64(blk)[..., None] * (u - 16)).reshape(M, K)


def _mut_q5_0_interleaved_bits(raw, M, K):
    # bit 2j -> element j, bit 2j+1 -> element j + 16
    blk, qh, qs = _bias_fields(raw, Q.FMT_Q5_0, M, K)
    bits = Q._high_bits(qh)
    u = Q._nibbles(qs) + 16 * np.concatenate([bits[..., 0::2], bits[..., 1::2]], axis=-1)
    return (Q._scale64(blk)[..., None] * (u - 16)).reshape(M, K)


def _mut_q5_1_codes_first(raw, M, K):
    # codes before the fifth-bit word
    blk = Q._blocks(raw, Q.FMT_Q5_1, M, K)
    u = Q._nibbles(blk[..., 4:20]) + 16 * Q._high_bits(blk[..., 20:24])
    return (Q._scale64(blk, 0)[..., None] * u + Q._scale64(blk, 2)[..., None]).reshape(M, K)


def _mut_q5_1_no_bias(raw, M, K):
    blk, qh, qs = _bias_fields(raw, Q.FMT_Q5_1, M, K)
    u = Q._nibbles(qs) + 16 * Q._high_bits(qh)
    return (Q._scale64(blk, 0)[..., None] * u).reshape(M, K)


def _mut_f16_ftz(raw, M, K):
    w = Q.unpack_f16(raw, M, K)
    w[np.abs(w) < 2.0 ** -14] = 0.0
    return w


def _dequant_with(fmt_mut, fn):
    def dq(fmt, raw, M, K):
        return fn(raw, M, K) if fmt == fmt_mut else Q.dequant(fmt, raw, M, K)
    return dq


def _matmul_with_dequant(dq):
    def mm(fmt, raw, x, M, K, rows=None, chunk_rows=8192):
        W = dq(fmt, raw, M, K)
        x64 = np.asarray(x).astype(np.float64).reshape(-1, K)
        return x64 @ W.T, np.abs(x64) @ np.abs(W).T
    return mm


def _mm_transposed(fmt, raw, x, M, K, rows=None, chunk_rows=8192):
    W = Q.dequant(fmt, raw, M, K)
    x64 = np.asarray(x).astype(np.float64).reshape(-1, K)
    return x64 @ W, np.abs(x64) @ np.abs(W)


def _mm_dropped_term(fmt, raw, x, M, K, rows=None, chunk_rows=8192):
    W = Q.dequant(fmt, raw, M, K)
    x64 = np.asarray(x).astype(np.float64).reshape(-1, K)
    return x64[:, :-1] @ W[:, :-1].T, np.abs(x64) @ np.abs(W).T


def _pins_pass(dq, mm):
    """True when every pin accepts the given decode/matmul pair (an error counts as a rejection)."""
    try:
        ok = all(check_golden(load_golden(p), dq, mm) for p in GOLDEN_FILES)
        for fmt in (Q.FMT_Q8_0, Q.FMT_Q4_0, Q.FMT_F16, *BIAS_FMTS):
            ok = ok and check_brute_force(fmt, 32, 32, 2, 5, mm) and check_brute_force(fmt, 3, 64, 2, 8, mm)
        return ok
    except ValueError:
        return False


@pytest.mark.parametrize("name,fmt,fn", [
    ("q4_interleaved", Q.FMT_Q4_0, _mut_q4_interleaved),
    ("q4_no_offset", Q.FMT_Q4_0, _mut_q4_no_offset),
    ("q8_unsigned", Q.FMT_Q8_0, _mut_q8_unsigned),
    ("q8_scale_last", Q.FMT_Q8_0, _mut_q8_scale_last),
    ("q8_big_endian_scale", Q.FMT_Q8_0, _mut_q8_big_endian_scale),
    ("f16_flush_subnormals", Q.FMT_F16, _mut_f16_ftz),
    ("q4_1_scale_bias_swapped", Q.FMT_Q4_1, _mut_q4_1_swapped),
    ("q4_1_bias_subtracted", Q.FMT_Q4_1, _mut_q4_1_minus_bias),
    ("q5_0_no_offset", Q.FMT_Q5_0, _mut_q5_0_no_offset),
    ("q5_0_reversed_bits", Q.FMT_Q5_0, _mut_q5_0_reversed_bits),
    ("q5_0_big_endian_word", Q.FMT_Q5_0, _mut_q5_0_big_endian_word),
    ("q5_0_interleaved_bits", Q.FMT_Q5_0, _mut_q5_0_interleaved_bits),
    ("q5_1_codes_first", Q.FMT_Q5_1, _mut_q5_1_codes_first),
    ("q5_1_no_bias", Q.FMT_Q5_1, _mut_q5_1_no_bias),
])
def test_mutated_unpack_is_caught(name, fmt, fn):
    dq = _dequant_with(fmt, fn)
    assert not _pins_pass(dq, _matmul_with_dequant(dq)), name


@pytest.mark.parametrize("mm", [_mm_transposed, _mm_dropped_term])
def test_mutated_matmul_is_caught(mm):
    assert not _pins_pass(Q.dequant, mm)


def test_unmutated_pins_pass():
    assert _pins_pass(Q.dequant, _matmul_with_dequant(Q.dequant))


# ------------------------------------------------------------- SwiGLU golden
SWIGLU_GOLDEN = os.path.join(GOLDEN, "swiglu", "q8_0_pair.txt")


def _load_swiglu_golden():
    fx = {"gate": [], "up": [], "x": {}, "g": {}, "u": {}, "h": {}}
    for line in open(SWIGLU_GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key in ("gate", "up"):
            fx[key].append(bytes(int(b, 16) for b in rest))
        elif key in ("x", "g", "u"):
            fx[key][int(rest[0])] = Fraction(rest[1])
        elif key == "h":
            fx["h"][int(rest[0])] = (float(rest[1]), float(rest[2]))
    return fx


def test_swiglu_golden_pair():
    """gate_up_silu_ref on hand-computed Q8_0 rows: g and u exactly, and h = a / (1 + e^b)
    from the fixture, so the SiLU sits on the gate and multiplies the up projection."""
    fx = _load_swiglu_golden()
    I, K = len(fx["gate"]), 32
    rg = np.frombuffer(b"".join(fx["gate"]), np.uint8)
    ru = np.frombuffer(b"".join(fx["up"]), np.uint8)
    x = np.zeros((1, K), np.float32)
    for k, v in fx["x"].items():
        x[0, k] = float(v)
    h, g, u, Sg, Su = Q.gate_up_silu_ref(Q.FMT_Q8_0, rg, ru, x, I, K)
    assert [Fraction(float(v)) for v in g[0]] == [fx["g"][i] for i in range(I)]
    assert [Fraction(float(v)) for v in u[0]] == [fx["u"][i] for i in range(I)]
    want = np.array([a / (1.0 + math.exp(b)) for a, b in (fx["h"][i] for i in range(I))])
    assert np.allclose(h[0], want, rtol=1e-15, atol=0)
    # The pair tells the readings apart: SiLU on the up projection, or no SiLU.
    gg, uu = g[0], u[0]
    assert not np.allclose(Q.silu(uu) * gg, want, rtol=1e-3)
    assert not np.allclose(gg * uu, want, rtol=1e-3)
