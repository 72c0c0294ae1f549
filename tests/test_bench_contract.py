"""Host-side checks of bench.py (no GPU): the one-GPU refusal and the key that ties the
committed HBM-traffic record to the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (bench imports torch only inside main())


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


CODE = """// leading comment
#include "a.hpp"
/* block
   comment */ int f(int x) {   // trailing
    const char* s = "// not a comment";
    return x + 'a';
}
"""


def test_code_only_ignores_comments_and_layout():
    base = bench._code_only(CODE)
    assert "leading" not in base and "block" not in base and "trailing" not in base
    assert '"// not a comment"' in base  # string literals are code
    assert bench._code_only(CODE.replace("// trailing", "// reworded")) == base
    assert bench._code_only(CODE.replace("    return", "\n\n  return")) == base
    # a change to the code itself changes the text
    assert bench._code_only(CODE.replace("x + 'a'", "x - 'a'")) != base
    assert bench._code_only(CODE.replace('"// not a comment"', '"// other"')) != base


def test_traffic_reported_only_for_the_sources_measured():
    """The committed record carries the digest of the sources it was measured on:
    bench.py reports its traffic while they are unchanged, and null once the kernel
    has changed (until the counters are taken again)."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    entry = rec["gemv_Q8_0:lm_head"]
    if entry["source_sha256"] == bench.sources_digest():
        assert bench.traffic_for("gemv_Q8_0:lm_head") == entry["bytes_per_launch"]
    else:
        assert bench.traffic_for("gemv_Q8_0:lm_head") is None
    assert bench.traffic_for("no such launch") is None


@pytest.mark.parametrize("files", [["gemv_dma.hip"], ["gemv_dma.hip", "dma.hpp"]])
def test_digest_depends_on_the_file_list(files):
    assert bench.sources_digest(files) != bench.sources_digest()


def test_timed_parity_passes_oracle_outputs_and_flags_a_wrong_one():
    """The re-check of timed outputs in the CPU-baseline leg: outputs equal to the
    oracle's pass; one output moved by twice its bound fails (no GPU: the "timed"
    outputs here are the oracle's own, for a single GEMV and a small prefill case)."""
    import numpy as np
    import oracle
    import seeded_inputs as si
    bench.TIMED_OUT.clear()
    raw = si.weights(si.FMT_Q8_0, 576, 576, 0)
    y, S = oracle.matmul_ref(si.FMT_Q8_0, raw, si.activations(1, 576, 1), 576, 576)
    bench.TIMED_OUT["single_gemv_576"] = y[0].astype(np.float32)
    M, K, T, fmt = 256, 256, 8, si.FMT_Q4_0
    Y, S2 = oracle.matmul_ref(fmt, si.weights(fmt, M, K, 7000 + M % 101 + fmt),
                              si.activations(T, K, 7100 + T, dtype=np.float16), M, K,
                              rows=np.arange(bench.PREFILL_CHECK_ROWS))
    bench.TIMED_OUT[("prefill", fmt, M, K, T)] = Y
    r = bench.timed_parity(oracle, si)
    assert r["ok"] and r["outputs_checked"] == 576 + T * bench.PREFILL_CHECK_ROWS
    assert r["max_err_over_bound"] < 0.01
    Y[3, 5] += 2.0 * float(oracle.tol_linear(S2)[3, 5])
    r = bench.timed_parity(oracle, si)
    assert not r["ok"] and r["max_err_over_bound"] > 1.5
    bench.TIMED_OUT.clear()


def test_timed_parity_covers_smollm2_and_small_batch_records():
    """The SmolLM2-135M and small-batch records of the re-check, filled here with the
    oracle's own outputs for the same inputs (no GPU), pass; a wrong small-batch output
    fails."""
    import numpy as np
    import oracle
    import seeded_inputs as si
    bench.TIMED_OUT.clear()
    S = si.SMOLLM2_135M
    H, I, V, Q = S["hidden"], S["intermediate"], S["vocab"], si.qkv_rows(S)
    fmt, base = si.FMT_Q4_0, 8500
    s0 = base + 10 * (S["layers"] - 1)
    x = si.activations(1, H, base + 998)
    rec = {"base": base}
    for key, i, M, K in (("y_qkv", 0, Q, H), ("y_o", 1, H, H)):
        rec[key] = oracle.matmul_ref(fmt, si.weights(fmt, M, K, s0 + i), x, M, K)[0][0].astype(np.float32)
    rec["h"] = oracle.gate_up_silu_ref(fmt, si.weights(fmt, I, H, s0 + 2), si.weights(fmt, I, H, s0 + 3), x, I,
                                       H)[0][0].astype(np.float32)
    rec["y_d"] = oracle.matmul_ref(fmt, si.weights(fmt, H, I, s0 + 4), rec["h"], H, I)[0][0].astype(np.float32)
    logits = np.zeros(V, dtype=np.float32)
    R = bench.DECODE_CHECK_ROWS
    logits[:R] = oracle.matmul_ref(fmt, si.weights(fmt, V, H, base + 999), x, V, H, rows=np.arange(R))[0][0]
    rec["logits"] = logits
    bench.TIMED_OUT[("smollm2", fmt)] = rec
    rng = np.random.default_rng(5)
    K, nt, R = 256, 2, bench.SB_CHECK_ROWS
    xs = rng.standard_normal(16 * K).astype(np.float32)
    w = [si.weights(si.FMT_Q8_0, R, K, 11), si.weights(si.FMT_Q8_0, R, K, 12)]
    y = oracle.matmul_ref(si.FMT_Q8_0, w[0], xs[:nt * K].reshape(nt, K), R, K)[0].astype(np.float32)
    h = oracle.gate_up_silu_ref(si.FMT_Q8_0, w[0], w[1], xs[:nt * K].reshape(nt, K), R, K)[0].astype(np.float32)
    bench.TIMED_OUT[("small_batch", si.FMT_Q8_0, "o")] = {"M": 4096, "K": K, "x": xs, "w": w[:1],
                                                           "y": {(nt, "valu"): y}}
    bench.TIMED_OUT[("small_batch", si.FMT_Q8_0, "gate_up")] = {"M": 14336, "K": K, "x": xs, "w": w,
                                                                 "y": {(nt, "mfma"): h}}
    r = bench.timed_parity(oracle, si)
    assert r["ok"], r
    assert r["outputs_checked"] == Q + H + I + H + bench.DECODE_CHECK_ROWS + 2 * nt * R
    y[1, 7] += 1.0
    assert not bench.timed_parity(oracle, si)["ok"]
    bench.TIMED_OUT.clear()


def test_timed_parity_decode_fused_expand_and_gather_records():
    """Decode, fused-step, expand-then-GEMM and row-gather records built from the
    oracle (no GPU) pass; a one-ulp change in an expanded weight or a gathered row,
    or a residual off by twice its bound, fails."""
    import numpy as np
    import oracle
    import seeded_inputs as si
    bench.TIMED_OUT.clear()
    L = si.LLAMA3_8B
    H, I = L["hidden"], L["intermediate"]
    R, fmt = bench.DECODE_CHECK_ROWS, si.FMT_Q4_1
    w = {k: si.weights(fmt, R, I if k == "d" else H, 40 + i) for i, k in enumerate(("qkv", "o", "g", "u", "d", "lm"))}
    x = si.activations(1, H, 47)[0]
    lin = lambda k, xin, K: oracle.matmul_ref(fmt, w[k], xin, R, K)[0][0].astype(np.float32)
    h = oracle.gate_up_silu_ref(fmt, w["g"], w["u"], x, R, H)[0][0].astype(np.float32)
    h_full = np.concatenate([h, np.zeros(I - R, np.float32)])
    rec = {"w": w, "x": x, "y_qkv": lin("qkv", x, H), "y_o": lin("o", x, H), "h": h_full,
           "y_d": lin("d", h_full, I), "logits": lin("lm", x, H)}
    bench.TIMED_OUT[("decode", fmt)] = rec
    gm = (1.0 + 0.1 * si.activations(1, H, 48)[0]).astype(np.float32)
    xn = oracle.rmsnorm_ref(x, gm, 1e-5)[0]
    hf = oracle.gate_up_silu_ref(fmt, w["g"], w["u"], xn, R, H)[0][0].astype(np.float32)
    hf_full = np.concatenate([hf, np.zeros(I - R, np.float32)])
    r0 = si.activations(1, H, 49)[0]
    r1 = oracle.matmul_add_ref(fmt, w["o"], x, r0[:R], R, H)[0][0]
    r2 = oracle.matmul_add_ref(fmt, w["d"], hf_full, r1, R, I)[0][0].astype(np.float32)
    fused = dict(rec, y_qkv=oracle.matmul_ref(fmt, w["qkv"], xn, R, H)[0][0].astype(np.float32), h=hf_full,
                 logits=oracle.matmul_ref(fmt, w["lm"], xn, R, H)[0][0].astype(np.float32), gamma=gm, eps=1e-5,
                 r0=np.concatenate([r0[:R], np.zeros(H - R, np.float32)]),
                 r2=np.concatenate([r2, np.zeros(H - R, np.float32)]))
    bench.TIMED_OUT[("fused", fmt)] = fused
    K, P, n = 256, bench.PREFILL_CHECK_ROWS, bench.TOKEN_CHECK
    we = si.weights(si.FMT_Q8_0, P, K, 50)
    xe = si.activations(n, K, 51, dtype=np.float16)
    bench.TIMED_OUT[("expand", si.FMT_Q8_0, 4096, K, 128)] = {
        "w": we, "w16": oracle.expand_f16_ref(si.FMT_Q8_0, we, P, K),
        "x": xe, "y": oracle.matmul_ref(si.FMT_Q8_0, we, xe, P, K)[0].astype(np.float32)}
    wg = si.weights(si.FMT_Q4_0, 16, K, 52)
    bench.TIMED_OUT[("get_rows", si.FMT_Q4_0, 1)] = {
        "w": wg, "out": oracle.get_rows_ref(si.FMT_Q4_0, wg, 16, K, np.arange(16)).astype(np.float32), "K": K}
    r = bench.timed_parity(oracle, si)
    assert r["ok"], r
    bench.TIMED_OUT[("expand", si.FMT_Q8_0, 4096, K, 128)]["w16"].view(np.uint16)[3, 4] ^= 1
    assert not bench.timed_parity(oracle, si)["ok"]
    bench.TIMED_OUT[("expand", si.FMT_Q8_0, 4096, K, 128)]["w16"].view(np.uint16)[3, 4] ^= 1
    bench.TIMED_OUT[("get_rows", si.FMT_Q4_0, 1)]["out"][2, 9] = np.nextafter(
        bench.TIMED_OUT[("get_rows", si.FMT_Q4_0, 1)]["out"][2, 9], np.float32(np.inf))
    assert not bench.timed_parity(oracle, si)["ok"]
    bench.TIMED_OUT.pop(("get_rows", si.FMT_Q4_0, 1))
    assert bench.timed_parity(oracle, si)["ok"]
    S1 = oracle.matmul_add_ref(fmt, w["o"], x, r0[:R], R, H)[1][0]
    S2 = oracle.matmul_add_ref(fmt, w["d"], hf_full, r1, R, I)[1][0]
    fused["r2"][5] += 2.0 * float(oracle.tol_residual(S1, r1)[5] + oracle.tol_residual(S2, r2)[5])
    assert not bench.timed_parity(oracle, si)["ok"]
    bench.TIMED_OUT.clear()


def test_timed_parity_tp8_shard_records():
    """Records of the 8-way tensor-parallel shard step built from the oracle (no GPU)
    pass; a down output moved by twice its bound fails, and so does a gate+up output
    computed from the wrong operand order (silu of the up sums)."""
    import numpy as np
    import oracle
    import seeded_inputs as si
    bench.TIMED_OUT.clear()
    L = si.LLAMA3_8B
    H, I, V, Q = L["hidden"], L["intermediate"], L["vocab"], si.qkv_rows(L)
    q8, o8, i8, v8 = Q // 8, H // 8, I // 8, V // 8
    fmt, R = si.FMT_Q8_0, bench.DECODE_CHECK_ROWS
    dims = {"qkv": (q8, H), "o": (H, o8), "gate_up": (i8, H), "down": (H, i8), "lm_head": (v8, H)}
    kdim = {"qkv": H, "o": o8, "g": H, "u": H, "d": i8, "lm": H}
    w = {k: si.weights(fmt, R, K, 60 + i) for i, (k, K) in enumerate(kdim.items())}
    x, xo = si.activations(1, H, 70)[0], si.activations(1, o8, 71)[0]
    hR, g, u, _, _ = oracle.gate_up_silu_ref(fmt, w["g"], w["u"], x, R, H)
    h = np.concatenate([hR[0], np.zeros(i8 - R)]).astype(np.float32)
    lin = lambda k, xin, K: oracle.matmul_ref(fmt, w[k], xin, R, K)[0][0].astype(np.float32)
    rec = {"x": x, "xo": xo, "h": h, "w": w, "dims": dims,
           "y": {"qkv": lin("qkv", x, H), "o": lin("o", xo, o8), "down": lin("d", h, i8), "lm_head": lin("lm", x, H)}}
    bench.TIMED_OUT[("tp8", fmt)] = rec
    r = bench.timed_parity(oracle, si)
    assert r["ok"] and r["outputs_checked"] == 5 * R, r
    S = oracle.matmul_ref(fmt, w["d"], h, R, i8)[1][0]
    rec["y"]["down"][7] += 2.0 * float(oracle.tol_linear(S)[7])
    assert not bench.timed_parity(oracle, si)["ok"]
    rec["y"]["down"] = lin("d", h, i8)
    assert bench.timed_parity(oracle, si)["ok"]
    rec["h"] = np.concatenate([(oracle.silu(u[0]) * g[0]), np.zeros(i8 - R)]).astype(np.float32)
    rec["y"]["down"] = lin("d", rec["h"], i8)  # down stays consistent with the (wrong) h it consumed
    assert not bench.timed_parity(oracle, si)["ok"]
    bench.TIMED_OUT.clear()
