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
    r = bench.timed_parity(oracle, {}, si, 512)
    assert r["ok"] and r["outputs_checked"] == 576 + T * bench.PREFILL_CHECK_ROWS
    assert r["max_err_over_bound"] < 0.01
    Y[3, 5] += 2.0 * float(oracle.tol_linear(S2)[3, 5])
    r = bench.timed_parity(oracle, {}, si, 512)
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
    logits[:64] = oracle.matmul_ref(fmt, si.weights(fmt, V, H, base + 999), x, V, H, rows=np.arange(64))[0][0]
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
    r = bench.timed_parity(oracle, {}, si, 64)
    assert r["ok"], r
    assert r["outputs_checked"] == Q + H + I + H + 64 + 2 * nt * R
    y[1, 7] += 1.0
    assert not bench.timed_parity(oracle, {}, si, 64)["ok"]
    bench.TIMED_OUT.clear()
