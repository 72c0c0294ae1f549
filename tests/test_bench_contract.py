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
