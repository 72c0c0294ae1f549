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
