"""Host-side checks of the C ABI (CPU only; no kernel is launched).

The library must load, export every function include/qmm.h declares, compute
row sizes, and reject every invalid argument before any HIP call.  The pointer
values used here are never dereferenced: each call fails validation first.
"""
import ctypes
import os
import re
import subprocess

import pytest

import block_quantized_weight_gguf_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

OK, E_NULL, E_FMT, E_SHAPE, E_ALIGN, E_OVF, E_HIP, E_VAR, E_ARG, E_WS, E_SCR = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10
A16 = 0x10000  # a 16-byte aligned fake address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted([
        "qmm_version", "qmm_strerror", "qmm_row_bytes", "qmm_dequant", "qmm_gemv", "qmm_gemv_variant",
        "qmm_gemv_choose", "qmm_gate_up_silu", "qmm_gate_up_silu_variant", "qmm_gemm",
        "qmm_gemm_gate_up_silu", "qmm_get_rows", "qmm_expand_f16", "qmm_rmsnorm_gemv",
        "qmm_rmsnorm_gate_up_silu", "qmm_gemv_add", "qmm_workspace_size", "qmm_gemm_noalloc",
        "qmm_stream_read"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(qmm.lib_path)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qmm.lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (qmm_[a-z_0-9]+)\b", out))
    assert set(declared_functions()) <= exported
    assert set(qmm.EXPORTED) == set(declared_functions())


def test_version_and_strerror():
    assert qmm.qmm_version() >= 100
    for s in (OK, E_NULL, E_FMT, E_SHAPE, E_ALIGN, E_OVF, E_HIP, E_VAR, E_ARG, E_WS, E_SCR):
        assert qmm.qmm_strerror(s) and "unknown qmm status" not in qmm.qmm_strerror(s)
    assert "unknown" in qmm.qmm_strerror(-99)


@pytest.mark.parametrize("fmt,K,want", [
    (8, 576, 612), (2, 576, 324), (1, 576, 1152), (8, 4096, 4352), (2, 4096, 2304),
    (8, 14336, 15232), (2, 14336, 8064), (1, 32, 64), (8, 32, 34), (2, 32, 18),
    (3, 32, 20), (6, 32, 22), (7, 32, 24), (3, 4096, 2560), (6, 4096, 2816), (7, 14336, 10752)])
def test_row_bytes(fmt, K, want):
    assert qmm._lib.qmm_row_bytes(fmt, K) == want


@pytest.mark.parametrize("fmt,K,want", [(4, 64, E_FMT), (5, 64, E_FMT), (9, 64, E_FMT), (0, 64, E_FMT),
                                        (8, 0, E_SHAPE), (8, 100, E_SHAPE), (6, 48, E_SHAPE),
                                        (2, -32, E_SHAPE), (1, 48, E_SHAPE), (8, 2**31, E_SHAPE)])
def test_row_bytes_errors(fmt, K, want):
    assert qmm._lib.qmm_row_bytes(fmt, K) == want


def test_gemv_validation():
    L = qmm._lib
    assert L.qmm_gemv(8, None, A16, A16, 4, 64, 1, None, 0, None) == E_NULL
    assert L.qmm_gemv(8, A16, None, A16, 4, 64, 1, None, 0, None) == E_NULL
    assert L.qmm_gemv(8, A16, A16, None, 4, 64, 1, None, 0, None) == E_NULL
    assert L.qmm_gemv(5, A16, A16, A16, 4, 64, 1, None, 0, None) == E_FMT
    assert L.qmm_gemv(8, A16, A16, A16, 0, 64, 1, None, 0, None) == E_SHAPE
    assert L.qmm_gemv(8, A16, A16, A16, 4, 0, 1, None, 0, None) == E_SHAPE
    assert L.qmm_gemv(8, A16, A16, A16, 4, 48, 1, None, 0, None) == E_SHAPE
    assert L.qmm_gemv(8, A16, A16, A16, 4, 64, 0, None, 0, None) == E_SHAPE
    assert L.qmm_gemv(8, A16, A16, A16, 2**31, 64, 1, None, 0, None) == E_SHAPE
    assert L.qmm_gemv(8, A16, A16, A16, 2**31 - 1, 2**31 - 32, 2**31 - 1, None, 0, None) == E_OVF
    assert L.qmm_gemv(8, A16 + 8, A16, A16, 4, 64, 1, None, 0, None) == E_ALIGN
    assert L.qmm_gemv(8, A16, A16 + 4, A16, 4, 64, 1, None, 0, None) == E_ALIGN
    assert L.qmm_gemv(8, A16, A16, A16 + 2, 4, 64, 1, None, 0, None) == E_ALIGN
    assert L.qmm_gemv_variant(8, A16, A16, A16 + 2, 4, 64, 1, 1, None, 0, None) == E_ALIGN


def test_gate_up_validation():
    L = qmm._lib
    assert L.qmm_gate_up_silu(2, A16, None, A16, A16, 4, 64, 1, None, 0, None) == E_NULL
    assert L.qmm_gate_up_silu(4, A16, A16, A16, A16, 4, 64, 1, None, 0, None) == E_FMT
    assert L.qmm_gate_up_silu(2, A16, A16, A16, A16, 4, 40, 1, None, 0, None) == E_SHAPE
    assert L.qmm_gate_up_silu(2, A16, A16 + 4, A16, A16, 4, 64, 1, None, 0, None) == E_ALIGN


def test_gemm_validation():
    L = qmm._lib
    assert L.qmm_gemm(8, A16, None, A16, 4, 64, 8, None, 0, None) == E_NULL
    assert L.qmm_gemm(8, A16, A16, A16, 4, 64, 0, None, 0, None) == E_SHAPE
    assert L.qmm_gemm(8, A16, A16 + 2, A16, 4, 64, 8, None, 0, None) == E_ALIGN
    assert L.qmm_gemm_gate_up_silu(8, A16, A16, A16, None, 4, 64, 8, None, 0, None) == E_NULL
    assert L.qmm_gemm_gate_up_silu(9, A16, A16, A16, A16, 4, 64, 8, None, 0, None) == E_FMT
    assert L.qmm_gemm_gate_up_silu(8, A16, A16, A16, A16 + 1, 4, 64, 8, None, 0, None) == E_ALIGN


def test_dequant_validation():
    L = qmm._lib
    assert L.qmm_dequant(8, None, A16, 4, 64, None) == E_NULL
    assert L.qmm_dequant(8, A16, A16, 4, 65, None) == E_SHAPE
    assert L.qmm_dequant(8, A16, A16 + 4, 4, 64, None) == E_ALIGN


def test_get_rows_validation():
    L = qmm._lib
    A4 = A16 + 4
    assert L.qmm_get_rows(8, A16, A16, A16, 4, 64, 0, None) == OK  # empty gather: nothing enqueued
    assert L.qmm_get_rows(8, None, None, None, 4, 64, 0, None) == OK
    assert L.qmm_get_rows(5, A16, A16, A16, 4, 64, 0, None) == E_FMT
    assert L.qmm_get_rows(8, None, A16, A16, 4, 64, 3, None) == E_NULL
    assert L.qmm_get_rows(8, A16, None, A16, 4, 64, 3, None) == E_NULL
    assert L.qmm_get_rows(8, A16, A16, None, 4, 64, 3, None) == E_NULL
    assert L.qmm_get_rows(4, A16, A16, A16, 4, 64, 3, None) == E_FMT
    assert L.qmm_get_rows(8, A16, A16, A16, 4, 64, -1, None) == E_SHAPE
    assert L.qmm_get_rows(8, A16, A16, A16, 0, 64, 3, None) == E_SHAPE
    assert L.qmm_get_rows(2, A16, A16, A16, 4, 33, 3, None) == E_SHAPE
    assert L.qmm_get_rows(8, A16, A16, A16, 4, 2**31 - 32, 2**31 - 1, None) == E_OVF
    assert L.qmm_get_rows(8, A16 + 2, A16, A16, 4, 64, 3, None) == E_ALIGN
    assert L.qmm_get_rows(8, A16, A16 + 2, A16, 4, 64, 3, None) == E_ALIGN
    assert L.qmm_get_rows(8, A16, A4, A16 + 4, 4, 64, 3, None) == E_ALIGN  # out needs 16 bytes


def test_expand_f16_validation():
    L = qmm._lib
    assert L.qmm_expand_f16(8, None, A16, 4, 64, None) == E_NULL
    assert L.qmm_expand_f16(8, A16, None, 4, 64, None) == E_NULL
    assert L.qmm_expand_f16(5, A16, A16, 4, 64, None) == E_FMT
    assert L.qmm_expand_f16(1, A16, A16, 4, 16, None) == E_SHAPE
    assert L.qmm_expand_f16(1, A16, A16, 0, 64, None) == E_SHAPE
    assert L.qmm_expand_f16(2, A16, A16 + 8, 4, 64, None) == E_ALIGN
    assert L.qmm_expand_f16(2, A16 + 2, A16, 4, 64, None) == E_ALIGN


def test_rmsnorm_gemv_validation():
    L = qmm._lib
    f = ctypes.c_float
    assert L.qmm_rmsnorm_gemv(8, A16, A16, None, f(1e-5), A16, 4, 64, 1, None) == E_NULL
    assert L.qmm_rmsnorm_gemv(8, None, A16, A16, f(1e-5), A16, 4, 64, 1, None) == E_NULL
    assert L.qmm_rmsnorm_gemv(8, A16, A16, A16, f(1e-5), None, 4, 64, 1, None) == E_NULL
    assert L.qmm_rmsnorm_gemv(4, A16, A16, A16, f(1e-5), A16, 4, 64, 1, None) == E_FMT
    assert L.qmm_rmsnorm_gemv(8, A16, A16, A16, f(1e-5), A16, 4, 50, 1, None) == E_SHAPE
    assert L.qmm_rmsnorm_gemv(8, A16, A16, A16, f(1e-5), A16, 4, 64, 0, None) == E_SHAPE
    for bad in (-1e-6, float("nan"), float("inf"), -float("inf")):
        assert L.qmm_rmsnorm_gemv(8, A16, A16, A16, f(bad), A16, 4, 64, 1, None) == E_ARG
    assert L.qmm_rmsnorm_gemv(8, A16, A16, A16 + 4, f(1e-5), A16, 4, 64, 1, None) == E_ALIGN
    assert L.qmm_rmsnorm_gemv(8, A16, A16 + 8, A16, f(1e-5), A16, 4, 64, 1, None) == E_ALIGN
    assert L.qmm_rmsnorm_gemv(8, A16, A16, A16, f(1e-5), A16 + 2, 4, 64, 1, None) == E_ALIGN
    assert L.qmm_rmsnorm_gate_up_silu(8, A16, A16, A16, None, f(1e-5), A16, 4, 64, 1, None) == E_NULL
    assert L.qmm_rmsnorm_gate_up_silu(8, A16, None, A16, A16, f(1e-5), A16, 4, 64, 1, None) == E_NULL
    assert L.qmm_rmsnorm_gate_up_silu(1, A16, A16, A16, A16, f(1e-5), A16, 4, 48, 1, None) == E_SHAPE
    assert L.qmm_rmsnorm_gate_up_silu(8, A16, A16, A16, A16, f(-1.0), A16, 4, 64, 1, None) == E_ARG
    assert L.qmm_rmsnorm_gate_up_silu(8, A16, A16, A16, A16 + 8, f(0.0), A16, 4, 64, 1, None) == E_ALIGN
    assert L.qmm_rmsnorm_gate_up_silu(8, A16, A16, A16, A16, f(0.0), A16 + 1, 4, 64, 1, None) == E_ALIGN


def test_gemv_add_validation():
    L = qmm._lib
    assert L.qmm_gemv_add(8, A16, A16, None, A16, 4, 64, 1, None) == E_NULL
    assert L.qmm_gemv_add(8, A16, None, A16, A16, 4, 64, 1, None) == E_NULL
    assert L.qmm_gemv_add(2, A16, A16, A16, None, 4, 64, 1, None) == E_NULL
    assert L.qmm_gemv_add(0, A16, A16, A16, A16, 4, 64, 1, None) == E_FMT
    assert L.qmm_gemv_add(2, A16, A16, A16, A16, 0, 64, 1, None) == E_SHAPE
    assert L.qmm_gemv_add(2, A16, A16, A16 + 2, A16, 4, 64, 1, None) == E_ALIGN
    assert L.qmm_gemv_add(2, A16, A16, A16, A16 + 2, 4, 64, 1, None) == E_ALIGN
    assert L.qmm_gemv_add(2, A16 + 4, A16, A16, A16, 4, 64, 1, None) == E_ALIGN


def test_variant_choice():
    L = qmm._lib
    for fmt in (1, 2, 8):
        assert L.qmm_gemv_choose(fmt, 4096, 4096, 1) == 1
        assert L.qmm_gemv_choose(fmt, 4096, 4096, 4096) == 2
        v = [L.qmm_gemv_choose(fmt, 4096, 4096, n) for n in range(1, 65)]
        assert v == sorted(v), "the choice must switch once, from VALU to MFMA"
    # Measured thresholds (MI355X, Llama-3-8B shapes).  Block formats: MFMA from 5
    # tokens; at 4 tokens on long rows (the down projection) and on the Q4_0 / Q4_1 LM
    # heads (>= 256 MiB); VALU at 2-3 tokens.
    for fmt in (2, 8):
        assert L.qmm_gemv_choose(fmt, 4096, 4096, 4) == 1       # 17.8 / 9.4 MB
        assert L.qmm_gemv_choose(fmt, 4096, 4096, 5) == 2
        assert L.qmm_gemv_choose(fmt, 128256, 4096, 4) == (2 if fmt == 2 else 1)     # LM head
        assert L.qmm_gemv_choose(fmt, 128256, 4096, 3) == 1
        assert L.qmm_gemv_choose(fmt, 128256, 4096, 2) == 1
        assert L.qmm_gemv_choose(fmt, 4096, 14336, 4) == 2      # down projection
        assert L.qmm_gemv_choose(fmt, 4096, 14336, 3) == 1
        assert L.qmm_gemv_choose(fmt, 14336, 4096, 3) == 1
    for fmt in (3, 6, 7):
        assert [L.qmm_gemv_choose(fmt, 4096, 4096, n) for n in (1, 3, 4, 5, 64)] == [1, 1, 1, 2, 2]
        assert L.qmm_gemv_choose(fmt, 4096, 14336, 4) == 2
        assert L.qmm_gemv_choose(fmt, 128256, 4096, 3) == 1
        assert L.qmm_gemv_choose(fmt, 128256, 4096, 4) == (2 if fmt == 3 else 1)
    # Long rows of few rows: not the MFMA kernel (under 16 MiB of weights).
    assert L.qmm_gemv_choose(8, 512, 14336, 4) == 1
    # F16 (MFMA = the tiled GEMM): from 5 tokens; from 2 on long rows over 32 MiB; at 4
    # from 64 MiB; at 3 from 256 MiB.
    assert [L.qmm_gemv_choose(1, 4096, 4096, n) for n in (2, 3, 4, 5)] == [1, 1, 1, 2]
    assert [L.qmm_gemv_choose(1, 4096, 14336, n) for n in (1, 2, 3)] == [1, 2, 2]
    assert [L.qmm_gemv_choose(1, 14336, 4096, n) for n in (3, 4)] == [1, 2]
    assert [L.qmm_gemv_choose(1, 128256, 4096, n) for n in (2, 3)] == [1, 2]
    assert L.qmm_gemv_choose(5, 4096, 4096, 1) == E_FMT
    assert L.qmm_gemv_choose(8, 4096, 100, 1) == E_SHAPE
    assert L.qmm_gemv_variant(8, A16, A16, A16 + 1, 4, 64, 1, 9, None, 0, None) == E_ALIGN
    assert L.qmm_gemv_variant(8, A16, A16, A16, 4, 64, 1, 9, None, 0, None) == E_VAR
    assert L.qmm_gemv_variant(8, A16, A16, A16, 4, 64, 1, -1, None, 0, None) == E_VAR
    assert L.qmm_gate_up_silu_variant(8, A16, None, A16, A16, 4, 64, 1, 1, None, 0, None) == E_NULL
    assert L.qmm_gate_up_silu_variant(5, A16, A16, A16, A16, 4, 64, 1, 1, None, 0, None) == E_FMT
    assert L.qmm_gate_up_silu_variant(8, A16, A16, A16, A16, 4, 48, 1, 1, None, 0, None) == E_SHAPE
    assert L.qmm_gate_up_silu_variant(8, A16, A16 + 8, A16, A16, 4, 64, 1, 1, None, 0, None) == E_ALIGN
    assert L.qmm_gate_up_silu_variant(8, A16, A16, A16, A16, 4, 64, 1, 5, None, 0, None) == E_VAR


def test_binding_raises():
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_gemv(8, 0, A16, A16, 4, 64, 1, stream=0)
    assert e.value.status == E_NULL



OP_GEMV, OP_GATE, OP_GEMM, OP_GEMM_GATE = 1, 2, 3, 4
AUTO, VALU, MFMA = 0, 1, 2


def test_workspace_size():
    """The size query: nothing for the register-decode products and for GEMMs whose
    tiles fill the GPU; split-K partials otherwise; the fp32-token MFMA products that
    run the GEMM add the scaled fp16 tokens and their scales (the MFMA GEMV converts
    its tokens itself).  Sizes are whole multiples of 256."""
    W = qmm._lib.qmm_workspace_size
    assert W(OP_GEMV, 8, 4096, 4096, 1, AUTO) == 0
    assert W(OP_GEMV, 8, 4096, 4096, 4, VALU) == 0
    assert W(OP_GATE, 2, 14336, 4096, 2, AUTO) == 0
    assert W(OP_GEMM, 8, 14336, 4096, 4096, AUTO) == 0             # 56 x 16 tiles: no split
    part = W(OP_GEMM, 8, 14336, 4096, 128, AUTO)                   # 56 tiles: K split
    assert part > 0 and part % 256 == 0
    assert part % (128 * 14336 * 4) == 0
    assert W(OP_GEMM_GATE, 8, 14336, 4096, 128, AUTO) >= 2 * part // 2
    # MFMA GEMV at 8 tokens: the partials alone (16 row tiles: K split 16 ways).
    v = W(OP_GEMV, 8, 4096, 4096, 8, AUTO)
    assert v == 16 * 8 * 4096 * 4
    assert W(OP_GEMV, 8, 4096, 4096, 8, MFMA) == v
    assert W(OP_GEMV, 8, 65536, 4096, 8, MFMA) == 0                # 256 row tiles: no split
    assert W(OP_GEMV, 1, 4096, 4096, 64, AUTO) >= 64 * 4096 * 2    # F16 through the GEMM
    assert W(OP_GEMV, 8, 4096, 4096, 33, MFMA) >= 33 * 4096 * 2    # 33 tokens: the GEMM
    # Errors: op, variant, shape.
    assert W(9, 8, 64, 64, 1, AUTO) == E_ARG
    assert W(OP_GEMV, 8, 64, 64, 1, 7) == E_VAR
    assert W(OP_GEMV, 8, 64, 48, 1, AUTO) == E_SHAPE
    assert W(OP_GEMM, 5, 64, 64, 1, AUTO) == E_FMT
    assert W(OP_GEMV, 8, 2**31 - 1, 2**31 - 32, 2**31 - 1, AUTO) == E_OVF


def test_workspace_is_checked_before_any_launch():
    """A call that needs a workspace refuses a missing, short or misaligned one (the
    fake addresses are never touched: validation fails first)."""
    L = qmm._lib
    need = L.qmm_workspace_size(OP_GEMM, 8, 14336, 4096, 128, AUTO)
    assert L.qmm_gemm(8, A16, A16, A16, 14336, 4096, 128, None, 0, None) == E_WS
    assert L.qmm_gemm(8, A16, A16, A16, 14336, 4096, 128, A16, need - 1, None) == E_WS
    assert L.qmm_gemm(8, A16, A16, A16, 14336, 4096, 128, A16 + 16, need, None) == E_ALIGN
    need = L.qmm_workspace_size(OP_GEMM_GATE, 2, 14336, 4096, 128, AUTO)
    assert L.qmm_gemm_gate_up_silu(2, A16, A16, A16, A16, 14336, 4096, 128, A16, need - 256, None) == E_WS
    need = L.qmm_workspace_size(OP_GEMV, 2, 4096, 4096, 8, MFMA)
    assert L.qmm_gemv_variant(2, A16, A16, A16, 4096, 4096, 8, MFMA, None, 0, None) == E_WS
    assert L.qmm_gemv(2, A16, A16, A16, 4096, 4096, 8, A16, need - 1, None) == E_WS
    need = L.qmm_workspace_size(OP_GATE, 8, 14336, 4096, 16, AUTO)
    assert L.qmm_gate_up_silu(8, A16, A16, A16, A16, 14336, 4096, 16, A16, need // 2, None) == E_WS
    assert L.qmm_gate_up_silu_variant(8, A16, A16, A16, A16, 14336, 4096, 16, MFMA, A16 + 128, need, None) == E_ALIGN


def test_gemm_noalloc_validation():
    """The allocation-free GEMM checks its arguments as qmm_gemm does, before any HIP
    call (the fake addresses are never touched)."""
    L = qmm._lib
    assert L.qmm_gemm_noalloc(8, None, A16, A16, 4, 64, 8, None) == E_NULL
    assert L.qmm_gemm_noalloc(8, A16, A16, None, 4, 64, 8, None) == E_NULL
    assert L.qmm_gemm_noalloc(5, A16, A16, A16, 4, 64, 8, None) == E_FMT
    assert L.qmm_gemm_noalloc(8, A16, A16, A16, 4, 48, 8, None) == E_SHAPE
    assert L.qmm_gemm_noalloc(8, A16, A16, A16, 4, 64, 0, None) == E_SHAPE
    assert L.qmm_gemm_noalloc(8, A16, A16 + 2, A16, 4, 64, 8, None) == E_ALIGN
    assert L.qmm_gemm_noalloc(8, A16, A16, A16 + 1, 4, 64, 8, None) == E_ALIGN


def test_gemm_workspace_fits_the_noalloc_scratch():
    """qmm_gemm's plan never needs more than the fixed 64 MiB of qmm_gemm_noalloc, over
    token counts and row counts around the split thresholds."""
    W = qmm._lib.qmm_workspace_size
    worst = 0
    for fmt in (1, 2, 8):
        for M in (1, 255, 256, 257, 4096, 12288, 14336, 49151, 49152):
            for T in (1, 100, 128, 129, 256, 1000, 2048, 2304, 4096):
                for K in (4096, 14336):
                    worst = max(worst, W(OP_GEMM, fmt, M, K, T, AUTO))
    assert 0 < worst <= qmm.QMM_NOALLOC_SCRATCH_BYTES


def test_stream_read_validation():
    """The streaming-read reference checks its arguments before any HIP call (the fake
    addresses are never touched)."""
    L = qmm._lib
    assert L.qmm_stream_read(None, 16, A16, None) == E_NULL
    assert L.qmm_stream_read(A16, 16, None, None) == E_NULL
    assert L.qmm_stream_read(A16, 0, A16, None) == E_SHAPE
    assert L.qmm_stream_read(A16, -16, A16, None) == E_SHAPE
    assert L.qmm_stream_read(A16, 24, A16, None) == E_SHAPE
    assert L.qmm_stream_read(A16 + 8, 16, A16, None) == E_ALIGN
    assert L.qmm_stream_read(A16, 16, A16 + 2, None) == E_ALIGN
    assert qmm.QMM_STREAM_READ_BLOCKS == int(re.search(r"#define QMM_STREAM_READ_BLOCKS (\d+)",
                                                       open(HEADER).read()).group(1))
