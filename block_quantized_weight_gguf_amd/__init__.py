"""Python binding of the qmm C ABI (include/qmm.h): GGUF block-quantized products on MI355X.

Argument marshalling only.  Each ``qmm_*`` function here has the C entry point's
name and argument order, with torch device tensors in place of pointers; it
checks nothing beyond what ctypes needs and raises ``QmmError`` on a negative
status.  Every step of the computation runs in the HIP kernels of libqmm.so;
PyTorch supplies device memory and the current stream.  There is no fallback:
importing this package fails loudly if libqmm.so is missing.

Workspace: the products that need one take ``workspace`` (a device tensor, or a raw
pointer with ``workspace_bytes``).  Left as None, a buffer of the size
``qmm_workspace_size`` reports is taken from torch's caching allocator on the
current stream for the call (pass one explicitly when launching on another stream).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "QMM_F16", "QMM_Q4_0", "QMM_Q4_1", "QMM_Q5_0", "QMM_Q5_1", "QMM_Q8_0", "QMM_VARIANT_AUTO", "QMM_VARIANT_VALU", "QMM_VARIANT_MFMA",
    "QmmError", "lib_path", "qmm_version", "qmm_strerror", "qmm_row_bytes", "qmm_dequant", "qmm_gemv",
    "qmm_gemv_variant", "qmm_gemv_choose", "qmm_gate_up_silu", "qmm_gate_up_silu_variant", "qmm_gemm",
    "qmm_gemm_gate_up_silu", "qmm_get_rows", "qmm_expand_f16", "qmm_rmsnorm_gemv", "qmm_rmsnorm_gate_up_silu",
    "qmm_gemv_add", "QMM_ERR_ARG", "QMM_ERR_WORKSPACE", "QMM_WORKSPACE_ALIGN", "qmm_workspace_size",
    "QMM_OP_GEMV", "QMM_OP_GATE_UP_SILU", "QMM_OP_GEMM", "QMM_OP_GEMM_GATE_UP_SILU", "qmm_gemm_noalloc",
    "QMM_ERR_SCRATCH", "QMM_NOALLOC_SCRATCH_BYTES", "qmm_stream_read", "QMM_STREAM_READ_BLOCKS",
    "gemv", "get_rows", "expand_f16", "rmsnorm_gemv", "rmsnorm_gate_up_silu", "gemv_add", "gate_up_silu", "gemm", "gemm_gate_up_silu", "dequant",
]

QMM_F16, QMM_Q4_0, QMM_Q4_1, QMM_Q5_0, QMM_Q5_1, QMM_Q8_0 = 1, 2, 3, 6, 7, 8
QMM_VARIANT_AUTO, QMM_VARIANT_VALU, QMM_VARIANT_MFMA = 0, 1, 2
QMM_ERR_ARG = -8
QMM_ERR_WORKSPACE = -9
QMM_ERR_SCRATCH = -10
QMM_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
QMM_STREAM_READ_BLOCKS = 8192
QMM_WORKSPACE_ALIGN = 256
QMM_OP_GEMV, QMM_OP_GATE_UP_SILU, QMM_OP_GEMM, QMM_OP_GEMM_GATE_UP_SILU = 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libqmm.so")

if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(or python block_quantized_weight_gguf_amd/build.py); there is no fallback path")

_lib = ctypes.CDLL(lib_path)

_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
_SIGS = {
    "qmm_version": (_i32, []),
    "qmm_strerror": (ctypes.c_char_p, [_i32]),
    "qmm_row_bytes": (_i64, [_i32, _i64]),
    "qmm_dequant": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp]),
    "qmm_get_rows": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "qmm_expand_f16": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp]),
    "qmm_workspace_size": (_i64, [_i32, _i32, _i64, _i64, _i64, _i32]),
    "qmm_gemv": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "qmm_gemv_variant": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _i64, _vp]),
    "qmm_gemv_choose": (_i32, [_i32, _i64, _i64, _i64]),
    "qmm_gate_up_silu": (_i32, [_i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "qmm_gate_up_silu_variant": (_i32, [_i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _i64, _vp]),
    "qmm_rmsnorm_gemv": (_i32, [_i32, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _i64, _i64, _vp]),
    "qmm_rmsnorm_gate_up_silu": (_i32, [_i32, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _i64, _i64, _vp]),
    "qmm_gemv_add": (_i32, [_i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "qmm_gemm": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "qmm_gemm_gate_up_silu": (_i32, [_i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "qmm_gemm_noalloc": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "qmm_stream_read": (_i32, [_vp, _i64, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class QmmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {qmm_strerror(status)} (status {status})")
        self.status = status


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int | None:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status < 0:
        raise QmmError(status, where)


def _device_of(*ts):
    for t in ts:
        if isinstance(t, torch.Tensor):
            return t.device
    return torch.device("cuda", torch.cuda.current_device())


def _workspace(op, fmt, M, K, N, variant, refs, workspace, workspace_bytes):
    """(pointer, bytes, buffer) of a call's workspace; see the module docstring.  When the
    size query itself fails, no buffer is made and the call reports the error."""
    if workspace is not None:
        if isinstance(workspace, torch.Tensor):
            nb = workspace.numel() * workspace.element_size()
            return workspace.data_ptr(), nb if workspace_bytes is None else workspace_bytes, None
        return int(workspace), int(workspace_bytes or 0), None
    need = _lib.qmm_workspace_size(op, fmt, M, K, N, variant)
    if need <= 0:
        return None, 0, None
    buf = torch.empty(need, dtype=torch.uint8, device=_device_of(*refs))
    return buf.data_ptr(), need, buf


# ------------------------------------------------------ same names as the C ABI
def qmm_version() -> int:
    return _lib.qmm_version()


def qmm_strerror(status: int) -> str:
    return _lib.qmm_strerror(status).decode()


def qmm_row_bytes(fmt: int, K: int) -> int:
    r = _lib.qmm_row_bytes(fmt, K)
    _check(r, "qmm_row_bytes")
    return r


def qmm_dequant(fmt, W, out, M, K, stream=None) -> None:
    _check(_lib.qmm_dequant(fmt, _ptr(W), _ptr(out), M, K, _stream(stream)), "qmm_dequant")


def qmm_get_rows(fmt, W, ids, out, M, K, n, stream=None) -> None:
    _check(_lib.qmm_get_rows(fmt, _ptr(W), _ptr(ids), _ptr(out), M, K, n, _stream(stream)), "qmm_get_rows")


def qmm_expand_f16(fmt, W, out, M, K, stream=None) -> None:
    _check(_lib.qmm_expand_f16(fmt, _ptr(W), _ptr(out), M, K, _stream(stream)), "qmm_expand_f16")


def qmm_workspace_size(op, fmt, M, K, N, variant=QMM_VARIANT_AUTO) -> int:
    r = _lib.qmm_workspace_size(op, fmt, M, K, N, variant)
    _check(r, "qmm_workspace_size")
    return r


def qmm_gemv(fmt, W, x, y, M, K, N, workspace=None, workspace_bytes=None, stream=None) -> None:
    wp, wb, _keep = _workspace(QMM_OP_GEMV, fmt, M, K, N, QMM_VARIANT_AUTO, (y, x), workspace, workspace_bytes)
    _check(_lib.qmm_gemv(fmt, _ptr(W), _ptr(x), _ptr(y), M, K, N, wp, wb, _stream(stream)), "qmm_gemv")


def qmm_gemv_variant(fmt, W, x, y, M, K, N, variant, workspace=None, workspace_bytes=None, stream=None) -> None:
    wp, wb, _keep = _workspace(QMM_OP_GEMV, fmt, M, K, N, variant, (y, x), workspace, workspace_bytes)
    _check(_lib.qmm_gemv_variant(fmt, _ptr(W), _ptr(x), _ptr(y), M, K, N, variant, wp, wb, _stream(stream)),
           "qmm_gemv_variant")


def qmm_gemv_choose(fmt, M, K, N) -> int:
    r = _lib.qmm_gemv_choose(fmt, M, K, N)
    _check(r, "qmm_gemv_choose")
    return r


def qmm_gate_up_silu(fmt, Wg, Wu, x, h, I, K, N, workspace=None, workspace_bytes=None, stream=None) -> None:
    wp, wb, _keep = _workspace(QMM_OP_GATE_UP_SILU, fmt, I, K, N, QMM_VARIANT_AUTO, (h, x), workspace,
                               workspace_bytes)
    _check(_lib.qmm_gate_up_silu(fmt, _ptr(Wg), _ptr(Wu), _ptr(x), _ptr(h), I, K, N, wp, wb, _stream(stream)),
           "qmm_gate_up_silu")


def qmm_gate_up_silu_variant(fmt, Wg, Wu, x, h, I, K, N, variant, workspace=None, workspace_bytes=None,
                             stream=None) -> None:
    wp, wb, _keep = _workspace(QMM_OP_GATE_UP_SILU, fmt, I, K, N, variant, (h, x), workspace, workspace_bytes)
    _check(_lib.qmm_gate_up_silu_variant(fmt, _ptr(Wg), _ptr(Wu), _ptr(x), _ptr(h), I, K, N, variant, wp, wb,
                                         _stream(stream)), "qmm_gate_up_silu_variant")


def qmm_rmsnorm_gemv(fmt, W, x, gamma, eps, y, M, K, N, stream=None) -> None:
    _check(_lib.qmm_rmsnorm_gemv(fmt, _ptr(W), _ptr(x), _ptr(gamma), eps, _ptr(y), M, K, N, _stream(stream)),
           "qmm_rmsnorm_gemv")


def qmm_rmsnorm_gate_up_silu(fmt, Wg, Wu, x, gamma, eps, h, I, K, N, stream=None) -> None:
    _check(_lib.qmm_rmsnorm_gate_up_silu(fmt, _ptr(Wg), _ptr(Wu), _ptr(x), _ptr(gamma), eps, _ptr(h), I, K, N,
                                         _stream(stream)), "qmm_rmsnorm_gate_up_silu")


def qmm_gemv_add(fmt, W, x, r, y, M, K, N, stream=None) -> None:
    _check(_lib.qmm_gemv_add(fmt, _ptr(W), _ptr(x), _ptr(r), _ptr(y), M, K, N, _stream(stream)), "qmm_gemv_add")


def qmm_gemm(fmt, W, X, Y, M, K, T, workspace=None, workspace_bytes=None, stream=None) -> None:
    wp, wb, _keep = _workspace(QMM_OP_GEMM, fmt, M, K, T, QMM_VARIANT_AUTO, (Y, X), workspace, workspace_bytes)
    _check(_lib.qmm_gemm(fmt, _ptr(W), _ptr(X), _ptr(Y), M, K, T, wp, wb, _stream(stream)), "qmm_gemm")


def qmm_gemm_noalloc(fmt, W, X, Y, M, K, T, stream=None) -> None:
    _check(_lib.qmm_gemm_noalloc(fmt, _ptr(W), _ptr(X), _ptr(Y), M, K, T, _stream(stream)), "qmm_gemm_noalloc")


def qmm_stream_read(buf, nbytes, sink, stream=None) -> None:
    _check(_lib.qmm_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "qmm_stream_read")


def qmm_gemm_gate_up_silu(fmt, Wg, Wu, X, H, I, K, T, workspace=None, workspace_bytes=None, stream=None) -> None:
    wp, wb, _keep = _workspace(QMM_OP_GEMM_GATE_UP_SILU, fmt, I, K, T, QMM_VARIANT_AUTO, (H, X), workspace,
                               workspace_bytes)
    _check(_lib.qmm_gemm_gate_up_silu(fmt, _ptr(Wg), _ptr(Wu), _ptr(X), _ptr(H), I, K, T, wp, wb, _stream(stream)),
           "qmm_gemm_gate_up_silu")


# ------------------------------------------- conveniences (allocate the output)
def _out(shape, like, out):
    if out is not None:
        return out
    return torch.empty(shape, dtype=torch.float32, device=like.device)


def dequant(fmt, W, M, K, out=None, stream=None):
    out = _out((M, K), W, out)
    qmm_dequant(fmt, W, out, M, K, stream)
    return out


def get_rows(fmt, W, ids, M, K, out=None, stream=None):
    """out[i] = W[ids[i]] in fp32 (ids: int32 device tensor)."""
    n = ids.numel()
    out = _out((n, K), W, out)
    qmm_get_rows(fmt, W, ids, out, M, K, n, stream)
    return out


def expand_f16(fmt, W, M, K, out=None, stream=None):
    """fp16 copy of the whole matrix (round to nearest even)."""
    if out is None:
        out = torch.empty((M, K), dtype=torch.float16, device=W.device)
    qmm_expand_f16(fmt, W, out, M, K, stream)
    return out


def gemv(fmt, W, x, M, K, out=None, variant=QMM_VARIANT_AUTO, workspace=None, stream=None):
    """y[N][M] = x[N][K] W^T for fp32 x (N = x.shape[0] or 1 for a vector)."""
    N = 1 if x.dim() == 1 else x.shape[0]
    out = _out((N, M), x, out)
    qmm_gemv_variant(fmt, W, x, out, M, K, N, variant, workspace, None, stream)
    return out


def gate_up_silu(fmt, Wg, Wu, x, I, K, out=None, variant=QMM_VARIANT_AUTO, workspace=None, stream=None):
    N = 1 if x.dim() == 1 else x.shape[0]
    out = _out((N, I), x, out)
    qmm_gate_up_silu_variant(fmt, Wg, Wu, x, out, I, K, N, variant, workspace, None, stream)
    return out


def rmsnorm_gemv(fmt, W, x, gamma, eps, M, K, out=None, stream=None):
    """y = rmsnorm(x; gamma, eps) W^T for fp32 x."""
    N = 1 if x.dim() == 1 else x.shape[0]
    out = _out((N, M), x, out)
    qmm_rmsnorm_gemv(fmt, W, x, gamma, eps, out, M, K, N, stream)
    return out


def rmsnorm_gate_up_silu(fmt, Wg, Wu, x, gamma, eps, I, K, out=None, stream=None):
    N = 1 if x.dim() == 1 else x.shape[0]
    out = _out((N, I), x, out)
    qmm_rmsnorm_gate_up_silu(fmt, Wg, Wu, x, gamma, eps, out, I, K, N, stream)
    return out


def gemv_add(fmt, W, x, r, M, K, out=None, stream=None):
    """y = x W^T + r; pass out=r to add into r in place."""
    N = 1 if x.dim() == 1 else x.shape[0]
    out = _out((N, M), x, out)
    qmm_gemv_add(fmt, W, x, r, out, M, K, N, stream)
    return out


def gemm(fmt, W, X, M, K, out=None, workspace=None, stream=None):
    """Y[T][M] = X[T][K] W^T for fp16 X."""
    T = X.shape[0]
    out = _out((T, M), X, out)
    qmm_gemm(fmt, W, X, out, M, K, T, workspace, None, stream)
    return out


def gemm_gate_up_silu(fmt, Wg, Wu, X, I, K, out=None, workspace=None, stream=None):
    T = X.shape[0]
    out = _out((T, I), X, out)
    qmm_gemm_gate_up_silu(fmt, Wg, Wu, X, out, I, K, T, workspace, None, stream)
    return out
