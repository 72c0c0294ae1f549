"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers (numpy ``Generator(PCG64(seed))``) and lays
them out in the GGUF block byte layouts through numpy structured dtypes.  It holds
none of the method's arithmetic: nothing here decodes a block or forms a product
with the activations (the one product, a bias drawn relative to its block's scale,
shapes a distribution).  Both the float64 oracle and the GPU library consume the
bytes it returns; each decodes them with its own code.

Block layouts (EdgeRunner Core Architecture, section 3.1 "Quantization Format
Summary" and section 3.2 "Q8_0 Layout"; GGUF type ids from section 1.3):

* Q8_0, type id 8: 34 bytes per 32 weights = fp16 scale (little endian) followed
  by 32 signed bytes.
* Q4_0, type id 2: 18 bytes per 32 weights = fp16 scale followed by 16 bytes
  holding 32 four-bit codes (two per byte).
* Q4_1, type id 3: 20 bytes = fp16 scale, fp16 bias, 16 code bytes.
* Q5_0, type id 6: 22 bytes = fp16 scale, 4 bytes of fifth bits, 16 code bytes.
* Q5_1, type id 7: 24 bytes = fp16 scale, fp16 bias, 4 bytes of fifth bits, 16 code
  bytes.  (The pages give these byte counts; the field order is the GGUF one.)
* F16, type id 1: 2 bytes per weight.

Distributions follow the workloads the library is measured on: Q8_0 codes uniform
in [-127, 127], Q4_0 codes uniform in 0..15 (a uniform byte carries two
independent uniform nibbles), fp16 scales uniform in [1e-3, 1e-2], F16 weights
normal with standard deviation 0.02, activations standard normal.  Q4_1 / Q5_0 /
Q5_1 code bytes and fifth-bit words are uniform bytes (uniform 4- and 5-bit codes);
the biases of Q4_1 and Q5_1 are drawn as -(6..9) scales per block and -(12..18) scales
per block respectively, where a min/max quantiser puts the block minimum of normal
weights.
"""
from __future__ import annotations

import numpy as np

FMT_F16 = 1
FMT_Q4_0 = 2
FMT_Q4_1 = 3
FMT_Q5_0 = 6
FMT_Q5_1 = 7
FMT_Q8_0 = 8
FORMATS = (FMT_F16, FMT_Q4_0, FMT_Q8_0)
BIAS_FORMATS = (FMT_Q4_1, FMT_Q5_0, FMT_Q5_1)
FMT_NAMES = {FMT_F16: "F16", FMT_Q4_0: "Q4_0", FMT_Q8_0: "Q8_0", FMT_Q4_1: "Q4_1", FMT_Q5_0: "Q5_0",
             FMT_Q5_1: "Q5_1"}

# Packed (unaligned) structured dtypes: itemsize 34, 18, 20, 22, 24 exactly.
Q8_0_BLOCK = np.dtype([("d", "<f2"), ("qs", "i1", (32,))])
Q4_0_BLOCK = np.dtype([("d", "<f2"), ("qs", "u1", (16,))])
Q4_1_BLOCK = np.dtype([("d", "<f2"), ("m", "<f2"), ("qs", "u1", (16,))])
Q5_0_BLOCK = np.dtype([("d", "<f2"), ("qh", "u1", (4,)), ("qs", "u1", (16,))])
Q5_1_BLOCK = np.dtype([("d", "<f2"), ("m", "<f2"), ("qh", "u1", (4,)), ("qs", "u1", (16,))])
BLOCK_DTYPES = {FMT_Q8_0: Q8_0_BLOCK, FMT_Q4_0: Q4_0_BLOCK, FMT_Q4_1: Q4_1_BLOCK, FMT_Q5_0: Q5_0_BLOCK,
                FMT_Q5_1: Q5_1_BLOCK}
assert [BLOCK_DTYPES[f].itemsize for f in (8, 2, 3, 6, 7)] == [34, 18, 20, 22, 24]

# Rows are drawn in fixed-size chunks so that very large matrices (a 128256-row
# output head) stay within host memory; the chunk size is part of the recipe.
_CHUNK_ROWS = 4096


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def layout_bytes(fmt: int, K: int) -> int:
    """Bytes of one row in the block layout (a size statement, used for allocation)."""
    if fmt == FMT_F16:
        return 2 * K
    if K % 32:
        raise ValueError("block formats need K % 32 == 0")
    return (K // 32) * BLOCK_DTYPES[fmt].itemsize


def _scales(g: np.random.Generator, rows: int, nb: int, scale_mode: str) -> np.ndarray:
    if scale_mode == "uniform":
        return g.uniform(1e-3, 1e-2, size=(rows, nb)).astype(np.float16)
    if scale_mode == "wide":
        # Any finite fp16 bit pattern with a random sign: zeros, subnormals,
        # negatives and the largest finite values all appear.
        bits = g.integers(0, 0x7C00, size=(rows, nb), dtype=np.uint16)
        bits |= (g.integers(0, 2, size=(rows, nb), dtype=np.uint16) << 15).astype(np.uint16)
        return bits.view(np.float16)
    if scale_mode == "gemm_wide":
        # Finite fp16 scales of either sign with magnitude below 2**8, so that
        # scale * code stays finite in fp16 (|code| <= 128).
        bits = g.integers(0, 0x5C00, size=(rows, nb), dtype=np.uint16)
        bits |= (g.integers(0, 2, size=(rows, nb), dtype=np.uint16) << 15).astype(np.uint16)
        return bits.view(np.float16)
    raise ValueError(scale_mode)


def weights(fmt: int, M: int, K: int, seed: int, *, scale_mode: str = "uniform",
            q8_low: int = -127) -> np.ndarray:
    """Raw weight bytes for an M x K matrix, row-major, as a flat uint8 array.

    Per chunk of rows the draw order is: codes, then scales (F16: values only).
    ``q8_low`` = -128 widens the Q8_0 code range to the full int8 range.
    """
    g = rng(seed)
    row_bytes = layout_bytes(fmt, K)
    out = np.empty(M * row_bytes, dtype=np.uint8)
    nb = K // 32
    for r0 in range(0, M, _CHUNK_ROWS):
        rows = min(_CHUNK_ROWS, M - r0)
        dst = out[r0 * row_bytes:(r0 + rows) * row_bytes]
        if fmt == FMT_Q8_0:
            blk = dst.view(Q8_0_BLOCK).reshape(rows, nb)
            blk["qs"] = g.integers(q8_low, 128, size=(rows, nb, 32), dtype=np.int8)
            blk["d"] = _scales(g, rows, nb, scale_mode)
        elif fmt == FMT_Q4_0:
            blk = dst.view(Q4_0_BLOCK).reshape(rows, nb)
            blk["qs"] = g.integers(0, 256, size=(rows, nb, 16), dtype=np.uint8)
            blk["d"] = _scales(g, rows, nb, scale_mode)
        elif fmt in BIAS_FORMATS:
            blk = dst.view(BLOCK_DTYPES[fmt]).reshape(rows, nb)
            blk["qs"] = g.integers(0, 256, size=(rows, nb, 16), dtype=np.uint8)
            if fmt != FMT_Q4_1:
                blk["qh"] = g.integers(0, 256, size=(rows, nb, 4), dtype=np.uint8)
            d = _scales(g, rows, nb, scale_mode)
            blk["d"] = d
            if fmt != FMT_Q5_0:
                if scale_mode == "uniform":
                    lo, hi = (6.0, 9.0) if fmt == FMT_Q4_1 else (12.0, 18.0)
                    blk["m"] = (-g.uniform(lo, hi, size=(rows, nb)) * d.astype(np.float64)).astype(np.float16)
                else:
                    blk["m"] = _scales(g, rows, nb, scale_mode)
        elif fmt == FMT_F16:
            dst.view(np.float16)[:] = g.normal(0.0, 0.02, size=rows * K).astype(np.float16)
        else:
            raise ValueError(f"unknown format {fmt}")
    return out


# fp16 bit patterns written into every block of device_weights: scale 2^-8 (0x1C00);
# the biased formats' bias -2^-4 (0xAC00), about -16 scales.
_DEV_SCALE = (0x00, 0x1C)
_DEV_BIAS = (0x00, 0xAC)


def device_weights(fmt: int, M: int, K: int, seed: int, device):
    """Raw weight bytes drawn on the device (torch's seeded generator), for matrices too
    large to draw on the host: uniform code bytes, and every block's scale (and bias)
    set to the fixed fp16 patterns above so that every weight is finite.  Returns a
    flat uint8 device tensor; tests read back the bytes of the rows they check."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    rb = layout_bytes(fmt, K)
    w = torch.randint(0, 256, (M * rb,), dtype=torch.uint8, device=device, generator=g)
    if fmt != FMT_F16:
        blk = w.view(-1, BLOCK_DTYPES[fmt].itemsize)
        blk[:, 0] = _DEV_SCALE[0]
        blk[:, 1] = _DEV_SCALE[1]
        if fmt in (FMT_Q4_1, FMT_Q5_1):
            blk[:, 2] = _DEV_BIAS[0]
            blk[:, 3] = _DEV_BIAS[1]
    else:
        # keep F16 weights finite: clear the top exponent bit of every half
        w.view(-1, 2)[:, 1] &= 0xBF
    return w


def activations(N: int, K: int, seed: int, dtype=np.float32) -> np.ndarray:
    """Standard-normal activations [N][K] (fp32 for decode, fp16 for prefill)."""
    return rng(seed).standard_normal((N, K)).astype(dtype)


def one_hot(N: int, K: int, cols, dtype=np.float32) -> np.ndarray:
    """Activations whose row n is the unit vector e_{cols[n]}."""
    x = np.zeros((N, K), dtype=dtype)
    for n, c in enumerate(cols):
        x[n, c] = 1
    return x


# Shapes of the workloads (hidden/intermediate sizes and head layouts).
SMOLLM2_135M = dict(layers=30, hidden=576, heads=9, kv_heads=3, head_dim=64,
                    intermediate=1536, vocab=49152)
LLAMA3_8B = dict(layers=32, hidden=4096, heads=32, kv_heads=8, head_dim=128,
                 intermediate=14336, vocab=128256)


def qkv_rows(cfg: dict) -> int:
    return (cfg["heads"] + 2 * cfg["kv_heads"]) * cfg["head_dim"]
