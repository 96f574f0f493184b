"""MX block-32 FP8 encoding of activations (oracle; test infrastructure only).

[RMSNORM-MX] ``qmx_output_dtype`` (float8_e4m3fn_x4 packed MX output) and ``pack_scales``:
``quantize_mx`` emits one uint8 (E8M0) scale per 32-element block of the hidden dimension.  The
pages' row packing of those scales and their H-swizzle belong to the other machine's transpose
and are not reproduced: here a row's codes are ``[H]`` E4M3 in natural H order and its scales
``[H // 32]`` E8M0, block b covering elements [32 b, 32 b + 32).

The shared exponent of a block follows the same rule as the weight's (the OCP Microscaling v1.0
rule, see mxweight.py): for block maximum magnitude m, E = clamp(floor(log2 m) - 8 + 127, 0, 254),
elements encoded as E4M3_RNE_satfinite(y / 2^(E - 127)); an all-zero block gets E = 0 and zero
codes.  A block along H of one token is a block along the contraction of one column of y^T, so
the encoding is the weight encoder applied to the transposed activations.
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_decode, e8m0_decode
from .mxweight import mx_weight_quantize


def mx_block_quantize(y, rows_per_chunk: int = 1024):
    """fp32 y [T, H] -> (codes uint8 [T, H], e8m0 uint8 [T, H // 32])."""
    y = np.asarray(y, dtype=np.float32)
    T, H = y.shape
    if H % 32:
        raise ValueError("H must be a multiple of 32")
    codes = np.empty((T, H), np.uint8)
    e8 = np.empty((T, H // 32), np.uint8)
    for t0 in range(0, T, rows_per_chunk):
        t1 = min(T, t0 + rows_per_chunk)
        c, e = mx_weight_quantize(y[t0:t1].T)            # [H // 4, t, 4], [H // 32, t]
        codes[t0:t1] = c.transpose(0, 2, 1).reshape(H, t1 - t0).T
        e8[t0:t1] = e.T
    return codes, e8


def mx_block_decode(codes, e8m0) -> np.ndarray:
    """(codes [T, H], e8m0 [T, H // 32]) -> float64 [T, H] (exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    T, H = c.shape
    sc = e8m0_decode(np.asarray(e8m0, dtype=np.uint8))
    if sc.shape != (T, H // 32):
        raise ValueError("e8m0 scales must be [T, H // 32]")
    return e4m3_decode(c) * np.repeat(sc, 32, axis=1)
