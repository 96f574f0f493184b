"""MX block-32 FP8 weight encoding and the pages' ``[H // 4, I, 4]`` weight layout
(oracle; test infrastructure only).

[QKV-CTE] "Interface": ``weight`` is ``[H // 4, I, 4]`` FP8, "MX-contiguous": four consecutive
contraction (H) elements of one output column share a 4-byte group, i.e. element (h, i) lives at
flat byte ``((h // 4) * I + i) * 4 + h % 4``.  The block scales are one E8M0 exponent per 32
consecutive H elements of a column, stored here as ``[H // 32, I]``.

How a weight's E8M0 exponent is chosen is not stated on the pages; the plain reading taken is
the OCP Microscaling (MX v1.0) shared-exponent rule: for a block with largest magnitude m,
X = floor(log2 m) - 8 (8 = the largest E4M3 exponent), E = X + 127 clamped to the finite E8M0
range [0, 254], and each element is encoded as E4M3_RNE_satfinite(w / 2^(E - 127)).  An
all-zero block gets E = 0 and zero codes.  The projection
consumes whatever codes and exponents it is given, so this choice only shapes the inputs.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import e4m3_decode, e4m3_encode, e8m0_decode


def _floor_log2(m: float) -> int:
    """floor(log2 m) for a positive finite double, exactly (via frexp: m = f * 2^e, 0.5<=f<1)."""
    _, e = math.frexp(m)
    return e - 1


def mx_weight_quantize(w, rows_per_chunk: int = 256):
    """fp32 W [H, I] -> (codes uint8 [H // 4, I, 4], e8m0 uint8 [H // 32, I]).

    Processed ``rows_per_chunk`` rows of H at a time (whole 32-row blocks) to bound the memory
    of the temporaries; the blocks are independent, so the result does not depend on it.
    """
    w = np.asarray(w, dtype=np.float32)
    H, I = w.shape
    if H % 32:
        raise ValueError("H must be a multiple of 32")
    step = max(32, rows_per_chunk - rows_per_chunk % 32)
    codes = np.empty((H // 4, I, 4), np.uint8)
    e8 = np.empty((H // 32, I), np.uint8)
    for h0 in range(0, H, step):
        h1 = min(H, h0 + step)
        c, e = _quantize_rows(w[h0:h1])
        codes[h0 // 4:h1 // 4] = c
        e8[h0 // 32:h1 // 32] = e
    return codes, e8


def _quantize_rows(w):
    """One group of whole 32-row blocks: fp32 [h, I] -> ([h // 4, I, 4], [h // 32, I])."""
    H, I = w.shape
    if not np.isfinite(w).all():
        raise ValueError("non-finite weight")
    nb = H // 32
    blocks = w.reshape(nb, 32, I)
    amax = np.max(np.abs(blocks), axis=1).astype(np.float64)        # [nb, I]
    nz = amax > 0
    fl = np.vectorize(_floor_log2, otypes=[np.int64])(np.where(nz, amax, 1.0))
    # E = X + 127 clamped to the finite E8M0 range [0, 254]; the element scale is 2^(E - 127)
    E = np.where(nz, np.clip(fl - 8 + 127, 0, 254), 0)
    X = E - 127
    # w / 2^X is exact in fp32: X >= -127, so a finite fp32 w (subnormals included) scales to
    # a value with at most 24 significant bits and magnitude between 2^-22 and 2^9; computed in
    # fp64 and narrowed exactly (checked below).
    scaled = blocks.astype(np.float64) * np.ldexp(1.0, -X)[:, None, :]
    scaled32 = scaled.astype(np.float32)
    if not np.array_equal(scaled32.astype(np.float64), scaled):
        raise ValueError("power-of-two rescale not exact")
    q = e4m3_encode(scaled32)                                        # [nb, 32, I]
    q = np.where(nz[:, None, :], q, 0).astype(np.uint8)
    q_hi = q.reshape(H, I)                                           # natural [H, I]
    codes = q_hi.reshape(H // 4, 4, I).transpose(0, 2, 1).copy()     # -> [H//4, I, 4]
    return codes, E.astype(np.uint8)


def mx_weight_decode(codes, e8m0) -> np.ndarray:
    """(codes [H // 4, I, 4], e8m0 [H // 32, I]) -> float64 W [H, I] (exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    H4, I, four = c.shape
    if four != 4:
        raise ValueError("weight codes must be [H // 4, I, 4]")
    H = H4 * 4
    # element (h, i) = c[h // 4, i, h % 4]
    nat = c.transpose(0, 2, 1).reshape(H, I)
    vals = e4m3_decode(nat)
    sc = e8m0_decode(np.asarray(e8m0, dtype=np.uint8))               # [H // 32, I]
    if sc.shape != (H // 32, I):
        raise ValueError("e8m0 scales must be [H // 32, I]")
    return vals * np.repeat(sc, 32, axis=0)
