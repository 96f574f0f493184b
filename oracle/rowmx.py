"""ROW_MX activation encoding (oracle; test infrastructure only).

[QKV-CTE] "Upstream behavior" and the ``packed_hidden`` row of the "Interface" table: the
activation arrives row-packed, ``[B, S, H + 4]``: H FP8 codes followed by a 4-byte fp32 dequant
scale tail; the projection kernel itself does not quantise bf16 input.

Encoding of one row y (fp32) used here (the plain reading):
  s     = fl32(max_h |y_h| / 448)              (IEEE fp32 division)
  q_h   = E4M3_RNE_satfinite(fl32(y_h / s))    (IEEE fp32 division, then one rounding to E4M3)
  bytes = q[0:H] ++ little-endian fp32 bits of s
A row of zeros gets s = 0 and all-zero codes.  Dequantisation is dec(q_h) * s.
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_encode, E4M3_MAX


def rowmx_quantize(y, rows_per_chunk: int = 1024) -> np.ndarray:
    """fp32 [T, H] -> packed uint8 [T, H + 4] (rows are independent; processed in chunks of
    ``rows_per_chunk`` to bound the memory of the temporaries)."""
    y = np.asarray(y, dtype=np.float32)
    if y.ndim != 2:
        raise ValueError("rows must be 2-D")
    if y.shape[0] > rows_per_chunk:
        out = np.empty((y.shape[0], y.shape[1] + 4), np.uint8)
        for r0 in range(0, y.shape[0], rows_per_chunk):
            out[r0:r0 + rows_per_chunk] = _quantize_rows(y[r0:r0 + rows_per_chunk])
        return out
    return _quantize_rows(y)


def _quantize_rows(y) -> np.ndarray:
    if not np.isfinite(y).all():
        raise ValueError("non-finite activation")
    T, H = y.shape
    amax = np.max(np.abs(y), axis=1) if H else np.zeros(T, np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)           # fp32 / fp32, RNE
    zero = s == 0
    safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
    v = (y / safe[:, None]).astype(np.float32)                       # fp32 / fp32, RNE
    q = e4m3_encode(v)
    q[zero] = 0
    out = np.empty((T, H + 4), np.uint8)
    out[:, :H] = q
    out[:, H:] = s.astype("<f4").view(np.uint8).reshape(T, 4)
    return out


def rowmx_unpack(packed, H: int):
    """packed [T, H + 4] -> (codes uint8 [T, H], scale float32 [T])."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.ndim != 2 or p.shape[1] != H + 4:
        raise ValueError("packed rows must be [T, H + 4]")
    codes = p[:, :H]
    scale = np.ascontiguousarray(p[:, H:H + 4]).view("<f4").reshape(-1).astype(np.float32)
    return codes, scale
