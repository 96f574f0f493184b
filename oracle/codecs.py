"""Number formats used by the ROW_MX / MX FP8 path (oracle; test infrastructure only).

* FP8 E4M3 ("fn" variant: no infinities, one NaN pattern per sign).  [QKV-CTE] "Upstream
  behavior" names the FP8 weight and the FP8 activation codes; [RMSNORM-MX] ``qmx_output_dtype``
  names ``float8_e4m3fn``.  Field layout: sign(1) exponent(4, bias 7) mantissa(3).
* E8M0 block scale: an unsigned biased exponent, value 2^(e - 127); 0xFF is NaN.
* bf16: the upper 16 bits of an IEEE binary32 (the dtype every output of the path is stored in).

Everything decodes to float64, in which every value of these formats is exact.
"""
from __future__ import annotations

import numpy as np


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes, from the bit fields (NaN for 0x7F / 0xFF)."""
    vals = np.empty(256, np.float64)
    for b in range(256):
        s = -1.0 if (b >> 7) & 1 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            vals[b] = np.nan
        elif e == 0:
            vals[b] = s * (m / 8.0) * 2.0 ** -6          # subnormal
        else:
            vals[b] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
E4M3_MAX = 448.0


def e4m3_decode(codes, allow_nan: bool = False) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values.  Raises on a NaN code unless ``allow_nan``."""
    c = np.asarray(codes, dtype=np.uint8)
    v = E4M3_VALUES[c]
    if not allow_nan and np.isnan(v).any():
        raise ValueError("NaN E4M3 code in input")
    return v


def e8m0_decode(codes) -> np.ndarray:
    """uint8 E8M0 scales -> float64 2^(e-127).  Raises on the NaN code 0xFF."""
    c = np.asarray(codes, dtype=np.uint8)
    if (c == 0xFF).any():
        raise ValueError("NaN E8M0 code in input")
    return np.ldexp(1.0, c.astype(np.int64) - 127)


# Non-negative finite E4M3 values in code order 0x00..0x7E (monotonically increasing).
_POS_VALUES = E4M3_VALUES[:0x7F].copy()


def e4m3_encode(v) -> np.ndarray:
    """float32 -> E4M3 code, round-to-nearest (ties to the even code), saturating to +-448.

    Written as the definition: among the 127 non-negative finite values pick the nearest to
    |v|; on an exact tie pick the code whose mantissa LSB is 0; magnitudes above 448 clamp to
    448 (0x7E) instead of becoming NaN.  The sign bit is copied from v, so -0.0 and negative
    values that round to zero give 0x80.  NaN input raises.
    """
    x = np.asarray(v, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN input to E4M3 encoder")
    neg = np.signbit(x)
    a = np.abs(x.astype(np.float64))
    a = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")            # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS_VALUES[hi], hi, code)            # exact hit
    return (code.astype(np.uint8) | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns with a single round-to-nearest-even (ties to even).

    Candidates are the two bf16 values bracketing x (truncation toward zero and the next one
    away from zero); the nearer wins, an exact tie goes to the even pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN input to bf16 rounding")
    neg = np.signbit(x)
    a = np.abs(x)
    # largest bf16 <= a: take the fp32 rounding-down of a, then clear the low 16 bits
    f = a.astype(np.float32)
    f = np.where(f.astype(np.float64) > a, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    lo_bits = f.view(np.uint32) & np.uint32(0xFFFF0000)
    lo = lo_bits.view(np.float32).astype(np.float64)
    hi_bits = lo_bits + np.uint32(0x10000)
    # value of the next bf16 step above lo, in fp64 (2^128 when the step overflows to +inf)
    e = ((lo_bits >> 23) & np.uint32(0xFF)).astype(np.int64)
    ulp = np.ldexp(1.0, np.where(e == 0, -133, e - 127 - 7))
    hi = lo + ulp
    d_lo = a - lo
    d_hi = hi - a
    even_lo = ((lo_bits >> 16) & 1) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~even_lo)
    bits = np.where(pick_hi, hi_bits, lo_bits) >> 16
    bits = bits.astype(np.uint32) | (neg.astype(np.uint32) << 15)
    return bits.astype(np.uint16)


def bf16_round_f32(x32) -> np.ndarray:
    """float32 -> bf16 bit patterns (RNE).  Every fp32 value is exact in fp64, so this is
    the single rounding of ``f64_to_bf16`` applied to the fp32 value."""
    x32 = np.asarray(x32, dtype=np.float32)
    return f64_to_bf16(x32.astype(np.float64))
