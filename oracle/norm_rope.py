"""Pass 2: across-heads RMSNorm and rotate-half RoPE on Q and K, in place; V untouched
(oracle; test infrastructure only).

[QKV-CTE] "Design 1)", step b: inv_rms = rsqrt(sum / (n_heads * d_head * tp) + eps) per token,
for Q and for K (tp = 1 here: every head is local).  Each segment uses its own head count.
Step c: re-read each token's Q / K as stored, multiply by the segment-wide per-channel gamma
(``[1, n_heads * d_head]``, "Interface") and by inv_rms, store the result over the
input; V is never normed and never re-read.
[QKV-CTE] "Design 2)": the norm precedes RoPE; rotate-half pairs lane j with lane j + d/2 and
out = (x * inv_rms) * cos + [-x_hi, x_lo] * inv_rms * sin, with the per-position cos / sin row
shared by every head.  The x in that formula is read here as the gamma-scaled value, i.e.
out = RoPE(RMSNorm_gamma(x)).
[QKV-CTE] "Design 5)": with num_kv_heads == 0 the whole projection is the Q segment.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f64

NORM_Q = 1
NORM_K = 2
FUSED_ROPE = 4


def inv_rms(ssq, n_heads: int, head_dim: int, eps: float) -> np.ndarray:
    """1 / sqrt(ssq / (n_heads * head_dim) + eps) in float64; eps is the fp32 value given."""
    ssq = np.asarray(ssq, dtype=np.float64)
    e = float(np.float32(eps))
    return 1.0 / np.sqrt(ssq / float(n_heads * head_dim) + e)


def _rotate_half(y, d: int):
    """[-y_hi, y_lo] per head: lane j < d/2 takes -y[j + d/2], lane j >= d/2 takes y[j - d/2]."""
    h = d // 2
    return np.concatenate([-y[..., h:], y[..., :h]], axis=-1)


def _segment(x, gamma_bf16, r, cos, sin, d: int, norm: bool, rope: bool):
    """x float64 [T, n*d] -> transformed float64 [T, n*d]."""
    T, w = x.shape
    n = w // d
    y = x
    if norm:
        y = y * bf16_to_f64(gamma_bf16)[None, :] * r[:, None]
    if rope:
        yh = y.reshape(T, n, d)
        c = np.asarray(cos, dtype=np.float32).astype(np.float64)[:, None, :]
        s = np.asarray(sin, dtype=np.float32).astype(np.float64)[:, None, :]
        yh = yh * c + _rotate_half(yh, d) * s
        y = yh.reshape(T, w)
    return y


def norm_rope(qkv_bf16, ssq, q_gamma_bf16, k_gamma_bf16, cos, sin, *, num_heads: int,
              num_kv_heads: int, head_dim: int, eps: float, flags: int,
              values=None) -> np.ndarray:
    """qkv_bf16 uint16 [T, I] (as stored by pass 1) -> float64 [T, I] after pass 2.

    ``flags``: NORM_Q / NORM_K select the across-heads norm per segment, FUSED_ROPE applies
    rotate-half RoPE to both Q and K.  Columns outside Q and K come back bit-for-bit.
    ``values`` (float64 [T, I]) replaces the stored bf16 input, e.g. with pass 1's unrounded
    result to follow the whole chain without intermediate rounding.
    """
    d = head_dim
    Iq = num_heads * d
    Ik = num_kv_heads * d
    x = bf16_to_f64(qkv_bf16) if values is None else np.asarray(values, dtype=np.float64)
    out = x.copy()
    rope = bool(flags & FUSED_ROPE)
    if rope and (cos is None or sin is None):
        raise ValueError("RoPE needs cos / sin tables")
    if (flags & NORM_K) and num_kv_heads == 0:
        raise ValueError("no K segment to norm")
    ssq = np.asarray(ssq, dtype=np.float64)
    rq = inv_rms(ssq[:, 0], num_heads, d, eps) if flags & NORM_Q else None
    out[:, :Iq] = _segment(x[:, :Iq], q_gamma_bf16, rq, cos, sin, d, bool(flags & NORM_Q), rope)
    if Ik:
        rk = inv_rms(ssq[:, 1], num_kv_heads, d, eps) if flags & NORM_K else None
        out[:, Iq:Iq + Ik] = _segment(x[:, Iq:Iq + Ik], k_gamma_bf16, rk, cos, sin, d,
                                      bool(flags & NORM_K), rope)
    return out
