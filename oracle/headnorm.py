"""Per-head qk-norm and rotate-half RoPE applied to the projection's result (oracle; test
infrastructure only).

[QKV-CTE] "Upstream behavior": the upstream kernel optionally fuses a *per-head* qk-norm
(RMS_NORM or LAYER_NORM) and rotate-half RoPE into the step that brings each finished matmul
result out of the accumulators, together with the dequant scaling and the bias add, so no HBM
round trip is needed.  "Design 1)": upstream qk-norm normalises each head's d_head slice by its
own statistics (as opposed to Wan's one RMS over the whole Q or K vector).

Readings taken (the pages do not spell them out):
  * the norm applies to the dequantised, bias-added fp32 value X of pass 1 (before rounding);
  * RMS_NORM:   y = x / sqrt(mean(x^2) + eps) * gamma
    LAYER_NORM: y = (x - mean(x)) / sqrt(mean((x - mean(x))^2) + eps) * gamma + beta
    with the statistics over the d_head values of one head of one token, gamma (and beta) of
    length d_head shared by the heads of a segment (Q and K each have their own), beta = 0 when
    absent; eps as the fp32 value given;
  * the norm precedes RoPE (as for the across-heads norm), RoPE pairs lane j with lane j + d/2
    of the same head with the angle of row position j (the rotate-half tables' two halves hold
    the same angle);
  * V is neither normalised nor rotated; the result is rounded to bf16 once, on store.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f64
from .norm_rope import _rotate_half

RMS_NORM = 1
LAYER_NORM = 2


def _norm_heads(x, kind: int, gamma_bf16, beta_bf16, eps: float, d: int):
    """x float64 [T, n * d] -> per-head normalised float64 [T, n * d]."""
    T, w = x.shape
    xh = x.reshape(T, w // d, d)
    e = float(np.float32(eps))
    if kind == RMS_NORM:
        y = xh / np.sqrt(np.mean(xh * xh, axis=-1, keepdims=True) + e)
    elif kind == LAYER_NORM:
        c = xh - np.mean(xh, axis=-1, keepdims=True)
        y = c / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + e)
    else:
        raise ValueError("norm kind must be RMS_NORM or LAYER_NORM")
    y = y * bf16_to_f64(gamma_bf16)[None, None, :]
    if beta_bf16 is not None:
        if kind != LAYER_NORM:
            raise ValueError("beta belongs to LAYER_NORM")
        y = y + bf16_to_f64(beta_bf16)[None, None, :]
    return y.reshape(T, w)


def _rope_heads(y, cos, sin, d: int):
    T, w = y.shape
    yh = y.reshape(T, w // d, d)
    c = np.asarray(cos, dtype=np.float32).astype(np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float32).astype(np.float64)[:, None, :]
    return (yh * c + _rotate_half(yh, d) * s).reshape(T, w)


def head_norm_rope(X, kind: int, q_gamma_bf16, k_gamma_bf16, eps: float, cos=None, sin=None, *,
                   num_heads: int, num_kv_heads: int, head_dim: int, q_beta_bf16=None,
                   k_beta_bf16=None) -> np.ndarray:
    """X float64 [T, I] (pass 1 before rounding) -> float64 [T, I] with the Q and K heads
    normalised per head (then rotated when cos / sin are given) and V unchanged."""
    X = np.asarray(X, dtype=np.float64)
    d = head_dim
    Iq, Ik = num_heads * d, num_kv_heads * d
    if (cos is None) != (sin is None):
        raise ValueError("cos and sin come together")
    out = X.copy()
    segs = [(0, Iq, q_gamma_bf16, q_beta_bf16)]
    if Ik:
        segs.append((Iq, Iq + Ik, k_gamma_bf16, k_beta_bf16))
    for lo, hi, g, b in segs:
        y = _norm_heads(X[:, lo:hi], kind, g, b, eps, d)
        if cos is not None:
            y = _rope_heads(y, cos, sin, d)
        out[:, lo:hi] = y
    return out
