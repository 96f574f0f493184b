"""Pass 1: the ROW_MX x MX FP8 QKV projection and the per-token segment sums of squares
(oracle; test infrastructure only).

[QKV-CTE] "Upstream behavior": O[S, I] = A[S, H] @ W[H, I] (+ bias), with
I = (num_q_heads + 2 * num_kv_heads) * d_head and the output columns ordered Q | K | V.
[QKV-CTE] "Applies to / Pattern": each output tile accumulates over the whole contraction, is
then dequantised, bias-added and stored.  "Interface": ``weight_scales`` is a per-output-channel
fp32 dequant scale ``[1, I]``; ``bias`` is ``[1, I]``; the result is bf16.

Dequantisation used (the plain reading of the two scale kinds: the pages' per-channel fp32
weight scale and the MX weight's per-32 E8M0 exponents both apply, and multiply):
  X[s, i] = sA[s] * c[i] * sum_h dec(A[s, h]) * dec(W[h, i]) * 2^(E[h // 32, i] - 127) + bias[i]
with sA the row's fp32 ROW_MX scale, c the per-channel weight scale (1 when absent) and E the
block exponent.  With MX block-32 activations ([RMSNORM-MX] ``qmx_output_dtype``) the row scale
is replaced by a per-block factor inside the sum: dec(A[s, h]) * 2^(Ea[s, h // 32] - 127).  Everything is evaluated in float64; the bf16 output is one rounding of X.

[QKV-CTE] "Design 1)", step a: per token, the sum of x^2 over the whole Q segment and over the
whole K segment of the un-normalised output; V is excluded.  "Design 5)": with
num_kv_heads == 0 there is no K segment and its sum is skipped (reported here as 0).
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f64, e4m3_decode
from .mxact import mx_block_decode
from .mxweight import mx_weight_decode


def segment_ssq(X, num_heads: int, num_kv_heads: int, head_dim: int) -> np.ndarray:
    """Per-token [sum over Q segment of X^2, sum over K segment of X^2] -> float64 [T, 2]."""
    X = np.asarray(X, dtype=np.float64)
    Iq = num_heads * head_dim
    Ik = num_kv_heads * head_dim
    out = np.zeros((X.shape[0], 2), np.float64)
    out[:, 0] = np.sum(X[:, :Iq] ** 2, axis=1)
    if Ik:
        out[:, 1] = np.sum(X[:, Iq:Iq + Ik] ** 2, axis=1)
    return out


def project(a_codes, a_scale, w_codes, w_e8m0, w_channel_scale=None, bias_bf16=None, *,
            num_heads: int, num_kv_heads: int, head_dim: int, w_dense=None, a_e8m0=None):
    """Returns (X float64 [T, I] before rounding, ssq float64 [T, 2]).

    a_codes uint8 [T, H]; a_scale fp32 [T]; w_codes uint8 [H // 4, I, 4]; w_e8m0 uint8
    [H // 32, I]; w_channel_scale fp32 [I] or None; bias_bf16 uint16 [I] or None.
    ``w_dense`` may pass a pre-decoded float64 W [H, I] (same values as decoding the codes)
    so that repeated calls on row samples do not decode the weight again.
    MX block-32 activations: pass ``a_e8m0`` uint8 [T, H // 32] and ``a_scale=None``; the
    activation is then dec(A[s, h]) * 2^(Ea[s, h // 32] - 127) and there is no row scale.
    """
    if a_e8m0 is not None:
        if a_scale is not None:
            raise ValueError("MX block-32 activations carry no row scale")
        A = mx_block_decode(a_codes, a_e8m0)                          # [T, H]
        a_scale = np.ones(A.shape[0], np.float32)
    else:
        A = e4m3_decode(a_codes)                                      # [T, H]
    W = mx_weight_decode(w_codes, w_e8m0) if w_dense is None else w_dense
    T, H = A.shape
    I = W.shape[1]
    if I != (num_heads + 2 * num_kv_heads) * head_dim:
        raise ValueError("I != (num_heads + 2 * num_kv_heads) * head_dim")
    if W.shape[0] != H:
        raise ValueError("contraction mismatch")
    sA = np.asarray(a_scale, dtype=np.float32).astype(np.float64)
    c = (np.ones(I) if w_channel_scale is None
         else np.asarray(w_channel_scale, dtype=np.float32).astype(np.float64))
    acc = A @ W                                                       # fp64 contraction
    X = acc * sA[:, None] * c[None, :]
    if bias_bf16 is not None:
        X = X + bf16_to_f64(bias_bf16)[None, :]
    return X, segment_ssq(X, num_heads, num_kv_heads, head_dim)


def abs_term_sum(a_codes, a_scale, w_codes, w_e8m0, w_channel_scale=None, *, a_e8m0=None):
    """Per output, the sum of the absolute values of the contraction's terms, float64 [T, I]:
    |sA[s] * c[i]| * sum_h |dec(A[s, h]) * dec(W[h, i]) * 2^(E[h // 32, i] - 127)| (with MX
    activations the per-block factor inside the sum, as in ``project``).

    This is the scale against which a summation error is measured: any summation of the terms
    whose every addition is exact to a relative error e lies within about (depth) * e times this
    value of the exact sum; an accumulator that rounds each partial sum relative to its inputs'
    magnitudes is bounded by a multiple of it even where the terms cancel."""
    if a_e8m0 is not None:
        A = np.abs(mx_block_decode(a_codes, a_e8m0))
        sA = np.ones(A.shape[0])
    else:
        A = np.abs(e4m3_decode(a_codes))
        sA = np.abs(np.asarray(a_scale, dtype=np.float32).astype(np.float64))
    W = np.abs(mx_weight_decode(w_codes, w_e8m0))
    c = (np.ones(W.shape[1]) if w_channel_scale is None
         else np.abs(np.asarray(w_channel_scale, dtype=np.float32).astype(np.float64)))
    return (A @ W) * sA[:, None] * c[None, :]
