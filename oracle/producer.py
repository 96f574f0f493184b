"""Producer: residual add + RMSNorm + ROW_MX quantisation of bf16 hidden states
(oracle; test infrastructure only).

[RMSNORM-MX] ``residual``: when given it is added to ``hidden_states`` before the norm and the
pre-norm sum is written out for the next layer's residual stream.  ``eps`` (default 1e-6).
``unpadded_hidden_size``: the sum of squares runs over the full (zero-padded) H, the mean divides
by the unpadded size.  ``emit_norm_bf16``: the normed value is (hidden [+ residual]) * inv_rms *
gamma computed in fp32.  [QKV-CTE] "Interface", ``packed_hidden``: the consumer expects ROW_MX
rows (H FP8 codes + an fp32 scale), so the MX quantisation step emits that layout here.

Steps, in the order taken (the readings are listed in the design doc):
  1. r   = bf16_RNE(fp32(hid) + fp32(res))          (written out; r = hid without residual)
  2. ss  = sum_h r_h^2                               (float64)
  3. inv = fp32( 1 / sqrt(ss / H_u + eps) )          (float64 sqrt and divide, one fp32 rounding)
  4. y_h = fl32( fl32(r_h * inv) * gamma_h )
  5. ROW_MX encode of y (see rowmx.py), or the MX block-32 encode (see mxact.py); with
     ``emit_norm_bf16`` y is also stored as bf16
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_round_f32, bf16_to_f64
from .mxact import mx_block_quantize
from .rowmx import rowmx_quantize


def rmsnorm_rowmx(hid_bf16, res_bf16, gamma_bf16, eps: float, unpadded_h: int = 0):
    """Returns (res_out bf16 bits [T, H] or None, packed uint8 [T, H + 4], y fp32 [T, H])."""
    res_out, y = _normed(hid_bf16, res_bf16, gamma_bf16, eps, unpadded_h)
    return res_out, rowmx_quantize(y), y


def rmsnorm_mx(hid_bf16, res_bf16, gamma_bf16, eps: float, unpadded_h: int = 0):
    """Steps 1-4, then the MX block-32 encoding of y ([RMSNORM-MX] ``qmx_output_dtype``; see
    mxact.py) and ``emit_norm_bf16``: the fp32 normed value y cast to bf16 (round to nearest
    even) on store.  Returns (res_out bf16 bits or None, codes uint8 [T, H], e8m0 uint8
    [T, H // 32], norm bf16 bits [T, H], y fp32 [T, H])."""
    res_out, y = _normed(hid_bf16, res_bf16, gamma_bf16, eps, unpadded_h)
    codes, e8 = mx_block_quantize(y)
    return res_out, codes, e8, bf16_round_f32(y), y


def _normed(hid_bf16, res_bf16, gamma_bf16, eps: float, unpadded_h: int = 0):
    """Steps 1-4 above: (res_out bf16 bits [T, H] or None, y fp32 [T, H])."""
    hid = bf16_to_f64(hid_bf16).astype(np.float32)                  # exact widening
    T, H = hid.shape
    Hu = H if not unpadded_h else int(unpadded_h)
    if Hu <= 0 or Hu > H:
        raise ValueError("unpadded size must be in (0, H]")
    if res_bf16 is not None:
        res = bf16_to_f64(res_bf16).astype(np.float32)
        s32 = (hid + res).astype(np.float32)                          # one fp32 rounding
        res_out = bf16_round_f32(s32)
        r = bf16_to_f64(res_out)                                      # the stored sum
    else:
        res_out = None
        r = hid.astype(np.float64)
    ss = np.sum(r * r, axis=1)                                        # float64
    e = float(np.float32(eps))
    inv = (1.0 / np.sqrt(ss / float(Hu) + e)).astype(np.float32)
    g = bf16_to_f64(gamma_bf16).astype(np.float32)
    y = ((r.astype(np.float32) * inv[:, None]).astype(np.float32) * g[None, :]).astype(np.float32)
    return res_out, y
