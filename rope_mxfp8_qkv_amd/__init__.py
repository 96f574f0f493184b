"""MI355X-native fused MXFP8 QKV projection, across-heads QK RMSNorm and rotate-half RoPE.

Thin Python binding over the C ABI in ``include/qkvmx.h`` (``libqkvmx.so``, built in-tree by
``rope_mxfp8_qkv_amd.build``).  The functions below only marshal arguments: they take torch
device tensors (torch is used for device memory and streams), pass raw pointers and the current
HIP stream to the library, and raise ``QkvmxError`` on a non-OK status.  Every computation runs
in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from . import _abi
from ._abi import (NORM_Q, NORM_K, FUSED_ROPE, LAYOUT_BSD, LAYOUT_NBSD, DTYPE_F32, DTYPE_BF16,
                   HEAD_RMS_NORM, HEAD_LAYER_NORM, QkvmxError, lib, lib_path)

__all__ = [
    "NORM_Q", "NORM_K", "FUSED_ROPE", "LAYOUT_BSD", "LAYOUT_NBSD", "DTYPE_F32", "DTYPE_BF16", "QkvmxError",
    "lib", "lib_path", "mx_weight_quantize", "qkv_weight_packed_bytes", "qkv_weight_prepack",
    "row_quantize_packed", "rmsnorm_mx_quantize", "qkvmx_workspace_bytes", "qkv_rowmx_project",
    "qk_norm_rope_apply", "prepare_weight", "mx_block_quantize", "rmsnorm_mx_block_quantize",
    "qkv_mx_workspace_bytes", "qkv_mx_project", "qkv_rowmx_project_headnorm", "HEAD_RMS_NORM",
    "HEAD_LAYER_NORM", "qkv_act_image_bytes", "row_quantize_staged", "rmsnorm_mx_quantize_staged",
    "qkv_staged_workspace_bytes", "qkv_rowmx_project_staged", "mfma_rate_probe",
    "qkv_act_exp_image_bytes", "mx_block_quantize_staged", "rmsnorm_mx_block_quantize_staged",
    "qkv_mx_project_staged", "projection_k_chunks", "qkv_rowmx_project_headnorm_staged",
]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise QkvmxError(f"expected a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise QkvmxError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, name: str):
    if status != 0:
        raise QkvmxError(f"{name}: {_abi.status_string(status)}: {_abi.last_error()}", status)


def mx_weight_quantize(w, codes_out, e8m0_out, stream=None):
    """fp32 W [H, I] -> codes [H // 4, I, 4] uint8 and E8M0 exponents [H // 32, I] uint8."""
    H, I = w.shape
    _check(lib().mx_weight_quantize(_ptr(w), H, I, _ptr(codes_out), _ptr(e8m0_out),
                                    _stream(stream)), "mx_weight_quantize")


def qkv_weight_packed_bytes(H: int, I: int) -> int:
    return int(lib().qkv_weight_packed_bytes(H, I))


def qkv_weight_prepack(codes, e8m0, H: int, I: int, packed_out, stream=None):
    _check(lib().qkv_weight_prepack(_ptr(codes), _ptr(e8m0), H, I, _ptr(packed_out),
                                    packed_out.numel() * packed_out.element_size(),
                                    _stream(stream)), "qkv_weight_prepack")


def prepare_weight(codes, e8m0, H: int, I: int, stream=None):
    """Allocates (torch) and fills the packed weight for an [H, I] projection."""
    import torch
    n = qkv_weight_packed_bytes(H, I)
    packed = torch.empty(n, dtype=torch.uint8, device=codes.device)
    qkv_weight_prepack(codes, e8m0, H, I, packed, stream)
    return packed


def row_quantize_packed(x, packed_out, stream=None):
    """x [T, H] fp32 or bf16 -> packed ROW_MX rows [T, H + 4] uint8."""
    import torch
    T, H = x.shape
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise QkvmxError("row_quantize_packed takes fp32 or bf16 rows")
    _check(lib().row_quantize_packed(_ptr(x), dt, T, H, _ptr(packed_out), _stream(stream)),
           "row_quantize_packed")


def rmsnorm_mx_quantize(hidden, gamma, eps: float, packed_out, residual=None, residual_out=None,
                        unpadded_h: int = 0, stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out (bf16) and packed ROW_MX rows."""
    T, H = hidden.shape
    _check(lib().rmsnorm_mx_quantize(_ptr(hidden), _ptr(residual), _ptr(gamma), float(eps), T, H,
                                     unpadded_h, _ptr(residual_out), _ptr(packed_out),
                                     _stream(stream)), "rmsnorm_mx_quantize")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def qkv_act_image_bytes(T: int, H: int) -> int:
    """Bytes of the staged activation image of T rows of H codes."""
    return int(lib().qkv_act_image_bytes(T, H))


def row_quantize_staged(x, act_image, row_scale, stream=None):
    """x [T, H] fp32 or bf16 -> ROW_MX codes in the staged image layout (uint8, at least
    qkv_act_image_bytes(T, H) bytes) and fp32 row scales [T]."""
    import torch
    T, H = x.shape
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise QkvmxError("row_quantize_staged takes fp32 or bf16 rows")
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _check(lib().row_quantize_staged(_ptr(x), dt, T, H, _ptr(act_image), _nbytes(act_image),
                                     _ptr(row_scale), _stream(stream)), "row_quantize_staged")


def rmsnorm_mx_quantize_staged(hidden, gamma, eps: float, act_image, row_scale, residual=None,
                               residual_out=None, unpadded_h: int = 0, stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out (bf16), ROW_MX codes in the staged image
    layout and fp32 row scales [T]."""
    T, H = hidden.shape
    _check(lib().rmsnorm_mx_quantize_staged(_ptr(hidden), _ptr(residual), _ptr(gamma), float(eps),
                                            T, H, unpadded_h, _ptr(residual_out), _ptr(act_image),
                                            _nbytes(act_image), _ptr(row_scale), _stream(stream)),
           "rmsnorm_mx_quantize_staged")


def mx_block_quantize(x, codes_out, e8m0_out, stream=None):
    """x [T, H] fp32 or bf16 -> MX block-32 codes [T, H] uint8 and E8M0 exponents [T, H // 32]."""
    import torch
    T, H = x.shape
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise QkvmxError("mx_block_quantize takes fp32 or bf16 rows")
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _check(lib().mx_block_quantize(_ptr(x), dt, T, H, _ptr(codes_out), _ptr(e8m0_out),
                                   _stream(stream)), "mx_block_quantize")


def rmsnorm_mx_block_quantize(hidden, gamma, eps: float, codes_out, e8m0_out, residual=None,
                              residual_out=None, norm_out=None, unpadded_h: int = 0,
                              stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out, MX block-32 codes / exponents and
    (norm_out) the bf16 normed rows."""
    T, H = hidden.shape
    _check(lib().rmsnorm_mx_block_quantize(_ptr(hidden), _ptr(residual), _ptr(gamma), float(eps),
                                           T, H, unpadded_h, _ptr(residual_out), _ptr(codes_out),
                                           _ptr(e8m0_out), _ptr(norm_out), _stream(stream)),
           "rmsnorm_mx_block_quantize")


def qkv_act_exp_image_bytes(T: int, H: int) -> int:
    """Bytes of the staged MX exponent image of T rows of H elements."""
    return int(lib().qkv_act_exp_image_bytes(T, H))


def mx_block_quantize_staged(x, act_image, exp_image, stream=None):
    """x [T, H] fp32 or bf16 -> MX block-32 codes in the staged image layout and exponents in
    the staged exponent image (uint8 / int32 tensors of at least qkv_act_image_bytes and
    qkv_act_exp_image_bytes bytes)."""
    import torch
    T, H = x.shape
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise QkvmxError("mx_block_quantize_staged takes fp32 or bf16 rows")
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _check(lib().mx_block_quantize_staged(_ptr(x), dt, T, H, _ptr(act_image), _nbytes(act_image),
                                          _ptr(exp_image), _nbytes(exp_image), _stream(stream)),
           "mx_block_quantize_staged")


def rmsnorm_mx_block_quantize_staged(hidden, gamma, eps: float, act_image, exp_image,
                                     residual=None, residual_out=None, norm_out=None,
                                     unpadded_h: int = 0, stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out, staged MX block-32 codes and exponents,
    and (norm_out) the bf16 normed rows."""
    T, H = hidden.shape
    _check(lib().rmsnorm_mx_block_quantize_staged(_ptr(hidden), _ptr(residual), _ptr(gamma),
                                                  float(eps), T, H, unpadded_h,
                                                  _ptr(residual_out), _ptr(act_image),
                                                  _nbytes(act_image), _ptr(exp_image),
                                                  _nbytes(exp_image), _ptr(norm_out),
                                                  _stream(stream)),
           "rmsnorm_mx_block_quantize_staged")


def qkv_mx_project_staged(act_image, exp_image, w_packed, out, *, T: int, H: int,
                          num_heads: int, num_kv_heads: int, head_dim: int, channel_scale=None,
                          bias=None, ssq=None, workspace=None, layout: int = LAYOUT_BSD,
                          stream=None):
    """Pass 1 on staged MX block-32 activations.  Output as qkv_mx_project."""
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace), _nbytes(workspace))
    _check(lib().qkv_mx_project_staged(_ptr(act_image), _nbytes(act_image), _ptr(exp_image),
                                       _nbytes(exp_image), _ptr(w_packed), _ptr(channel_scale),
                                       _ptr(bias), T, H, num_heads, num_kv_heads, head_dim,
                                       layout, _ptr(out), _ptr(ssq), ws_ptr, ws_n,
                                       _stream(stream)), "qkv_mx_project_staged")


def qkv_mx_workspace_bytes(T: int, H: int, I: int) -> int:
    return int(lib().qkv_mx_workspace_bytes(T, H, I))


def qkv_mx_project(a_codes, a_e8m0, w_packed, out, *, H: int, num_heads: int, num_kv_heads: int,
                   head_dim: int, channel_scale=None, bias=None, ssq=None, workspace=None,
                   layout: int = LAYOUT_BSD, stream=None):
    """Pass 1 on MX block-32 activations: codes [T, stride >= H] and exponents
    [T, stride >= H / 32] (row strides taken from the tensors' shapes)."""
    T = a_codes.shape[0]
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace),
                                                        workspace.numel() * workspace.element_size())
    _check(lib().qkv_mx_project(_ptr(a_codes), a_codes.shape[1], _ptr(a_e8m0), a_e8m0.shape[1],
                                _ptr(w_packed), _ptr(channel_scale), _ptr(bias), T, H, num_heads,
                                num_kv_heads, head_dim, layout, _ptr(out), _ptr(ssq), ws_ptr,
                                ws_n, _stream(stream)), "qkv_mx_project")


def qkvmx_workspace_bytes(T: int, H: int, I: int) -> int:
    return int(lib().qkvmx_workspace_bytes(T, H, I))


def qkv_rowmx_project(packed_a, w_packed, out, *, H: int, num_heads: int, num_kv_heads: int,
                      head_dim: int, channel_scale=None, bias=None, ssq=None, workspace=None,
                      a_scales=None, a_row_stride: Optional[int] = None,
                      a_scale_stride: Optional[int] = None, layout: int = LAYOUT_BSD,
                      stream=None):
    """Pass 1 on packed ROW_MX rows ``packed_a`` [T, H + 4] (or codes [T, stride] with a
    separate ``a_scales`` tensor).  ``out`` is bf16 [T, I] (LAYOUT_BSD) or [I / head_dim, T,
    head_dim] (LAYOUT_NBSD); ``ssq`` fp32 [T, 2] or None."""
    T = packed_a.shape[0]
    a_ptr = _ptr(packed_a)
    if a_scales is None:
        s_ptr = a_ptr + H
        rs = packed_a.shape[1] if a_row_stride is None else a_row_stride
        ss = rs if a_scale_stride is None else a_scale_stride
    else:
        s_ptr = _ptr(a_scales)
        rs = packed_a.shape[1] if a_row_stride is None else a_row_stride
        ss = 4 if a_scale_stride is None else a_scale_stride
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace),
                                                        workspace.numel() * workspace.element_size())
    _check(lib().qkv_rowmx_project(a_ptr, rs, s_ptr, ss, _ptr(w_packed), _ptr(channel_scale),
                                   _ptr(bias), T, H, num_heads, num_kv_heads, head_dim, layout,
                                   _ptr(out), _ptr(ssq), ws_ptr, ws_n, _stream(stream)),
           "qkv_rowmx_project")


def qkv_staged_workspace_bytes(T: int, I: int) -> int:
    return int(lib().qkv_staged_workspace_bytes(T, I))


def projection_k_chunks(T: int, H: int, I: int, layout: int = LAYOUT_BSD) -> int:
    """K chunks the projections split a [T, H] x [H, I] call into (1: no split)."""
    return int(lib().qkvmx_projection_k_chunks(T, H, I, layout))


def qkv_rowmx_project_staged(act_image, row_scale, w_packed, out, *, H: int, num_heads: int,
                             num_kv_heads: int, head_dim: int, channel_scale=None, bias=None,
                             ssq=None, workspace=None, layout: int = LAYOUT_BSD, stream=None):
    """Pass 1 on staged ROW_MX activations (``act_image`` from a staged producer, fp32
    ``row_scale`` [T]); T is taken from ``row_scale``.  Output as qkv_rowmx_project."""
    T = row_scale.shape[0]
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace), _nbytes(workspace))
    _check(lib().qkv_rowmx_project_staged(_ptr(act_image), _nbytes(act_image), _ptr(row_scale),
                                          _ptr(w_packed), _ptr(channel_scale), _ptr(bias), T, H,
                                          num_heads, num_kv_heads, head_dim, layout, _ptr(out),
                                          _ptr(ssq), ws_ptr, ws_n, _stream(stream)),
           "qkv_rowmx_project_staged")


def qkv_rowmx_project_headnorm(packed_a, w_packed, out, *, H: int, num_heads: int,
                               num_kv_heads: int, head_dim: int, norm_kind: int, q_gamma,
                               k_gamma=None, q_beta=None, k_beta=None, eps: float = 1e-6,
                               cos=None, sin=None, bias=None, workspace=None,
                               layout: int = LAYOUT_BSD, stream=None):
    """Pass 1 on packed ROW_MX rows [T, H + 4] with the per-head qk-norm (HEAD_RMS_NORM or
    HEAD_LAYER_NORM, gamma / beta [head_dim]) and optional rotate-half RoPE fused into the
    epilogue."""
    T = packed_a.shape[0]
    a_ptr = _ptr(packed_a)
    rs = packed_a.shape[1]
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace),
                                                        workspace.numel() * workspace.element_size())
    _check(lib().qkv_rowmx_project_headnorm(a_ptr, rs, a_ptr + H, rs, _ptr(w_packed), _ptr(bias),
                                            T, H, num_heads, num_kv_heads, head_dim, layout,
                                            norm_kind, _ptr(q_gamma), _ptr(k_gamma), _ptr(q_beta),
                                            _ptr(k_beta), float(eps), _ptr(cos), _ptr(sin),
                                            _ptr(out), ws_ptr, ws_n, _stream(stream)),
           "qkv_rowmx_project_headnorm")


def qkv_rowmx_project_headnorm_staged(act_image, row_scale, w_packed, out, *, H: int,
                                      num_heads: int, num_kv_heads: int, head_dim: int,
                                      norm_kind: int, q_gamma, k_gamma=None, q_beta=None,
                                      k_beta=None, eps: float = 1e-6, cos=None, sin=None,
                                      bias=None, workspace=None, layout: int = LAYOUT_BSD,
                                      stream=None):
    """qkv_rowmx_project_headnorm on staged ROW_MX activations (``act_image`` from a staged
    producer, fp32 ``row_scale`` [T]); T is taken from ``row_scale``."""
    T = row_scale.shape[0]
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace), _nbytes(workspace))
    _check(lib().qkv_rowmx_project_headnorm_staged(
        _ptr(act_image), _nbytes(act_image), _ptr(row_scale), _ptr(w_packed), _ptr(bias), T, H,
        num_heads, num_kv_heads, head_dim, layout, norm_kind, _ptr(q_gamma), _ptr(k_gamma),
        _ptr(q_beta), _ptr(k_beta), float(eps), _ptr(cos), _ptr(sin), _ptr(out), ws_ptr, ws_n,
        _stream(stream)), "qkv_rowmx_project_headnorm_staged")


def qk_norm_rope_apply(qkv, *, num_heads: int, num_kv_heads: int, head_dim: int, eps: float,
                       flags: int, ssq=None, q_gamma=None, k_gamma=None, cos=None, sin=None,
                       layout: int = LAYOUT_BSD, stream=None):
    """Pass 2, in place on ``qkv`` (bf16 [T, I], or [I / head_dim, T, head_dim] with
    LAYOUT_NBSD)."""
    T = qkv.shape[1] if layout == LAYOUT_NBSD else qkv.shape[0]
    _check(lib().qk_norm_rope_apply(_ptr(qkv), _ptr(ssq), _ptr(q_gamma), _ptr(k_gamma), _ptr(cos),
                                    _ptr(sin), T, num_heads, num_kv_heads, head_dim, float(eps),
                                    flags, layout, _stream(stream)), "qk_norm_rope_apply")


def mfma_rate_probe(blocks: int, iters: int, random_operands: bool, sink, clocks, stream=None):
    """Roofline calibration: launches the MFMA issue-rate probe (see include/qkvmx.h);
    ``sink`` fp32 [blocks * 256], ``clocks`` int64 [blocks, 2] (cycles, 100 MHz ticks)."""
    _check(lib().qkvmx_mfma_rate_probe(blocks, iters, int(bool(random_operands)), _ptr(sink),
                                       _ptr(clocks), _stream(stream)), "qkvmx_mfma_rate_probe")
