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
    "qkv_rowmx_project_staged_noalloc", "noalloc_scratch_bytes", "e4m3_convert_check",
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


# The C ABI receives raw pointers and cannot see a buffer's extent, so every wrapper checks the
# dtype and size of each tensor against the call's dimensions before calling the library: a
# mis-sized or mis-typed tensor raises QkvmxError and launches nothing.

def _dt(name: str):
    import torch
    return {"u8": torch.uint8, "f32": torch.float32, "bf16": torch.bfloat16,
            "i32": torch.int32, "i64": torch.int64}[name]


def _need(t, what: str, dtypes, numel=None, min_bytes=None, optional=False):
    """Checks tensor ``t`` (None allowed when ``optional``): dtype in ``dtypes`` (names as in
    _dt; None accepts any), exactly ``numel`` elements and / or at least ``min_bytes`` bytes."""
    if t is None:
        if optional:
            return
        raise QkvmxError(f"{what} is required")
    if dtypes is not None:
        allowed = [_dt(d) for d in ((dtypes,) if isinstance(dtypes, str) else dtypes)]
        if t.dtype not in allowed:
            raise QkvmxError(f"{what}: dtype {t.dtype}, expected "
                             f"{' or '.join(str(a) for a in allowed)}")
    if numel is not None and t.numel() != numel:
        raise QkvmxError(f"{what}: {t.numel()} elements ({tuple(t.shape)}), expected {numel}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise QkvmxError(f"{what}: {t.numel() * t.element_size()} bytes, needs at least "
                         f"{min_bytes}")


def _rows2d(t, what: str, dtypes):
    """Shape (T, H) of a 2-D row tensor, after checking its rank and dtype."""
    _need(t, what, dtypes)
    if t.dim() != 2:
        raise QkvmxError(f"{what}: expected a 2-D [T, H] tensor, got shape {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


def _width(num_heads: int, num_kv_heads: int, head_dim: int) -> int:
    return (int(num_heads) + 2 * int(num_kv_heads)) * int(head_dim)


def _check_projection_io(what, T, H, I, w_packed, channel_scale, bias, out, ssq):
    """The tensors every projection entry point shares (T, H, I already known)."""
    _need(w_packed, f"{what}: w_packed", None, min_bytes=qkv_weight_packed_bytes(H, I))
    _need(channel_scale, f"{what}: channel_scale", "f32", numel=I, optional=True)
    _need(bias, f"{what}: bias", "bf16", numel=I, optional=True)
    _need(out, f"{what}: out", "bf16", numel=T * I)
    _need(ssq, f"{what}: ssq", "f32", numel=T * 2, optional=True)


def _check_head_params(what, T, d, q_gamma, k_gamma, q_beta, k_beta, cos, sin):
    for t, n in ((q_gamma, "q_gamma"), (k_gamma, "k_gamma"), (q_beta, "q_beta"),
                 (k_beta, "k_beta")):
        _need(t, f"{what}: {n}", "bf16", numel=d, optional=True)
    for t, n in ((cos, "cos"), (sin, "sin")):
        _need(t, f"{what}: {n}", "f32", numel=T * d, optional=True)


def _producer_common(what, hidden, gamma, residual, residual_out):
    """Checks the producers' shared tensors; returns (T, H)."""
    T, H = _rows2d(hidden, f"{what}: hidden", "bf16")
    _need(gamma, f"{what}: gamma", "bf16", numel=H)
    _need(residual, f"{what}: residual", "bf16", numel=T * H, optional=True)
    _need(residual_out, f"{what}: residual_out", "bf16", numel=T * H, optional=True)
    return T, H


def mx_weight_quantize(w, codes_out, e8m0_out, stream=None):
    """fp32 W [H, I] -> codes [H // 4, I, 4] uint8 and E8M0 exponents [H // 32, I] uint8."""
    H, I = _rows2d(w, "mx_weight_quantize: w", "f32")
    _need(codes_out, "mx_weight_quantize: codes_out", "u8", numel=H * I)
    _need(e8m0_out, "mx_weight_quantize: e8m0_out", "u8", numel=(H // 32) * I)
    _check(lib().mx_weight_quantize(_ptr(w), H, I, _ptr(codes_out), _ptr(e8m0_out),
                                    _stream(stream)), "mx_weight_quantize")


def qkv_weight_packed_bytes(H: int, I: int) -> int:
    return int(lib().qkv_weight_packed_bytes(H, I))


def qkv_weight_prepack(codes, e8m0, H: int, I: int, packed_out, stream=None):
    _need(codes, "qkv_weight_prepack: codes", "u8", numel=H * I)
    _need(e8m0, "qkv_weight_prepack: e8m0", "u8", numel=(H // 32) * I)
    _need(packed_out, "qkv_weight_prepack: packed_out", None)
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
    T, H = _rows2d(x, "row_quantize_packed: x", ("f32", "bf16"))
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _need(packed_out, "row_quantize_packed: packed_out", "u8", numel=T * (H + 4))
    _check(lib().row_quantize_packed(_ptr(x), dt, T, H, _ptr(packed_out), _stream(stream)),
           "row_quantize_packed")


def rmsnorm_mx_quantize(hidden, gamma, eps: float, packed_out, residual=None, residual_out=None,
                        unpadded_h: int = 0, stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out (bf16) and packed ROW_MX rows."""
    T, H = _producer_common("rmsnorm_mx_quantize", hidden, gamma, residual, residual_out)
    _need(packed_out, "rmsnorm_mx_quantize: packed_out", "u8", numel=T * (H + 4))
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
    T, H = _rows2d(x, "row_quantize_staged: x", ("f32", "bf16"))
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _need(act_image, "row_quantize_staged: act_image", None)
    _need(row_scale, "row_quantize_staged: row_scale", "f32", numel=T)
    _check(lib().row_quantize_staged(_ptr(x), dt, T, H, _ptr(act_image), _nbytes(act_image),
                                     _ptr(row_scale), _stream(stream)), "row_quantize_staged")


def rmsnorm_mx_quantize_staged(hidden, gamma, eps: float, act_image, row_scale, residual=None,
                               residual_out=None, unpadded_h: int = 0, stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out (bf16), ROW_MX codes in the staged image
    layout and fp32 row scales [T]."""
    T, H = _producer_common("rmsnorm_mx_quantize_staged", hidden, gamma, residual, residual_out)
    _need(act_image, "rmsnorm_mx_quantize_staged: act_image", None)
    _need(row_scale, "rmsnorm_mx_quantize_staged: row_scale", "f32", numel=T)
    _check(lib().rmsnorm_mx_quantize_staged(_ptr(hidden), _ptr(residual), _ptr(gamma), float(eps),
                                            T, H, unpadded_h, _ptr(residual_out), _ptr(act_image),
                                            _nbytes(act_image), _ptr(row_scale), _stream(stream)),
           "rmsnorm_mx_quantize_staged")


def mx_block_quantize(x, codes_out, e8m0_out, stream=None):
    """x [T, H] fp32 or bf16 -> MX block-32 codes [T, H] uint8 and E8M0 exponents [T, H // 32]."""
    import torch
    T, H = _rows2d(x, "mx_block_quantize: x", ("f32", "bf16"))
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _need(codes_out, "mx_block_quantize: codes_out", "u8", numel=T * H)
    _need(e8m0_out, "mx_block_quantize: e8m0_out", "u8", numel=T * (H // 32))
    _check(lib().mx_block_quantize(_ptr(x), dt, T, H, _ptr(codes_out), _ptr(e8m0_out),
                                   _stream(stream)), "mx_block_quantize")


def rmsnorm_mx_block_quantize(hidden, gamma, eps: float, codes_out, e8m0_out, residual=None,
                              residual_out=None, norm_out=None, unpadded_h: int = 0,
                              stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out, MX block-32 codes / exponents and
    (norm_out) the bf16 normed rows."""
    T, H = _producer_common("rmsnorm_mx_block_quantize", hidden, gamma, residual, residual_out)
    _need(codes_out, "rmsnorm_mx_block_quantize: codes_out", "u8", numel=T * H)
    _need(e8m0_out, "rmsnorm_mx_block_quantize: e8m0_out", "u8", numel=T * (H // 32))
    _need(norm_out, "rmsnorm_mx_block_quantize: norm_out", "bf16", numel=T * H, optional=True)
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
    T, H = _rows2d(x, "mx_block_quantize_staged: x", ("f32", "bf16"))
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _need(act_image, "mx_block_quantize_staged: act_image", None)
    _need(exp_image, "mx_block_quantize_staged: exp_image", None)
    _check(lib().mx_block_quantize_staged(_ptr(x), dt, T, H, _ptr(act_image), _nbytes(act_image),
                                          _ptr(exp_image), _nbytes(exp_image), _stream(stream)),
           "mx_block_quantize_staged")


def rmsnorm_mx_block_quantize_staged(hidden, gamma, eps: float, act_image, exp_image,
                                     residual=None, residual_out=None, norm_out=None,
                                     unpadded_h: int = 0, stream=None):
    """bf16 hidden [T, H] (+ residual) -> residual_out, staged MX block-32 codes and exponents,
    and (norm_out) the bf16 normed rows."""
    T, H = _producer_common("rmsnorm_mx_block_quantize_staged", hidden, gamma, residual,
                            residual_out)
    _need(act_image, "rmsnorm_mx_block_quantize_staged: act_image", None)
    _need(exp_image, "rmsnorm_mx_block_quantize_staged: exp_image", None)
    _need(norm_out, "rmsnorm_mx_block_quantize_staged: norm_out", "bf16", numel=T * H,
          optional=True)
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
    I = _width(num_heads, num_kv_heads, head_dim)
    _need(act_image, "qkv_mx_project_staged: act_image", None)
    _need(exp_image, "qkv_mx_project_staged: exp_image", None)
    _check_projection_io("qkv_mx_project_staged", T, H, I, w_packed, channel_scale, bias, out, ssq)
    _need(workspace, "qkv_mx_project_staged: workspace", None, optional=True)
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
    T, cstride = _rows2d(a_codes, "qkv_mx_project: a_codes", "u8")
    Te, estride = _rows2d(a_e8m0, "qkv_mx_project: a_e8m0", "u8")
    if Te != T or cstride < H or estride < H // 32:
        raise QkvmxError(f"qkv_mx_project: codes {tuple(a_codes.shape)} and exponents "
                         f"{tuple(a_e8m0.shape)} do not cover [{T}, {H}] / [{T}, {H // 32}]")
    I = _width(num_heads, num_kv_heads, head_dim)
    _check_projection_io("qkv_mx_project", T, H, I, w_packed, channel_scale, bias, out, ssq)
    _need(workspace, "qkv_mx_project: workspace", None, optional=True)
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
    T, width = _rows2d(packed_a, "qkv_rowmx_project: packed_a", "u8")
    rs = width if a_row_stride is None else int(a_row_stride)
    a_bytes = packed_a.numel()
    if a_scales is None:
        ss = rs if a_scale_stride is None else int(a_scale_stride)
        # codes of row t at t * rs, its scale at H + t * ss, both inside packed_a
        need_scales = H + (T - 1) * ss + 4
        if need_scales > a_bytes:
            raise QkvmxError(f"qkv_rowmx_project: the scale tail of row {T - 1} ends at byte "
                             f"{need_scales}, beyond packed_a's {a_bytes} bytes (rows must be "
                             f"[T, H + 4] when no a_scales tensor is given)")
    else:
        _need(a_scales, "qkv_rowmx_project: a_scales", ("f32", "u8"))
        ss = 4 if a_scale_stride is None else int(a_scale_stride)
        need = (T - 1) * ss + 4
        if need > a_scales.numel() * a_scales.element_size():
            raise QkvmxError(f"qkv_rowmx_project: a_scales holds "
                             f"{a_scales.numel() * a_scales.element_size()} bytes, {need} needed")
    if (T - 1) * rs + H > a_bytes:
        raise QkvmxError(f"qkv_rowmx_project: codes of row {T - 1} end at byte "
                         f"{(T - 1) * rs + H}, beyond packed_a's {a_bytes} bytes")
    I = _width(num_heads, num_kv_heads, head_dim)
    _check_projection_io("qkv_rowmx_project", T, H, I, w_packed, channel_scale, bias, out, ssq)
    _need(workspace, "qkv_rowmx_project: workspace", None, optional=True)
    a_ptr = _ptr(packed_a)
    s_ptr = a_ptr + H if a_scales is None else _ptr(a_scales)
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
    _need(row_scale, "qkv_rowmx_project_staged: row_scale", "f32")
    T = row_scale.numel()
    I = _width(num_heads, num_kv_heads, head_dim)
    _need(act_image, "qkv_rowmx_project_staged: act_image", None)
    _check_projection_io("qkv_rowmx_project_staged", T, H, I, w_packed, channel_scale, bias, out,
                         ssq)
    _need(workspace, "qkv_rowmx_project_staged: workspace", None, optional=True)
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace), _nbytes(workspace))
    _check(lib().qkv_rowmx_project_staged(_ptr(act_image), _nbytes(act_image), _ptr(row_scale),
                                          _ptr(w_packed), _ptr(channel_scale), _ptr(bias), T, H,
                                          num_heads, num_kv_heads, head_dim, layout, _ptr(out),
                                          _ptr(ssq), ws_ptr, ws_n, _stream(stream)),
           "qkv_rowmx_project_staged")


def noalloc_scratch_bytes() -> int:
    """Bytes of the static device scratch behind qkv_rowmx_project_staged_noalloc."""
    return int(lib().qkvmx_noalloc_scratch_bytes())


def qkv_rowmx_project_staged_noalloc(act_image, row_scale, w_packed, out, *, H: int,
                                     num_heads: int, num_kv_heads: int, head_dim: int,
                                     channel_scale=None, bias=None, ssq=None,
                                     layout: int = LAYOUT_BSD, stream=None):
    """qkv_rowmx_project_staged without a workspace: the library's static per-GPU scratch
    holds the projection's scratch, so the call allocates nothing.  Calls that overlap on one
    GPU race on that scratch."""
    _need(row_scale, "qkv_rowmx_project_staged_noalloc: row_scale", "f32")
    T = row_scale.numel()
    I = _width(num_heads, num_kv_heads, head_dim)
    _need(act_image, "qkv_rowmx_project_staged_noalloc: act_image", None)
    _check_projection_io("qkv_rowmx_project_staged_noalloc", T, H, I, w_packed, channel_scale,
                         bias, out, ssq)
    _check(lib().qkv_rowmx_project_staged_noalloc(
        _ptr(act_image), _nbytes(act_image), _ptr(row_scale), _ptr(w_packed), _ptr(channel_scale),
        _ptr(bias), T, H, num_heads, num_kv_heads, head_dim, layout, _ptr(out), _ptr(ssq),
        _stream(stream)), "qkv_rowmx_project_staged_noalloc")


def qkv_rowmx_project_headnorm(packed_a, w_packed, out, *, H: int, num_heads: int,
                               num_kv_heads: int, head_dim: int, norm_kind: int, q_gamma,
                               k_gamma=None, q_beta=None, k_beta=None, eps: float = 1e-6,
                               cos=None, sin=None, bias=None, workspace=None,
                               layout: int = LAYOUT_BSD, stream=None):
    """Pass 1 on packed ROW_MX rows [T, H + 4] with the per-head qk-norm (HEAD_RMS_NORM or
    HEAD_LAYER_NORM, gamma / beta [head_dim]) and optional rotate-half RoPE fused into the
    epilogue."""
    T, rs = _rows2d(packed_a, "qkv_rowmx_project_headnorm: packed_a", "u8")
    if rs < H + 4:
        raise QkvmxError(f"qkv_rowmx_project_headnorm: packed_a rows are {rs} bytes, H + 4 = "
                         f"{H + 4} needed (codes and the fp32 scale tail)")
    I = _width(num_heads, num_kv_heads, head_dim)
    _check_projection_io("qkv_rowmx_project_headnorm", T, H, I, w_packed, None, bias, out, None)
    _check_head_params("qkv_rowmx_project_headnorm", T, head_dim, q_gamma, k_gamma, q_beta,
                       k_beta, cos, sin)
    _need(workspace, "qkv_rowmx_project_headnorm: workspace", None, optional=True)
    a_ptr = _ptr(packed_a)
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
    _need(row_scale, "qkv_rowmx_project_headnorm_staged: row_scale", "f32")
    T = row_scale.numel()
    I = _width(num_heads, num_kv_heads, head_dim)
    _need(act_image, "qkv_rowmx_project_headnorm_staged: act_image", None)
    _check_projection_io("qkv_rowmx_project_headnorm_staged", T, H, I, w_packed, None, bias, out,
                         None)
    _check_head_params("qkv_rowmx_project_headnorm_staged", T, head_dim, q_gamma, k_gamma,
                       q_beta, k_beta, cos, sin)
    _need(workspace, "qkv_rowmx_project_headnorm_staged: workspace", None, optional=True)
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
    _need(qkv, "qk_norm_rope_apply: qkv", "bf16")
    I = _width(num_heads, num_kv_heads, head_dim)
    if qkv.dim() != (3 if layout == LAYOUT_NBSD else 2):
        raise QkvmxError(f"qk_norm_rope_apply: qkv of shape {tuple(qkv.shape)} is not "
                         f"{'[I / d, T, d]' if layout == LAYOUT_NBSD else '[T, I]'}")
    T = int(qkv.shape[1] if layout == LAYOUT_NBSD else qkv.shape[0])
    _need(qkv, "qk_norm_rope_apply: qkv", "bf16", numel=T * I)
    _need(ssq, "qk_norm_rope_apply: ssq", "f32", numel=T * 2, optional=True)
    _need(q_gamma, "qk_norm_rope_apply: q_gamma", "bf16", numel=num_heads * head_dim,
          optional=True)
    _need(k_gamma, "qk_norm_rope_apply: k_gamma", "bf16", numel=num_kv_heads * head_dim,
          optional=True)
    for t, n in ((cos, "cos"), (sin, "sin")):
        _need(t, f"qk_norm_rope_apply: {n}", "f32", numel=T * head_dim, optional=True)
    _check(lib().qk_norm_rope_apply(_ptr(qkv), _ptr(ssq), _ptr(q_gamma), _ptr(k_gamma), _ptr(cos),
                                    _ptr(sin), T, num_heads, num_kv_heads, head_dim, float(eps),
                                    flags, layout, _stream(stream)), "qk_norm_rope_apply")


def mfma_rate_probe(blocks: int, iters: int, random_operands: bool, sink, clocks, stream=None):
    """Roofline calibration: launches the MFMA issue-rate probe (see include/qkvmx.h);
    ``sink`` fp32 [blocks * 256], ``clocks`` int64 [blocks, 2] (cycles, 100 MHz ticks)."""
    _need(sink, "mfma_rate_probe: sink", "f32", numel=blocks * 256)
    _need(clocks, "mfma_rate_probe: clocks", "i64", numel=blocks * 2)
    _check(lib().qkvmx_mfma_rate_probe(blocks, iters, int(bool(random_operands)), _ptr(sink),
                                       _ptr(clocks), _stream(stream)), "qkvmx_mfma_rate_probe")


def e4m3_convert_check(counts, first_bad=None, stream=None):
    """The producers' hardware E4M3 conversion against the software encoder on every finite
    fp32 value (include/qkvmx.h); ``counts`` int64 [3] zeroed, ``first_bad`` int32 [8] or None."""
    _need(counts, "e4m3_convert_check: counts", "i64", numel=3)
    _need(first_bad, "e4m3_convert_check: first_bad", "i32", numel=8, optional=True)
    _check(lib().qkvmx_e4m3_convert_check(_ptr(counts), _ptr(first_bad), _stream(stream)),
           "qkvmx_e4m3_convert_check")
