"""The C-ABI library: it loads, exports every function include/qkvmx.h declares with the
binding's signatures, and rejects bad arguments on the host before any HIP call (these status
paths run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkvmx.h")


def _lib():
    from rope_mxfp8_qkv_amd import _abi
    if not os.path.exists(_abi.lib_path()):
        pytest.fail("libqkvmx.so is not built (run `python -m rope_mxfp8_qkv_amd.build`)")
    return _abi.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_functions_exported_and_bound():
    from rope_mxfp8_qkv_amd import _abi
    L = _lib()
    names = _declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), n
        assert n in _abi.SIGNATURES, n
    assert set(_abi.SIGNATURES) == set(names)


def test_status_strings():
    from rope_mxfp8_qkv_amd import _abi
    _lib()
    assert _abi.status_string(0) == "QKVMX_OK"
    assert _abi.status_string(7) == "QKVMX_ERR_HIP"


def test_size_queries():
    L = _lib()
    assert L.qkv_weight_packed_bytes(5120, 15360) >= 5120 * 15360 + 15360 * 20 * 8
    assert L.qkv_weight_packed_bytes(100, 16) == 0           # H % 32 != 0
    # activation stage images (296 token tiles x 80 stages x 16 KiB) + 120 partials per token
    assert L.qkvmx_workspace_bytes(75600, 5120, 15360) == 296 * 80 * 16384 + 120 * 75600 * 8 + 256
    assert L.qkvmx_workspace_bytes(0, 256, 16) == 0
    assert L.qkvmx_workspace_bytes(4, 100, 16) == 0
    # staged activations: the image alone (whole 256-row tiles x KS stages x 16 KiB); the staged
    # projection's workspace holds only the partials and the counter block
    assert L.qkv_act_image_bytes(75600, 5120) == 296 * 80 * 16384
    assert L.qkv_act_image_bytes(300, 2080) == 2 * 36 * 16384
    assert L.qkv_act_image_bytes(4, 100) == 0
    assert L.qkv_staged_workspace_bytes(75600, 15360) == 120 * 75600 * 8 + 256
    # few tiles: + min(3, 256 // tiles) fp32 [T, I] planes of the split contraction
    # (512 x 5120: 2 x 20 = 40 tiles -> 3 planes; partials 40 x 512 x 8 bytes)
    assert L.qkv_staged_workspace_bytes(512, 5120) == 40 * 512 * 8 + 256 + 3 * 512 * 5120 * 4
    assert (L.qkvmx_workspace_bytes(512, 5120, 5120)
            == 2 * 80 * 16384 + 40 * 512 * 8 + 256 + 3 * 512 * 5120 * 4)


def test_split_contraction_plan():
    """K chunks per call: supersteps of 256 K-bytes cut into min(3, 256 // tiles) chunks of
    ceil(supersteps / that) supersteps, at most 128 tiles, either output layout."""
    L = _lib()
    f = L.qkvmx_projection_k_chunks
    assert f(512, 5120, 5120, 0) == 3          # 40 tiles -> 3-way, 20 supersteps -> 7, 7, 6
    assert f(512, 5120, 5120, 1) == 3          # NBSd: the same plan
    assert f(512, 1792, 5120, 0) == 3          # 7 supersteps -> 3, 3, 1
    assert f(300, 512, 640, 0) == 2            # 6 tiles -> 3-way, but 2 supersteps
    assert f(512, 512 * 3, 5120, 0) == 3       # 6 supersteps -> 2, 2, 2
    assert f(128, 256, 384, 0) == 1            # one superstep
    assert f(75600, 5120, 15360, 0) == 1       # 17760 tiles
    assert f(4096, 5120, 15360, 0) == 1        # 960 tiles
    assert f(1100, 512, 6528, 0) == 1          # 130 tiles
    assert f(32768, 5120, 256, 0) == 2         # 128 tiles -> 2-way
    assert f(0, 256, 384, 0) == 0 and f(4, 250, 384, 0) == 0 and f(4, 256, 384, 7) == 0
    assert L.qkv_staged_workspace_bytes(0, 16) == 0


P = 0x10000   # a fake, well-aligned device address: validation fails before it is used


@pytest.fixture(autouse=True)
def _no_gpu_launches():
    """These checks hand the library fake pointers and rely on validation failing first; where
    a GPU is present a check that unexpectedly passed validation would launch a kernel on them,
    so the module runs only on hosts without one."""
    try:
        import torch
        if torch.cuda.device_count() > 0:
            pytest.skip("fake-pointer validation checks run on GPU-less hosts only")
    except ImportError:
        pass
    yield


def _proj(L, **kw):
    a = dict(a_codes=P, a_row_stride=260, a_scales=P + 256, a_scale_stride=260, w_packed=P,
             w_channel_scale=None, bias=None, T=4, H=256, num_heads=2, num_kv_heads=2,
             head_dim=64, layout=0, out=P, ssq=None, workspace=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.qkv_rowmx_project(*a.values())


def _nr(L, **kw):
    a = dict(qkv=P, ssq=P, q_gamma=P, k_gamma=P, cos=P, sin=P, T=4, num_heads=2, num_kv_heads=2,
             head_dim=64, eps=1e-6, flags=7, layout=0, stream=None)
    a.update(kw)
    return L.qk_norm_rope_apply(*a.values())


def test_projection_validation():
    from rope_mxfp8_qkv_amd import _abi
    L = _lib()
    assert _proj(L, a_codes=None) == 1
    assert _proj(L, H=100, a_row_stride=104, a_scale_stride=104) == 2
    assert _proj(L, head_dim=40) == 2
    assert _proj(L, T=0) == 2
    assert _proj(L, layout=2) == 4                                # unknown layout
    assert _proj(L, layout=1, T=4_000_000) == 6                   # NBSd offsets past 2^31
    assert _proj(L, a_row_stride=258) == 2
    assert _proj(L, workspace=None) == 5                          # workspace is required
    assert _proj(L, ssq=P, workspace=P, ws_bytes=8) == 5          # workspace too small
    assert _proj(L, workspace=P + 16) == 3
    assert _proj(L, out=P + 2) == 3
    assert _proj(L, a_scales=P + 2) == 3
    assert _proj(L, w_packed=P + 16) == 3
    assert "alignment" in _abi.last_error()


def test_norm_rope_validation():
    L = _lib()
    assert _nr(L, qkv=None) == 1
    assert _nr(L, cos=None) == 4                                  # RoPE without tables
    assert _nr(L, num_kv_heads=0) == 4                            # k_gamma with no K segment
    assert _nr(L, num_kv_heads=0, k_gamma=None) == 4              # NORM_K with no K segment
    assert _nr(L, flags=1 | 4, k_gamma=P) == 4                    # k_gamma without NORM_K
    assert _nr(L, q_gamma=None) == 4
    assert _nr(L, ssq=None) == 4
    assert _nr(L, flags=8) == 4
    assert _nr(L, head_dim=24) == 2
    assert _nr(L, eps=-1.0) == 4
    assert _nr(L, layout=2) == 4                                  # unknown layout
    assert _nr(L, qkv=P + 8) == 3


def test_producer_and_weight_validation():
    L = _lib()
    assert L.rmsnorm_mx_quantize(P, P, P, 1e-6, 4, 256, 0, None, P, None) == 4   # no residual_out
    assert L.rmsnorm_mx_quantize(P, None, P, 1e-6, 4, 256, 0, P, P, None) == 4   # stray residual_out
    assert L.rmsnorm_mx_quantize(P, None, P, 1e-6, 4, 250, 0, None, P, None) == 2
    assert L.rmsnorm_mx_quantize(P, None, P, 1e-6, 4, 256, 257, None, P, None) == 2
    assert L.rmsnorm_mx_quantize(P, None, P, 1e-6, 4, 32768, 0, None, P, None) == 6
    assert L.rmsnorm_mx_quantize(P, None, P, 1e-6, 4, 16384 + 32, 0, None, P, None) == 6  # widest: 16384
    assert L.row_quantize_packed(P, 0, 4, 16384 + 32, P, None) == 6
    assert L.rmsnorm_mx_quantize(None, None, P, 1e-6, 4, 256, 0, None, P, None) == 1
    assert L.row_quantize_packed(P, 5, 4, 256, P, None) == 4
    assert L.row_quantize_packed(P, 0, 4, 96 + 8, P, None) == 2
    assert L.row_quantize_packed(P + 4, 0, 4, 256, P, None) == 3
    assert L.mx_weight_quantize(P, 100, 16, P, P, None) == 2
    assert L.qkv_weight_prepack(P, P, 256, 16, P, 10, None) == 2                 # buffer too small
    assert L.qkv_weight_prepack(P, P, 256, 16, P + 64, 1 << 20, None) == 3


def _stproj(L, **kw):
    a = dict(act_image=P, image_bytes=1 << 30, row_scale=P, w_packed=P, w_channel_scale=None,
             bias=None, T=4, H=256, num_heads=2, num_kv_heads=2, head_dim=64, layout=0, out=P,
             ssq=None, workspace=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.qkv_rowmx_project_staged(*a.values())


def test_staged_path_validation():
    L = _lib()
    assert _stproj(L, act_image=None) == 1
    assert _stproj(L, row_scale=None) == 1
    assert _stproj(L, H=100) == 2
    assert _stproj(L, image_bytes=16384 * 4 - 1) == 2              # image too small for H = 256
    assert _stproj(L, head_dim=40) == 2
    assert _stproj(L, layout=2) == 4
    assert _stproj(L, workspace=None) == 5
    assert _stproj(L, ws_bytes=8) == 5
    assert _stproj(L, act_image=P + 16) == 3
    assert _stproj(L, row_scale=P + 2) == 3
    assert _stproj(L, out=P + 2) == 3
    # producers: (x, dtype, T, H, image, image_bytes, row_scale, stream)
    assert L.row_quantize_staged(P, 0, 4, 256, P, 1 << 20, None, None) == 1
    assert L.row_quantize_staged(P, 3, 4, 256, P, 1 << 20, P, None) == 4
    assert L.row_quantize_staged(P, 0, 4, 250, P, 1 << 20, P, None) == 2
    assert L.row_quantize_staged(P, 0, 4, 256, P, 100, P, None) == 2
    assert L.row_quantize_staged(P, 0, 4, 32768, P, 1 << 30, P, None) == 6
    assert L.row_quantize_staged(P, 0, 4, 16384 + 32, P, 1 << 30, P, None) == 6
    assert L.row_quantize_staged(P, 0, 4, 256, P + 8, 1 << 20, P, None) == 3
    # (hidden, residual, gamma, eps, T, H, Hu, residual_out, image, image_bytes, row_scale, s)
    assert L.rmsnorm_mx_quantize_staged(P, P, P, 1e-6, 4, 256, 0, None, P, 1 << 20, P, None) == 4
    assert L.rmsnorm_mx_quantize_staged(P, None, P, 1e-6, 4, 256, 300, None, P, 1 << 20, P, None) == 2
    assert L.rmsnorm_mx_quantize_staged(P, None, P, -1.0, 4, 256, 0, None, P, 1 << 20, P, None) == 4
    assert L.rmsnorm_mx_quantize_staged(P, None, P, 1e-6, 4, 256, 0, None, P, 10, P, None) == 2
    assert L.rmsnorm_mx_quantize_staged(P, None, P, 1e-6, 4, 256, 0, None, P, 1 << 20, P + 2, None) == 3
    assert L.rmsnorm_mx_quantize_staged(None, None, P, 1e-6, 4, 256, 0, None, P, 1 << 20, P, None) == 1


def _stproj_na(L, **kw):
    a = dict(act_image=P, image_bytes=1 << 30, row_scale=P, w_packed=P, w_channel_scale=None,
             bias=None, T=4, H=256, num_heads=2, num_kv_heads=2, head_dim=64, layout=0, out=P,
             ssq=None, stream=None)
    a.update(kw)
    return L.qkv_rowmx_project_staged_noalloc(*a.values())


def test_noalloc_projection_validation():
    """The entry point without a workspace: the same host checks as the staged projection, and
    calls whose scratch would exceed the static array are refused before any HIP call."""
    L = _lib()
    cap = L.qkvmx_noalloc_scratch_bytes()
    assert cap == 80 << 20
    # the full-video call fits, with its 120 partials per token
    assert L.qkv_staged_workspace_bytes(75600, 15360) <= cap
    assert _stproj_na(L, act_image=None) == 1
    assert _stproj_na(L, out=None) == 1
    assert _stproj_na(L, H=100) == 2
    assert _stproj_na(L, head_dim=40) == 2
    assert _stproj_na(L, layout=2) == 4
    assert _stproj_na(L, image_bytes=16384 * 4 - 1) == 2
    assert _stproj_na(L, act_image=P + 16) == 3
    assert _stproj_na(L, out=P + 2) == 3
    # too large for the scratch: T = 90000 tokens at I = 15360 needs 120 * 90000 * 8 bytes
    assert L.qkv_staged_workspace_bytes(90000, 15360) > cap
    assert _stproj_na(L, T=90000, num_heads=40, num_kv_heads=40, head_dim=128) == 5
    from rope_mxfp8_qkv_amd import _abi
    assert "static scratch holds" in _abi.last_error()


def test_mx_staged_validation():
    L = _lib()
    # exponent image: 296 token tiles x 20 supersteps x 256 rows x 2 dwords
    assert L.qkv_act_exp_image_bytes(75600, 5120) == 296 * 20 * 256 * 8
    assert L.qkv_act_exp_image_bytes(300, 2080) == 2 * 9 * 256 * 8
    assert L.qkv_act_exp_image_bytes(4, 100) == 0
    big = 1 << 30
    # (x, dtype, T, H, image, image_bytes, exp_image, exp_bytes, stream)
    assert L.mx_block_quantize_staged(P, 0, 4, 256, P, big, None, big, None) == 1
    assert L.mx_block_quantize_staged(P, 2, 4, 256, P, big, P, big, None) == 4
    assert L.mx_block_quantize_staged(P, 0, 4, 100, P, big, P, big, None) == 2
    assert L.mx_block_quantize_staged(P, 0, 4, 256, P, big, P, 100, None) == 2
    assert L.mx_block_quantize_staged(P, 0, 4, 256, P, big, P + 4, big, None) == 3
    # (hidden, residual, gamma, eps, T, H, Hu, residual_out, image, ib, exp, eb, norm_out, s)
    assert L.rmsnorm_mx_block_quantize_staged(P, P, P, 1e-6, 4, 256, 0, None, P, big, P, big, None, None) == 4
    assert L.rmsnorm_mx_block_quantize_staged(P, None, P, 1e-6, 4, 256, 0, None, P, 10, P, big, None, None) == 2
    assert L.rmsnorm_mx_block_quantize_staged(P, None, P, 1e-6, 4, 256, 0, None, P, big, P, big, P + 8, None) == 3
    a = dict(act_image=P, image_bytes=big, exp_image=P, exp_bytes=big, w_packed=P,
             w_channel_scale=None, bias=None, T=4, H=256, num_heads=2, num_kv_heads=2,
             head_dim=64, layout=0, out=P, ssq=None, workspace=P, ws_bytes=big, stream=None)
    call = lambda **kw: L.qkv_mx_project_staged(*{**a, **kw}.values())
    assert call(exp_image=None) == 1
    assert call(exp_bytes=8) == 2
    assert call(layout=5) == 4
    assert call(workspace=None) == 5
    assert call(ws_bytes=8) == 5
    assert call(exp_image=P + 16) == 3


def test_calibration_probe_validation():
    L = _lib()
    assert L.qkvmx_mfma_rate_probe(0, 10, 1, P, P, None) == 2
    assert L.qkvmx_mfma_rate_probe(4, 0, 1, P, P, None) == 2
    assert L.qkvmx_mfma_rate_probe(4, 10, 1, None, P, None) == 1
    assert L.qkvmx_mfma_rate_probe(4, 10, 1, P, P + 4, None) == 3


def _mxproj(L, **kw):
    a = dict(a_codes=P, a_row_stride=256, a_e8m0=P, a_e8m0_stride=8, w_packed=P,
             w_channel_scale=None, bias=None, T=4, H=256, num_heads=2, num_kv_heads=2,
             head_dim=64, layout=0, out=P, ssq=None, workspace=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.qkv_mx_project(*a.values())


def test_mx_path_validation():
    from rope_mxfp8_qkv_amd import _abi
    L = _lib()
    # workspace: code stage images (296 token tiles x 80 stages x 16 KiB), exponent images
    # (296 x 20 supersteps x 2 KiB), the sum-of-squares partials (one per 128 output channels:
    # 120 at I = 15360), 256-byte alignment, the counter block
    part_end = 296 * 80 * 16384 + 296 * 20 * 2048 + 120 * 75600 * 8
    assert L.qkv_mx_workspace_bytes(75600, 5120, 15360) == (part_end + 255) // 256 * 256 + 256
    assert L.qkv_mx_workspace_bytes(4, 100, 16) == 0
    assert _mxproj(L, a_e8m0=None) == 1
    assert _mxproj(L, H=100, a_row_stride=100, a_e8m0_stride=4) == 2    # H % 32 != 0
    assert _mxproj(L, a_row_stride=258) == 2                           # not a multiple of 4
    assert _mxproj(L, a_e8m0_stride=4) == 2                            # < H / 32
    assert _mxproj(L, a_codes=P + 2) == 3                              # codes 4-byte aligned
    assert _mxproj(L, workspace=None) == 5
    assert _mxproj(L, ssq=P, ws_bytes=8) == 5
    assert _mxproj(L, layout=3) == 4
    assert "layout" in _abi.last_error()
    assert L.mx_block_quantize(P, 0, 4, 100, P, P, None) == 2
    assert L.mx_block_quantize(P, 2, 4, 256, P, P, None) == 4
    assert L.mx_block_quantize(P, 0, 4, 256, P + 4, P, None) == 3
    assert L.mx_block_quantize(P, 0, 4, 32768, P, P, None) == 6
    assert L.mx_block_quantize(P, 0, 4, 16384 + 32, P, P, None) == 6
    assert L.rmsnorm_mx_block_quantize(P, P, P, 1e-6, 4, 256, 0, None, P, P, None, None) == 4
    assert L.rmsnorm_mx_block_quantize(P, None, P, 1e-6, 4, 256, 0, None, P, P, P + 8, None) == 3
    assert L.rmsnorm_mx_block_quantize(P, None, P, -1.0, 4, 256, 0, None, P, P, None, None) == 4
    assert L.rmsnorm_mx_block_quantize(None, None, P, 1e-6, 4, 256, 0, None, P, P, None, None) == 1


def _hnproj(L, staged, **kw):
    if staged:
        a = dict(act_image=P, image_bytes=1 << 30, row_scale=P, w_packed=P, bias=None, T=4,
                 H=256, num_heads=2, num_kv_heads=2, head_dim=64, layout=0, norm_kind=1,
                 q_gamma=P, k_gamma=P, q_beta=None, k_beta=None, eps=1e-6, cos_tab=None,
                 sin_tab=None, out=P, workspace=P, ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return L.qkv_rowmx_project_headnorm_staged(*a.values())
    a = dict(a_codes=P, a_row_stride=260, a_scales=P + 256, a_scale_stride=260, w_packed=P,
             bias=None, T=4, H=256, num_heads=2, num_kv_heads=2, head_dim=64, layout=0,
             norm_kind=1, q_gamma=P, k_gamma=P, q_beta=None, k_beta=None, eps=1e-6, cos_tab=None,
             sin_tab=None, out=P, workspace=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.qkv_rowmx_project_headnorm(*a.values())


@pytest.mark.parametrize("staged", [False, True], ids=["packed", "staged"])
def test_headnorm_validation(staged):
    """The per-head qk-norm projections (rows and staged) reject every invalid argument on the
    host with the documented status."""
    L = _lib()
    f = lambda **kw: _hnproj(L, staged, **kw)
    assert f(w_packed=None) == 1
    assert f(out=None) == 1
    assert f(**({"act_image": None} if staged else {"a_codes": None})) == 1
    assert f(workspace=None) == 5
    assert f(norm_kind=0) == 4 and f(norm_kind=3) == 4
    assert f(T=0) == 2 and f(H=100) == 2
    assert f(head_dim=96) == 6                          # fused epilogue: d = 64 or 128
    assert f(num_heads=1) == 6                          # Q segment of 64 channels
    assert f(layout=2) == 4
    assert f(q_gamma=None) == 4 and f(k_gamma=None) == 4
    assert f(num_kv_heads=0) == 4                       # k_gamma given without a K segment
    assert f(q_beta=P) == 4                             # beta with RMS_NORM
    assert f(norm_kind=2, q_beta=P, k_beta=P, ws_bytes=100) == 5   # LAYER_NORM takes betas
    assert f(cos_tab=P) == 4                            # cos without sin
    assert f(eps=-1.0) == 4 and f(eps=float("nan")) == 4
    assert f(ws_bytes=100) == 5
    assert f(q_gamma=P + 2) == 3 and f(out=P + 8) == 3
    if staged:
        assert f(image_bytes=100) == 2
        assert f(act_image=P + 16) == 3
        assert f(row_scale=P + 2) == 3
    else:
        assert f(a_row_stride=100) == 2
