"""The Python binding checks every tensor's dtype and size against the call's dimensions before
it calls the library (the C ABI receives raw pointers and cannot see a buffer's extent).

Run on the CPU with host tensors: a mis-sized or mis-typed tensor must raise QkvmxError naming
that tensor; with every tensor sized correctly the call gets past the checks and stops at the
device check ("expected a device tensor"), so no pointer of a wrong-sized buffer ever reaches
the library.  The GPU counterpart (tests/test_gpu_binding_checks.py) passes device tensors and
checks that nothing was written.
"""
import pytest
import torch

import rope_mxfp8_qkv_amd as q

u8, f32, bf16, i64 = torch.uint8, torch.float32, torch.bfloat16, torch.int64
DEVICE_MSG = "expected a device tensor"


def z(shape, dt):
    return torch.zeros(shape, dtype=dt)


def raises(fn, match):
    with pytest.raises(q.QkvmxError, match=match):
        fn()


T, H, nq, nkv, d = 6, 256, 2, 1, 64
I = (nq + 2 * nkv) * d
HEADS = dict(num_heads=nq, num_kv_heads=nkv, head_dim=d)


def proj_ok():
    return dict(w_packed=z(q.qkv_weight_packed_bytes(H, I), u8), out=z((T, I), bf16),
                bias=z(I, bf16), ssq=z((T, 2), f32), workspace=z(1 << 16, u8))


def test_encoders():
    raises(lambda: q.mx_weight_quantize(z((H, I), bf16), z((H // 4, I, 4), u8),
                                        z((H // 32, I), u8)), "w: dtype")
    raises(lambda: q.mx_weight_quantize(z((H, I), f32), z((H // 4, I, 2), u8),
                                        z((H // 32, I), u8)), "codes_out")
    raises(lambda: q.mx_weight_quantize(z((H, I), f32), z((H // 4, I, 4), u8),
                                        z((H // 16, I), u8)), "e8m0_out")
    raises(lambda: q.mx_weight_quantize(z((H, I), f32), z((H // 4, I, 4), u8),
                                        z((H // 32, I), u8)), DEVICE_MSG)
    raises(lambda: q.row_quantize_packed(z((T, H), f32), z((T, H), u8)), "packed_out")
    raises(lambda: q.row_quantize_packed(z((T, H), torch.float16), z((T, H + 4), u8)), "x: dtype")
    raises(lambda: q.row_quantize_packed(z((T, H), f32), z((T, H + 4), u8)), DEVICE_MSG)
    raises(lambda: q.mx_block_quantize(z((T, H), f32), z((T, H), u8), z((T, H // 16), u8)),
           "e8m0_out")
    raises(lambda: q.row_quantize_staged(z((T, H), f32), z(q.qkv_act_image_bytes(T, H), u8),
                                         z(T + 1, f32)), "row_scale")
    raises(lambda: q.qkv_weight_prepack(z((H // 4, I, 4), u8), z((H // 32, I + 1), u8), H, I,
                                        z(q.qkv_weight_packed_bytes(H, I), u8)), "e8m0")


def test_producers():
    hid, gam = z((T, H), bf16), z(H, bf16)
    raises(lambda: q.rmsnorm_mx_quantize(hid, z(H - 2, bf16), 1e-6, z((T, H + 4), u8)), "gamma")
    raises(lambda: q.rmsnorm_mx_quantize(hid, gam, 1e-6, z((T, H + 4), u8), residual=z((T, H), f32),
                                         residual_out=z((T, H), bf16)), "residual: dtype")
    raises(lambda: q.rmsnorm_mx_quantize(hid, gam, 1e-6, z((T, H + 4), u8), residual=z((T, H), bf16),
                                         residual_out=z((T - 1, H), bf16)), "residual_out")
    raises(lambda: q.rmsnorm_mx_quantize(hid, gam, 1e-6, z((T, H + 3), u8)), "packed_out")
    raises(lambda: q.rmsnorm_mx_quantize(hid.float(), gam, 1e-6, z((T, H + 4), u8)), "hidden")
    raises(lambda: q.rmsnorm_mx_block_quantize(hid, gam, 1e-6, z((T, H), u8), z((T, H // 32), u8),
                                               norm_out=z((T, H), f32)), "norm_out")
    raises(lambda: q.rmsnorm_mx_quantize(hid, gam, 1e-6, z((T, H + 4), u8)), DEVICE_MSG)


def test_projections():
    packed = z((T, H + 4), u8)
    k = proj_ok()
    raises(lambda: q.qkv_rowmx_project(packed, k["w_packed"], z((T, I - 64), bf16), H=H, **HEADS),
           "out")
    raises(lambda: q.qkv_rowmx_project(packed, k["w_packed"], k["out"], H=H, ssq=z((T, 2), bf16),
                                       **HEADS), "ssq: dtype")
    raises(lambda: q.qkv_rowmx_project(packed, k["w_packed"], k["out"], H=H, bias=z(I - 16, bf16),
                                       **HEADS), "bias")
    raises(lambda: q.qkv_rowmx_project(packed, k["w_packed"], k["out"], H=H,
                                       channel_scale=z(I, bf16), **HEADS), "channel_scale")
    raises(lambda: q.qkv_rowmx_project(packed, k["w_packed"][:100], k["out"], H=H, **HEADS),
           "w_packed")
    # rows too short for the implied scale tail (the last row's scale would be read past the end)
    raises(lambda: q.qkv_rowmx_project(z((T, H), u8), k["w_packed"], k["out"], H=H, **HEADS),
           "scale tail")
    raises(lambda: q.qkv_rowmx_project(packed, k["w_packed"], k["out"], H=H,
                                       a_scales=z(T - 1, f32), **HEADS), "a_scales")
    raises(lambda: q.qkv_rowmx_project(packed, **k, H=H, **HEADS), DEVICE_MSG)
    raises(lambda: q.qkv_mx_project(z((T, H), u8), z((T, H // 64), u8), k["w_packed"], k["out"],
                                    H=H, **HEADS), "do not cover")
    raises(lambda: q.qkv_rowmx_project_staged(z(q.qkv_act_image_bytes(T, H), u8), z(T, f32),
                                              k["w_packed"], z((T + 1, I), bf16), H=H, **HEADS),
           "out")
    raises(lambda: q.qkv_rowmx_project_headnorm(packed, k["w_packed"], k["out"], H=H, norm_kind=1,
                                                q_gamma=z(2 * d, bf16), **HEADS), "q_gamma")
    raises(lambda: q.qkv_rowmx_project_headnorm(packed, k["w_packed"], k["out"], H=H, norm_kind=1,
                                                q_gamma=z(d, bf16), cos=z((T, d), bf16),
                                                sin=z((T, d), f32), **HEADS), "cos: dtype")


def test_norm_rope():
    qkv = z((T, I), bf16)
    fl = q.NORM_Q | q.NORM_K | q.FUSED_ROPE
    ok = dict(ssq=z((T, 2), f32), q_gamma=z(nq * d, bf16), k_gamma=z(nkv * d, bf16),
              cos=z((T, d), f32), sin=z((T, d), f32))
    for name, bad, match in (("ssq", z((T, 3), f32), "ssq"), ("q_gamma", z(nq * d + 8, bf16), "q_gamma"),
                             ("k_gamma", z(nq * d, bf16), "k_gamma"), ("cos", z((T, d // 2), f32), "cos"),
                             ("sin", z((T, d), bf16), "sin: dtype")):
        kw = dict(ok)
        kw[name] = bad
        raises(lambda: q.qk_norm_rope_apply(qkv, eps=1e-6, flags=fl, **kw, **HEADS), match)
    raises(lambda: q.qk_norm_rope_apply(z((T, I + 2), bf16), eps=1e-6, flags=fl, **ok, **HEADS),
           "qkv")
    raises(lambda: q.qk_norm_rope_apply(qkv, eps=1e-6, flags=fl, layout=q.LAYOUT_NBSD, **ok,
                                        **HEADS), "is not")
    raises(lambda: q.qk_norm_rope_apply(qkv, eps=1e-6, flags=fl, **ok, **HEADS), DEVICE_MSG)


def test_probe():
    raises(lambda: q.mfma_rate_probe(4, 10, True, z(4 * 255, f32), z((4, 2), i64)), "sink")
    raises(lambda: q.mfma_rate_probe(4, 10, True, z(4 * 256, f32), z((4, 2), f32)), "clocks")


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises: there is no fallback path (the
    size queries and the operations all go through the one loader)."""
    from rope_mxfp8_qkv_amd import _abi
    monkeypatch.setattr(_abi, "_LIB_PATH", str(tmp_path / "libqkvmx.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(q.QkvmxError, match="is missing"):
        q.qkv_weight_packed_bytes(H, I)
    with pytest.raises(q.QkvmxError, match="is missing"):
        q.lib()
