"""Mis-sized device tensors are refused by the binding before the library is called: the call
raises QkvmxError and the outputs it was given still hold their sentinel bytes after the
stream has drained (no kernel ran).  Host-side coverage of every wrapper's checks is in
tests/test_binding_checks.py."""
import pytest

import gpu_common as G

pytestmark = pytest.mark.gpu


def test_mis_sized_device_tensors_launch_nothing():
    import torch
    import rope_mxfp8_qkv_amd as q
    q.lib()
    dev = G.torch_dev()
    T, H, nq, nkv, d = 40, 256, 2, 1, 64
    I = (nq + 2 * nkv) * d
    kw = dict(num_heads=nq, num_kv_heads=nkv, head_dim=d)
    packed = torch.zeros((T, H + 4), dtype=torch.uint8, device=dev)
    wp = torch.zeros(q.qkv_weight_packed_bytes(H, I), dtype=torch.uint8, device=dev)
    ws = torch.zeros(q.qkvmx_workspace_bytes(T, H, I), dtype=torch.uint8, device=dev)
    out = torch.full((T, I), 3.0, dtype=torch.bfloat16, device=dev)
    ssq_small = torch.full((T - 1, 2), 7.0, dtype=torch.float32, device=dev)
    cases = [
        # ssq one token short: the projection would write past its end
        lambda: q.qkv_rowmx_project(packed, wp, out, H=H, ssq=ssq_small, workspace=ws, **kw),
        # bias of the wrong dtype (fp32 read as bf16 pairs)
        lambda: q.qkv_rowmx_project(packed, wp, out, H=H, workspace=ws,
                                    bias=torch.zeros(I, dtype=torch.float32, device=dev), **kw),
        # rows without the scale tail
        lambda: q.qkv_rowmx_project(packed[:, :H].contiguous(), wp, out, H=H, workspace=ws, **kw),
        # cos / sin tables one token short
        lambda: q.qk_norm_rope_apply(out, eps=1e-6, flags=q.NORM_Q | q.FUSED_ROPE,
                                     ssq=torch.ones((T, 2), dtype=torch.float32, device=dev),
                                     q_gamma=torch.ones(nq * d, dtype=torch.bfloat16, device=dev),
                                     cos=torch.zeros((T - 1, d), dtype=torch.float32, device=dev),
                                     sin=torch.zeros((T - 1, d), dtype=torch.float32, device=dev),
                                     **kw),
        # a bf16 weight read as fp32 (twice its size)
        lambda: q.mx_weight_quantize(torch.zeros((H, I), dtype=torch.bfloat16, device=dev),
                                     torch.zeros((H // 4, I, 4), dtype=torch.uint8, device=dev),
                                     torch.zeros((H // 32, I), dtype=torch.uint8, device=dev)),
    ]
    for i, fn in enumerate(cases):
        with pytest.raises(q.QkvmxError) as ei:
            fn()
        assert ei.value.status == -1, (i, str(ei.value))
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 3.0))
    assert torch.equal(ssq_small, torch.full_like(ssq_small, 7.0))
