"""The projection entry point that allocates nothing (qkv_rowmx_project_staged_noalloc) against
the workspace entry point it mirrors (qkv_rowmx_project_staged), through the C ABI.

Both launch the same kernels, the first on the library's static per-GPU scratch, the second on
a caller-provided workspace, so out and ssq must agree bit for bit (stronger than the bf16 /
sum-of-squares tolerances).  Two calls in a row on the shared scratch, the second with a
smaller input (the scratch keeps the first call's contents, so a stale counter or partial would
show), then a call with few output tiles (its split-contraction planes also live in the
scratch), then a call too large for the scratch, refused before any kernel runs.  The first
call is also checked against the oracle on sampled rows."""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth

pytestmark = pytest.mark.gpu


def _run_pair(q, p, dev, seed):
    import torch
    x = synth.activation(p)
    codes, e8 = oracle.mx_weight_quantize(synth.weight(p))
    bias = synth.bias_bf16(p)
    xd = G.to_dev(x, dev)
    img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
    sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
    q.row_quantize_staged(xd, img, sc)
    wp = q.prepare_weight(G.to_dev(codes, dev), G.to_dev(e8, dev), p.H, p.I)
    kw = dict(H=p.H, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
              bias=G.bf16_dev(bias, dev))
    out_a = torch.full((p.T, p.I), float("nan"), dtype=torch.bfloat16, device=dev)
    ssq_a = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    q.qkv_rowmx_project_staged_noalloc(img, sc, wp, out_a, ssq=ssq_a, **kw)
    out_b = torch.full((p.T, p.I), float("nan"), dtype=torch.bfloat16, device=dev)
    ssq_b = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project_staged(img, sc, wp, out_b, ssq=ssq_b, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), p.name
    assert torch.equal(ssq_a, ssq_b), p.name
    return x, codes, e8, bias, out_a, ssq_a


def test_noalloc_matches_workspace_entry_point():
    import torch
    import rope_mxfp8_qkv_amd as q
    q.lib()
    dev = G.torch_dev()
    big = G.custom_projection("na1", T=4100, H=1024, nq=8, nkv=4, d=128)      # 17 x 8 tiles
    mid = G.custom_projection("na2", T=3000, H=512, nq=12, nkv=6, d=128)      # 12 x 12 tiles
    small = G.custom_projection("na3", T=300, H=512, nq=2, nkv=1, d=64)
    split = G.custom_projection("na4", T=512, H=5120, nq=20, nkv=0, d=128, rope=None)
    assert q.projection_k_chunks(big.T, big.H, big.I) == 1
    assert q.projection_k_chunks(mid.T, mid.H, mid.I) == 1
    assert q.projection_k_chunks(split.T, split.H, split.I) > 1
    x, codes, e8, bias, out, ssq = _run_pair(q, big, dev, 1)
    rows = np.array([0, 1, 255, 256, 777, 1023, 2048, 4095, 4096, 4099])
    packed = oracle.rowmx_quantize(x[rows])
    c, sA = oracle.rowmx_unpack(packed, big.H)
    X, ssq_ref = oracle.project(c, sA, codes, e8, None, bias, num_heads=big.num_heads,
                                num_kv_heads=big.num_kv_heads, head_dim=big.head_dim)
    G.check_close(G.bf16_host(out)[rows], X, "noalloc vs oracle")
    G.check_ssq(ssq.cpu().numpy()[rows], ssq_ref, "noalloc ssq vs oracle")
    _run_pair(q, mid, dev, 2)                   # second call, smaller input
    _run_pair(q, small, dev, 3)
    _run_pair(q, split, dev, 4)                 # split contraction: planes in the scratch
    # a call too large for the scratch is refused on the host; nothing is written
    T = 90000
    assert q.qkv_staged_workspace_bytes(T, 15360) > q.noalloc_scratch_bytes()
    img = torch.zeros(q.qkv_act_image_bytes(T, 256), dtype=torch.uint8, device=dev)
    sc = torch.zeros((T,), dtype=torch.float32, device=dev)
    wp = torch.zeros(q.qkv_weight_packed_bytes(256, 15360), dtype=torch.uint8, device=dev)
    o = torch.full((T, 15360), 5.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(q.QkvmxError) as ei:
        q.qkv_rowmx_project_staged_noalloc(img, sc, wp, o, H=256, num_heads=40, num_kv_heads=40,
                                           head_dim=128)
    assert ei.value.status == 5 and "static scratch holds" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((o == 5.0).all())
