"""GPU parity of the projection with the per-head qk-norm (RMS_NORM / LAYER_NORM) and
rotate-half RoPE fused into its epilogue ([QKV-CTE] "Upstream behavior"), against the oracle's
pass 1 followed by its per-head norm and RoPE (fp64, one bf16 rounding on the GPU side only).
Covers head_dim 64 and 128, LayerNorm with and without beta, RoPE on and off, with and without
a bias, GQA, a single segment, ragged T and I, T = 1 and both output layouts, with the staged hand-over giving the
same bytes as the packed rows; that only the first half of each table row is read; and the
unsupported shapes."""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth
from oracle import codecs

pytestmark = pytest.mark.gpu

RMS, LN = 1, 2
CASES = [
    # name, projection, kind, rope, beta, layout, bias
    ("d64-rms-rope", G.custom_projection("hn1", T=128, H=256, nq=2, nkv=2, d=64), RMS, True, False, "bsd", True),
    ("d128-ln-beta-rope-nbsd", G.custom_projection("hn2", T=300, H=512, nq=3, nkv=1, d=128), LN, True, True, "nbsd", True),
    ("d64-rms-T1", G.custom_projection("hn3", T=1, H=256, nq=2, nkv=2, d=64), RMS, False, False, "bsd", True),
    ("single-seg-ln", G.custom_projection("hn4", T=257, H=1024, nq=4, nkv=0, d=128, rope="1d"), LN, True, False, "bsd", True),
    ("gqa-d128-rms", G.custom_projection("hn5", T=700, H=1024, nq=8, nkv=2, d=128), RMS, True, False, "bsd", True),
    ("d64-ln-nbsd", G.custom_projection("hn6", T=130, H=512, nq=6, nkv=2, d=64), LN, False, True, "nbsd", True),
    # without a bias (the epilogue's bias-free instantiations)
    ("d128-rms-rope-nobias", G.custom_projection("hn7", T=300, H=512, nq=3, nkv=1, d=128), RMS, True, False, "bsd", False),
    ("d64-ln-beta-rope-nobias-nbsd", G.custom_projection("hn8", T=200, H=256, nq=4, nkv=2, d=64), LN, True, True, "nbsd", False),
    ("single-seg-rms-nobias", G.custom_projection("hn9", T=90, H=256, nq=2, nkv=0, d=128, rope=None), RMS, False, False, "bsd", False),
]


@pytest.mark.parametrize("name,p,kind,rope,beta,layout,with_bias", CASES, ids=[c[0] for c in CASES])
def test_headnorm_parity(name, p, kind, rope, beta, layout, with_bias):
    import torch
    import rope_mxfp8_qkv_amd as q
    q.lib()
    dev = G.torch_dev()
    inp = G.make_inputs(p, with_bias=with_bias)
    d = p.head_dim
    rng = np.random.default_rng(17)
    gq = codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(d))
    gk = codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(d)) if p.num_kv_heads else None
    bq = codecs.f64_to_bf16(0.1 * rng.standard_normal(d)) if beta else None
    bk = codecs.f64_to_bf16(0.1 * rng.standard_normal(d)) if beta and p.num_kv_heads else None
    cos, sin = (inp.cos, inp.sin) if rope else (None, None)
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    X, _ = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, None, inp.bias,
                          num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=d)
    ref = oracle.head_norm_rope(X, kind, gq, gk, 1e-6, cos, sin, num_heads=p.num_heads,
                                num_kv_heads=p.num_kv_heads, head_dim=d, q_beta_bf16=bq,
                                k_beta_bf16=bk)
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    shape = (p.I // d, p.T, d) if layout == "nbsd" else (p.T, p.I)
    out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    opt = lambda a: None if a is None else G.bf16_dev(a, dev)
    kw = dict(H=p.H, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=d,
              norm_kind=kind, q_gamma=opt(gq), k_gamma=opt(gk), q_beta=opt(bq), k_beta=opt(bk),
              eps=1e-6, cos=None if cos is None else G.to_dev(cos, dev),
              sin=None if sin is None else G.to_dev(sin, dev), bias=opt(inp.bias),
              layout=q.LAYOUT_NBSD if layout == "nbsd" else q.LAYOUT_BSD)
    q.qkv_rowmx_project_headnorm(G.to_dev(inp.packed, dev), wp, out, workspace=ws, **kw)
    # the staged hand-over of the same codes and scales (the staged encoder matches the oracle's
    # rows bit for bit): the same bytes, without the per-call re-layout
    img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
    sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
    q.row_quantize_staged(G.to_dev(inp.x, dev), img, sc)
    out_s = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ws_s = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project_headnorm_staged(img, sc, wp, out_s, workspace=ws_s, **kw)
    torch.cuda.synchronize()
    got = G.bf16_host(out)
    if layout == "nbsd":
        got = oracle.nbsd_to_bsd(got)
    G.check_close(got, ref, f"{name} output")
    assert torch.equal(out_s.view(torch.int16), out.view(torch.int16)), f"{name}: staged != rows"


@pytest.mark.parametrize("d", [64, 128])
def test_headnorm_reads_first_half_of_tables(d):
    """The rotate-half tables hold each angle in both halves of a row, and the fused path reads
    the first half only (the contract of qkv_rowmx_project_headnorm): NaN in every second
    half leaves the output bit for bit unchanged."""
    import torch
    import rope_mxfp8_qkv_amd as q
    q.lib()
    dev = G.torch_dev()
    p = G.custom_projection(f"hnh{d}", T=300, H=256, nq=256 // d * 2, nkv=256 // d, d=d)
    inp = G.make_inputs(p)
    rng = np.random.default_rng(23)
    gq = G.bf16_dev(codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(d)), dev)
    gk = G.bf16_dev(codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(d)), dev)
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    ws = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    cos, sin = G.to_dev(inp.cos, dev), G.to_dev(inp.sin, dev)
    cos_nan, sin_nan = cos.clone(), sin.clone()
    cos_nan[:, d // 2:] = float("nan")
    sin_nan[:, d // 2:] = float("nan")
    outs = []
    for c, s_ in ((cos, sin), (cos_nan, sin_nan)):
        out = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev)
        q.qkv_rowmx_project_headnorm(G.to_dev(inp.packed, dev), wp, out, H=p.H,
                                     num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                     head_dim=d, norm_kind=RMS, q_gamma=gq, k_gamma=gk, eps=1e-6,
                                     cos=c, sin=s_, bias=G.bf16_dev(inp.bias, dev), workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0].float()).any()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_headnorm_unsupported_shapes():
    import torch
    import rope_mxfp8_qkv_amd as q
    q.lib()
    dev = G.torch_dev()
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    g = torch.ones(128, dtype=torch.bfloat16, device=dev)
    out = torch.empty((4, 512), dtype=torch.bfloat16, device=dev)
    wp = torch.zeros(q.qkv_weight_packed_bytes(256, 512), dtype=torch.uint8, device=dev)
    packed = torch.zeros((4, 260), dtype=torch.uint8, device=dev)
    g32 = torch.ones(32, dtype=torch.bfloat16, device=dev)
    g64 = torch.ones(64, dtype=torch.bfloat16, device=dev)
    out320 = torch.empty((4, 320), dtype=torch.bfloat16, device=dev)
    wp320 = torch.zeros(q.qkv_weight_packed_bytes(256, 320), dtype=torch.uint8, device=dev)
    with pytest.raises(q.QkvmxError) as ei:           # head_dim 32
        q.qkv_rowmx_project_headnorm(packed, wp, out, H=256, num_heads=8, num_kv_heads=4,
                                     head_dim=32, norm_kind=1, q_gamma=g32, k_gamma=g32,
                                     workspace=buf)
    assert ei.value.status == 6
    with pytest.raises(q.QkvmxError) as ei:           # Q segment of 192 channels
        q.qkv_rowmx_project_headnorm(packed, wp320, out320, H=256, num_heads=3, num_kv_heads=1,
                                     head_dim=64, norm_kind=1, q_gamma=g64, k_gamma=g64,
                                     workspace=buf)
    assert ei.value.status == 6
    with pytest.raises(q.QkvmxError) as ei:           # beta with RMS_NORM
        q.qkv_rowmx_project_headnorm(packed, wp, out, H=256, num_heads=2, num_kv_heads=1,
                                     head_dim=128, norm_kind=1, q_gamma=g, k_gamma=g, q_beta=g,
                                     workspace=buf)
    assert ei.value.status == 4
