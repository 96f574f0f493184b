"""GPU parity of the staged paths: producers that write the codes in the projection's
stage-image layout (plus fp32 row scales for ROW_MX, or an exponent image for MX block-32) and
the projections that consume them without a per-call re-layout.

Codes and scales are compared bit for bit with the oracle's ROW_MX rows (the image is read back
through the layout formula of include/qkvmx.h, restated in gpu_common.staged_index); the padding
of the image (K past H, rows past T in the last 256-row tile) must hold zero codes.  The staged
projection must give the same bytes as the packed-row projection on the same codes and scales,
and both are checked against the oracle.
"""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth

pytestmark = pytest.mark.gpu


def _lib():
    import rope_mxfp8_qkv_amd as q
    q.lib()
    return q


def _image(q, T, H, dev):
    import torch
    return torch.full((q.qkv_act_image_bytes(T, H),), 0xA5, dtype=torch.uint8, device=dev)


_check_padding = G.check_stage_padding


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_quantize_staged_bit_exact(dtype):
    import torch
    q = _lib()
    dev = G.torch_dev()
    rng = np.random.default_rng(17)
    T, H = 300, 2080                      # ragged last tile; K padding (2080 = 8 x 256 + 32)
    x = (rng.standard_normal((T, H)) * rng.uniform(1e-3, 1e3, (T, 1))).astype(np.float32)
    x[4] = 0.0
    x[5, :7] = -0.0
    x[6, 3] = -1e-30
    if dtype == "bf16":
        bits = synth.to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(bits)
        xd = G.bf16_dev(bits, dev)
    else:
        xd = G.to_dev(x, dev)
    codes_ref, s_ref = oracle.rowmx_unpack(oracle.rowmx_quantize(x), H)
    img = _image(q, T, H, dev)
    sc = torch.full((T,), float("nan"), dtype=torch.float32, device=dev)
    q.row_quantize_staged(xd, img, sc)
    torch.cuda.synchronize()
    G.check_equal(G.unstage(img, np.arange(T), H), codes_ref, "staged codes")
    G.check_equal(sc.cpu().numpy().view(np.uint32), s_ref.astype(np.float32).view(np.uint32),
                  "row scales")
    _check_padding(img, T, H)


@pytest.mark.parametrize("with_res,Hu", [(True, 0), (False, 0), (True, 4000)])
def test_rmsnorm_quantize_staged_bit_exact(with_res, Hu):
    import torch
    q = _lib()
    dev = G.torch_dev()
    T, H = 300, 5120
    hid, res, gam = synth.producer_inputs(77, T, H)
    if Hu:
        hid[:, Hu:] = 0
        res[:, Hu:] = 0
    res_ref, packed_ref, _ = oracle.rmsnorm_rowmx(hid, res if with_res else None, gam, 1e-6, Hu)
    codes_ref, s_ref = oracle.rowmx_unpack(packed_ref, H)
    img = _image(q, T, H, dev)
    sc = torch.full((T,), float("nan"), dtype=torch.float32, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if with_res else None
    q.rmsnorm_mx_quantize_staged(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, img, sc,
                                 residual=G.bf16_dev(res, dev) if with_res else None,
                                 residual_out=res_out, unpadded_h=Hu)
    torch.cuda.synchronize()
    if with_res:
        G.check_equal(G.bf16_host(res_out), res_ref, "residual_out")
    G.check_equal(G.unstage(img, np.arange(T), H), codes_ref, "staged codes")
    G.check_equal(sc.cpu().numpy().view(np.uint32), s_ref.astype(np.float32).view(np.uint32),
                  "row scales")
    _check_padding(img, T, H)


STAGED_CASES = [
    ("C1", synth.CONFIGS[1].calls[0], 0),
    ("T1", G.custom_projection("t1", T=1, H=256, nq=2, nkv=2, d=64), 0),
    ("gqa-ragged", G.custom_projection("gqa", T=129, H=96, nq=4, nkv=2, d=64), 0),
    ("ragged-N-nbsd", G.custom_projection("rn", T=300, H=512, nq=3, nkv=1, d=128), 1),
    ("single-seg", G.custom_projection("ss", T=257, H=1024, nq=5, nkv=0, d=128, rope=None), 0),
]


@pytest.mark.parametrize("name,p,layout", STAGED_CASES, ids=[c[0] for c in STAGED_CASES])
def test_projection_staged_parity(name, p, layout):
    """Staged producer -> staged projection == packed producer -> packed projection (bytes),
    and both within tolerance of the oracle."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(p)
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    X, ssq_ref = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, None, inp.bias,
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                head_dim=p.head_dim)
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    shape = (p.I // p.head_dim, p.T, p.head_dim) if layout else (p.T, p.I)
    bias = G.bf16_dev(inp.bias, dev)
    xd = G.to_dev(inp.x, dev)
    # packed rows
    packed = torch.empty((p.T, p.H + 4), dtype=torch.uint8, device=dev)
    q.row_quantize_packed(xd, packed)
    out_p = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ssq_p = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws_p = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project(packed, wp, out_p, H=p.H, num_heads=p.num_heads,
                        num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, bias=bias, ssq=ssq_p,
                        workspace=ws_p, layout=layout)
    # staged
    img = _image(q, p.T, p.H, dev)
    sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
    q.row_quantize_staged(xd, img, sc)
    out_s = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ssq_s = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws_s = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project_staged(img, sc, wp, out_s, H=p.H, num_heads=p.num_heads,
                               num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, bias=bias,
                               ssq=ssq_s, workspace=ws_s, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(out_s.view(torch.int16), out_p.view(torch.int16)), f"{name}: outputs differ"
    assert torch.equal(ssq_s, ssq_p), f"{name}: sums differ"
    got = G.bf16_host(out_s)
    if layout:
        got = oracle.nbsd_to_bsd(got)
    G.check_close(got, X, f"{name} X")
    G.check_ssq(ssq_s.cpu().numpy(), ssq_ref, f"{name} ssq")


def test_projection_staged_repeated_calls_share_workspace():
    """Two calls in a row on one workspace (the tile counters are reset by each call), the
    second with fewer tokens."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    p = G.custom_projection("rep", T=700, H=512, nq=2, nkv=2, d=128)
    inp = G.make_inputs(p)
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    for T in (p.T, 300):
        img = _image(q, T, p.H, dev)
        sc = torch.empty((T,), dtype=torch.float32, device=dev)
        q.row_quantize_staged(G.to_dev(inp.x[:T], dev), img, sc)
        out = torch.full((T, p.I), float("nan"), dtype=torch.bfloat16, device=dev)
        q.qkv_rowmx_project_staged(img, sc, wp, out, H=p.H, num_heads=2, num_kv_heads=2,
                                   head_dim=128, bias=G.bf16_dev(inp.bias, dev), workspace=ws)
        torch.cuda.synchronize()
        X, _ = oracle.project(codes[:T], sA[:T], inp.w_codes, inp.w_e8m0, None, inp.bias,
                              num_heads=2, num_kv_heads=2, head_dim=128)
        G.check_close(G.bf16_host(out), X, f"T={T} X")


# ----------------------------------------------------------------------------------------------
# MX block-32
# ----------------------------------------------------------------------------------------------

def _exp_image(q, T, H, dev):
    import torch
    n = q.qkv_act_exp_image_bytes(T, H)
    return torch.full((n // 4,), 0x5A5A5A5A, dtype=torch.int32, device=dev)


_check_exp_padding = G.check_exp_padding


def _blocky(T, H, seed, spread=6):
    """N(0,1) rows with a random power of two in 2^-spread .. 2^spread per 32-element block, a
    zero block and a tiny block.  The projection tests use spread 2: one FP8 MFMA sums its 64
    products only to a small fraction of their absolute sum, so wide spreads produce outputs that
    cancel below the plain bf16 tolerance on any encoding (the encoder tests use the wide spread;
    test_gpu_accumulation.py checks wide spreads against the tolerance plus that bound)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= np.ldexp(1.0, rng.integers(-spread, spread + 1, (T, H // 32))).repeat(32, axis=1).astype(np.float32)
    x[0, 32:64] = 0.0
    if T > 1:
        x[1, :32] *= np.float32(1e-30)
    return x


@pytest.mark.parametrize("dtype,H", [("f32", 2080), ("bf16", 5120)])
def test_mx_block_quantize_staged_bit_exact(dtype, H):
    import torch
    q = _lib()
    dev = G.torch_dev()
    T = 300
    x = _blocky(T, H, 13)
    fb = G.floor_blocks(np.random.default_rng(14))     # exponent clamps to 0 (E8M0 floor)
    for j, blk in enumerate(fb):
        x[20 + j, 96:128] = blk
    if dtype == "bf16":
        bits = synth.to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(bits)
        xd = G.bf16_dev(bits, dev)
    else:
        xd = G.to_dev(x, dev)
    codes_ref, e8_ref = oracle.mx_block_quantize(x)
    assert (e8_ref[20:20 + len(fb), 3] == 0).sum() >= 6
    img, eimg = _image(q, T, H, dev), _exp_image(q, T, H, dev)
    q.mx_block_quantize_staged(xd, img, eimg)
    torch.cuda.synchronize()
    G.check_equal(G.unstage(img, np.arange(T), H), codes_ref, "staged codes")
    G.check_equal(G.unstage_exp(eimg, np.arange(T), H), e8_ref, "staged exponents")
    _check_padding(img, T, H)
    _check_exp_padding(eimg, T, H)


@pytest.mark.parametrize("with_res,emit,Hu", [(True, True, 0), (False, False, 0), (True, True, 4000)])
def test_rmsnorm_mx_block_staged_bit_exact(with_res, emit, Hu):
    import torch
    q = _lib()
    dev = G.torch_dev()
    T, H = 300, 5120
    hid, res, gam = synth.producer_inputs(79, T, H)
    if Hu:
        hid[:, Hu:] = 0
        res[:, Hu:] = 0
    res_ref, codes_ref, e8_ref, norm_ref, _ = oracle.rmsnorm_mx(hid, res if with_res else None,
                                                                gam, 1e-6, Hu)
    img, eimg = _image(q, T, H, dev), _exp_image(q, T, H, dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if with_res else None
    norm = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if emit else None
    q.rmsnorm_mx_block_quantize_staged(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, img,
                                       eimg, residual=G.bf16_dev(res, dev) if with_res else None,
                                       residual_out=res_out, norm_out=norm, unpadded_h=Hu)
    torch.cuda.synchronize()
    if with_res:
        G.check_equal(G.bf16_host(res_out), res_ref, "residual_out")
    if emit:
        G.check_equal(G.bf16_host(norm), norm_ref, "bf16 norm output")
    G.check_equal(G.unstage(img, np.arange(T), H), codes_ref, "staged codes")
    G.check_equal(G.unstage_exp(eimg, np.arange(T), H), e8_ref, "staged exponents")
    _check_padding(img, T, H)
    _check_exp_padding(eimg, T, H)


MX_STAGED_CASES = [
    ("C1", synth.CONFIGS[1].calls[0], 0, False),
    ("ragged-T-N-chan", G.custom_projection("mrn", T=300, H=512, nq=3, nkv=1, d=128), 0, True),
    ("nbsd-ragged-H", G.custom_projection("mnb", T=200, H=352, nq=3, nkv=1, d=64), 1, False),
    ("T1", G.custom_projection("mt1", T=1, H=256, nq=2, nkv=2, d=64), 0, False),
]


@pytest.mark.parametrize("name,p,layout,chan", MX_STAGED_CASES, ids=[c[0] for c in MX_STAGED_CASES])
def test_mx_projection_staged_parity(name, p, layout, chan):
    """Staged MX producer -> staged MX projection == natural-order MX producer -> MX projection
    (bytes), and within tolerance of the oracle."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    x = _blocky(p.T, p.H, 23, spread=2)
    codes_ref, e8_ref = oracle.mx_block_quantize(x)
    w_codes, w_e8m0 = oracle.mx_weight_quantize(synth.weight(p))
    bias = synth.bias_bf16(p)
    rng = np.random.default_rng(6)
    cs = (0.5 + rng.random(p.I)).astype(np.float32) if chan else None
    X, ssq_ref = oracle.project(codes_ref, None, w_codes, w_e8m0, cs, bias,
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                head_dim=p.head_dim, a_e8m0=e8_ref)
    wp = q.prepare_weight(G.to_dev(w_codes, dev), G.to_dev(w_e8m0, dev), p.H, p.I)
    shape = (p.I // p.head_dim, p.T, p.head_dim) if layout else (p.T, p.I)
    kw = dict(H=p.H, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
              channel_scale=None if cs is None else G.to_dev(cs, dev),
              bias=G.bf16_dev(bias, dev), layout=layout)
    xd = G.to_dev(x, dev)
    codes = torch.empty((p.T, p.H), dtype=torch.uint8, device=dev)
    e8 = torch.empty((p.T, p.H // 32), dtype=torch.uint8, device=dev)
    q.mx_block_quantize(xd, codes, e8)
    out_n = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ssq_n = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws_n = torch.empty(q.qkv_mx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    q.qkv_mx_project(codes, e8, wp, out_n, ssq=ssq_n, workspace=ws_n, **kw)
    img, eimg = _image(q, p.T, p.H, dev), _exp_image(q, p.T, p.H, dev)
    q.mx_block_quantize_staged(xd, img, eimg)
    out_s = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ssq_s = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws_s = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    q.qkv_mx_project_staged(img, eimg, wp, out_s, T=p.T, ssq=ssq_s, workspace=ws_s, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_s.view(torch.int16), out_n.view(torch.int16)), f"{name}: outputs differ"
    assert torch.equal(ssq_s, ssq_n), f"{name}: sums differ"
    got = G.bf16_host(out_s)
    if layout:
        got = oracle.nbsd_to_bsd(got)
    G.check_close(got, X, f"{name} X")
    G.check_ssq(ssq_s.cpu().numpy(), ssq_ref, f"{name} ssq")
