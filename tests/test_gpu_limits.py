"""GPU parity at the widest rows the row kernels accept (H = 16384: a producer block keeps one
whole row in registers, and the C ABI rejects wider rows host-side with QKVMX_ERR_UNSUPPORTED).

Every producer and encoder, in the pages' row layouts and staged, must match the oracle bit for
bit at that width; the projections (packed and staged ROW_MX, staged MX) must stay within the
output tolerance over a 16384-long contraction, 64 K-steps of 256 bytes.
"""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth

pytestmark = pytest.mark.gpu

HMAX = 16384
T = 37


def _lib():
    import rope_mxfp8_qkv_amd as q
    q.lib()
    return q


def _x(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, HMAX)) * rng.uniform(1e-2, 1e2, (T, 1))).astype(np.float32)
    x[3] = 0.0
    x[4, 100:132] = 0.0                     # a zero MX block inside a non-zero row
    x[5, 7] = 1e5                           # one element far above the rest of its row / block
    return x


def test_row_encoders_max_width():
    import torch
    q = _lib()
    dev = G.torch_dev()
    x = _x(31)
    xd = G.to_dev(x, dev)
    packed_ref = oracle.rowmx_quantize(x)
    packed = torch.empty((T, HMAX + 4), dtype=torch.uint8, device=dev)
    q.row_quantize_packed(xd, packed)
    img = torch.full((q.qkv_act_image_bytes(T, HMAX),), 0xA5, dtype=torch.uint8, device=dev)
    sc = torch.empty((T,), dtype=torch.float32, device=dev)
    q.row_quantize_staged(xd, img, sc)
    torch.cuda.synchronize()
    G.check_equal(packed.cpu().numpy(), packed_ref, "ROW_MX rows")
    codes_ref, s_ref = oracle.rowmx_unpack(packed_ref, HMAX)
    G.check_equal(G.unstage(img, np.arange(T), HMAX), codes_ref, "staged ROW_MX codes")
    G.check_equal(sc.cpu().numpy().view(np.uint32), s_ref.astype(np.float32).view(np.uint32),
                  "row scales")

    codes_ref, e8_ref = oracle.mx_block_quantize(x)
    codes = torch.empty((T, HMAX), dtype=torch.uint8, device=dev)
    e8 = torch.empty((T, HMAX // 32), dtype=torch.uint8, device=dev)
    q.mx_block_quantize(xd, codes, e8)
    eimg = torch.empty(q.qkv_act_exp_image_bytes(T, HMAX) // 4, dtype=torch.int32, device=dev)
    q.mx_block_quantize_staged(xd, img, eimg)
    torch.cuda.synchronize()
    G.check_equal(codes.cpu().numpy(), codes_ref, "MX codes")
    G.check_equal(e8.cpu().numpy(), e8_ref, "MX exponents")
    G.check_equal(G.unstage(img, np.arange(T), HMAX), codes_ref, "staged MX codes")
    G.check_equal(G.unstage_exp(eimg, np.arange(T), HMAX), e8_ref, "staged MX exponents")


def test_producers_max_width():
    import torch
    q = _lib()
    dev = G.torch_dev()
    hid, res, gam = synth.producer_inputs(79, T, HMAX)
    hd, rd, gd = G.bf16_dev(hid, dev), G.bf16_dev(res, dev), G.bf16_dev(gam, dev)

    res_ref, packed_ref, _ = oracle.rmsnorm_rowmx(hid, res, gam, 1e-6)
    packed = torch.empty((T, HMAX + 4), dtype=torch.uint8, device=dev)
    res_out = torch.empty((T, HMAX), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_quantize(hd, gd, 1e-6, packed, residual=rd, residual_out=res_out)
    img = torch.full((q.qkv_act_image_bytes(T, HMAX),), 0xA5, dtype=torch.uint8, device=dev)
    sc = torch.empty((T,), dtype=torch.float32, device=dev)
    res_out2 = torch.empty((T, HMAX), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_quantize_staged(hd, gd, 1e-6, img, sc, residual=rd, residual_out=res_out2)
    torch.cuda.synchronize()
    G.check_equal(G.bf16_host(res_out), res_ref, "residual_out (ROW_MX producer)")
    G.check_equal(G.bf16_host(res_out2), res_ref, "residual_out (staged ROW_MX producer)")
    G.check_equal(packed.cpu().numpy(), packed_ref, "ROW_MX producer rows")
    codes_ref, s_ref = oracle.rowmx_unpack(packed_ref, HMAX)
    G.check_equal(G.unstage(img, np.arange(T), HMAX), codes_ref, "staged ROW_MX producer codes")
    G.check_equal(sc.cpu().numpy().view(np.uint32), s_ref.astype(np.float32).view(np.uint32),
                  "staged ROW_MX producer scales")

    res_ref, codes_ref, e8_ref, norm_ref, _ = oracle.rmsnorm_mx(hid, res, gam, 1e-6)
    codes = torch.empty((T, HMAX), dtype=torch.uint8, device=dev)
    e8 = torch.empty((T, HMAX // 32), dtype=torch.uint8, device=dev)
    norm = torch.empty((T, HMAX), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_block_quantize(hd, gd, 1e-6, codes, e8, residual=rd, residual_out=res_out,
                                norm_out=norm)
    eimg = torch.empty(q.qkv_act_exp_image_bytes(T, HMAX) // 4, dtype=torch.int32, device=dev)
    q.rmsnorm_mx_block_quantize_staged(hd, gd, 1e-6, img, eimg, residual=rd,
                                       residual_out=res_out2, norm_out=None)
    torch.cuda.synchronize()
    G.check_equal(G.bf16_host(res_out), res_ref, "residual_out (MX producer)")
    G.check_equal(G.bf16_host(res_out2), res_ref, "residual_out (staged MX producer)")
    G.check_equal(G.bf16_host(norm), norm_ref, "bf16 norm output")
    G.check_equal(codes.cpu().numpy(), codes_ref, "MX producer codes")
    G.check_equal(e8.cpu().numpy(), e8_ref, "MX producer exponents")
    G.check_equal(G.unstage(img, np.arange(T), HMAX), codes_ref, "staged MX producer codes")
    G.check_equal(G.unstage_exp(eimg, np.arange(T), HMAX), e8_ref, "staged MX producer exponents")


def test_projections_max_width():
    """ROW_MX packed and staged, MX staged: a 16384-long contraction into Q, K and V."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    p = G.custom_projection("hmax", T=T, H=HMAX, nq=2, nkv=1, d=64)
    inp = G.make_inputs(p)
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    X, ssq_ref = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, None, inp.bias,
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                head_dim=p.head_dim)
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    bias = G.bf16_dev(inp.bias, dev)
    kw = dict(num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, bias=bias)

    out = torch.full((p.T, p.I), float("nan"), dtype=torch.bfloat16, device=dev)
    ssq = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project(G.to_dev(inp.packed, dev), wp, out, H=p.H, ssq=ssq, workspace=ws, **kw)

    xd = G.to_dev(inp.x, dev)
    img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
    sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
    q.row_quantize_staged(xd, img, sc)
    out_s = torch.full((p.T, p.I), float("nan"), dtype=torch.bfloat16, device=dev)
    ssq_s = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws_s = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project_staged(img, sc, wp, out_s, H=p.H, ssq=ssq_s, workspace=ws_s, **kw)
    torch.cuda.synchronize()
    G.check_close(G.bf16_host(out), X, "packed ROW_MX X")
    G.check_ssq(ssq.cpu().numpy(), ssq_ref, "packed ROW_MX ssq")
    G.check_equal(G.bf16_host(out_s), G.bf16_host(out), "staged vs packed ROW_MX X")
    G.check_equal(ssq_s.cpu().numpy(), ssq.cpu().numpy(), "staged vs packed ROW_MX ssq")

    mcodes, me8 = oracle.mx_block_quantize(inp.x)
    Xm, ssq_m_ref = oracle.project(mcodes, None, inp.w_codes, inp.w_e8m0, None, inp.bias,
                                   num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                   head_dim=p.head_dim, a_e8m0=me8)
    eimg = torch.empty(q.qkv_act_exp_image_bytes(p.T, p.H) // 4, dtype=torch.int32, device=dev)
    q.mx_block_quantize_staged(xd, img, eimg)
    out_m = torch.full((p.T, p.I), float("nan"), dtype=torch.bfloat16, device=dev)
    q.qkv_mx_project_staged(img, eimg, wp, out_m, T=p.T, H=p.H, ssq=ssq_s, workspace=ws_s, **kw)
    torch.cuda.synchronize()
    G.check_close(G.bf16_host(out_m), Xm, "staged MX X")
    G.check_ssq(ssq_s.cpu().numpy(), ssq_m_ref, "staged MX ssq")
