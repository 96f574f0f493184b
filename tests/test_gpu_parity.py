"""GPU parity: every entry point of the C ABI against the CPU oracle on the same seeded inputs.

Inputs come from ``synth`` and, where an encoding is needed, from the oracle; expected values come
from the oracle only.  Shapes span several tiles with ragged tails (T not a multiple of 256, I not
a multiple of 256, H not a multiple of the 256-byte K superstep), GQA head counts, head_dim 64
and 128, single-segment calls and T = 1.
"""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth
from oracle import codecs

pytestmark = pytest.mark.gpu


def _lib():
    import rope_mxfp8_qkv_amd as q
    q.lib()
    return q


# ----------------------------------------------------------------------------------------------
# encoders (bit-exact)
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("H,I", [(256, 384), (96, 48), (5120, 640)])
def test_mx_weight_quantize_bit_exact(H, I):
    import torch
    q = _lib()
    dev = G.torch_dev()
    rng = np.random.default_rng(H + I)
    w = (0.02 * rng.standard_normal((H, I))).astype(np.float32)
    w[:32, 0] = 0.0                       # zero block
    w[32:64, 1] *= 1e-30                  # tiny block (amax ~ 2^-104: exponent 14)
    w[5, 2] = -3.0                        # saturating element
    # blocks at the E8M0 floor (largest magnitude below 2^-119, fp32 subnormals, -0.0): the
    # exponent clamps to 0; the oracle's exponents for them are pinned in rationals on the CPU
    fb = G.floor_blocks(rng)
    for j, blk in enumerate(fb):
        w[64:96, 3 + j] = blk
    ref_e8 = oracle.mx_weight_quantize(w)[1]
    assert (ref_e8[2, 3:3 + len(fb)] == 0).sum() >= 6   # the clamp is reached
    codes_ref, e8_ref = oracle.mx_weight_quantize(w)
    codes = torch.empty((H // 4, I, 4), dtype=torch.uint8, device=dev)
    e8 = torch.empty((H // 32, I), dtype=torch.uint8, device=dev)
    q.mx_weight_quantize(G.to_dev(w, dev), codes, e8)
    torch.cuda.synchronize()
    G.check_equal(e8.cpu().numpy(), e8_ref, "e8m0")
    G.check_equal(codes.cpu().numpy(), codes_ref, "codes")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_quantize_bit_exact(dtype):
    import torch
    q = _lib()
    dev = G.torch_dev()
    rng = np.random.default_rng(7)
    T, H = 129, 2080
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
    ref = oracle.rowmx_quantize(x)
    out = torch.empty((T, H + 4), dtype=torch.uint8, device=dev)
    q.row_quantize_packed(xd, out)
    torch.cuda.synchronize()
    G.check_equal(out.cpu().numpy(), ref, "ROW_MX rows")


@pytest.mark.parametrize("with_res,Hu", [(True, 0), (False, 0), (True, 4000)])
def test_rmsnorm_quantize_bit_exact(with_res, Hu):
    import torch
    q = _lib()
    dev = G.torch_dev()
    T, H = 300, 5120
    hid, res, gam = synth.producer_inputs(77, T, H)
    if Hu:
        hid[:, Hu:] = 0
        res[:, Hu:] = 0
    res_ref, packed_ref, _ = oracle.rmsnorm_rowmx(hid, res if with_res else None, gam, 1e-6, Hu)
    packed = torch.empty((T, H + 4), dtype=torch.uint8, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if with_res else None
    q.rmsnorm_mx_quantize(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, packed,
                          residual=G.bf16_dev(res, dev) if with_res else None,
                          residual_out=res_out, unpadded_h=Hu)
    torch.cuda.synchronize()
    if with_res:
        G.check_equal(G.bf16_host(res_out), res_ref, "residual_out")
    G.check_equal(packed.cpu().numpy(), packed_ref, "packed rows")


# ----------------------------------------------------------------------------------------------
# pass 1
# ----------------------------------------------------------------------------------------------

PROJ_CASES = [
    ("C1", synth.CONFIGS[1].calls[0]),
    ("T1", G.custom_projection("t1", T=1, H=256, nq=2, nkv=2, d=64)),
    ("gqa-ragged", G.custom_projection("gqa", T=129, H=96, nq=4, nkv=2, d=64)),
    ("ragged-N", G.custom_projection("rn", T=300, H=512, nq=3, nkv=1, d=128)),
    ("single-seg", G.custom_projection("ss", T=257, H=1024, nq=5, nkv=0, d=128, rope=None)),
]


def run_projection(q, inp: G.ProjInputs, dev, chan_scale=None, with_ssq=True):
    import torch
    p = inp.p
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    out = torch.full((p.T, p.I), float("nan"), dtype=torch.bfloat16, device=dev)
    ssq = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev) if with_ssq else None
    ws = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project(G.to_dev(inp.packed, dev), wp, out, H=p.H, num_heads=p.num_heads,
                        num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                        channel_scale=None if chan_scale is None else G.to_dev(chan_scale, dev),
                        bias=None if inp.bias is None else G.bf16_dev(inp.bias, dev), ssq=ssq,
                        workspace=ws)
    return out, ssq, wp


@pytest.mark.parametrize("name,p", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_projection_parity(name, p):
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(p)
    rng = np.random.default_rng(3)
    cs = (0.5 + rng.random(p.I)).astype(np.float32) if name == "ragged-N" else None
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    X, ssq_ref = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, cs, inp.bias,
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                head_dim=p.head_dim)
    out, ssq, _ = run_projection(q, inp, dev, chan_scale=cs)
    torch.cuda.synchronize()
    G.check_close(G.bf16_host(out), X, f"{name} X")
    G.check_ssq(ssq.cpu().numpy(), ssq_ref, f"{name} ssq")


def test_projection_separate_scale_buffer_and_no_bias():
    """Codes and scales in separate buffers (row stride H), no bias, no sums requested."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    p = G.custom_projection("sep", T=200, H=384, nq=2, nkv=1, d=64)
    inp = G.make_inputs(p, with_bias=False)
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    X, _ = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, None, None, num_heads=2,
                          num_kv_heads=1, head_dim=64)
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    out = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project(G.to_dev(np.ascontiguousarray(codes), dev), wp, out, H=p.H, num_heads=2,
                        num_kv_heads=1, head_dim=64, a_scales=G.to_dev(sA, dev), a_row_stride=p.H,
                        a_scale_stride=4, workspace=ws)
    torch.cuda.synchronize()
    G.check_close(G.bf16_host(out), X, "separate-scale X")


def test_projection_deterministic():
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(G.custom_projection("det", T=600, H=1024, nq=4, nkv=4, d=128))
    o1, s1, _ = run_projection(q, inp, dev)
    o2, s2, _ = run_projection(q, inp, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1, s2)


# ----------------------------------------------------------------------------------------------
# pass 2
# ----------------------------------------------------------------------------------------------

NR_CASES = [
    ("C1-norm-rope", synth.CONFIGS[1].calls[0], None),
    ("norm-only", G.custom_projection("no", T=130, H=256, nq=3, nkv=2, d=128, rope=None), None),
    ("rope-only", G.custom_projection("ro", T=70, H=256, nq=2, nkv=2, d=64), 4),
    ("k-only", G.custom_projection("ko", T=50, H=256, nq=2, nkv=2, d=64, rope=None), 2),
    ("single-seg", G.custom_projection("sq", T=90, H=256, nq=4, nkv=0, d=64, rope=None), None),
    # head widths whose d / 16 chunk lanes do not divide the 64 lanes of a token (idle lanes),
    # the narrowest head (64 head groups per token) and the widest (one group per token)
    ("d16", G.custom_projection("b16", T=77, H=256, nq=4, nkv=2, d=16), None),
    ("d48", G.custom_projection("b48", T=130, H=256, nq=5, nkv=3, d=48), None),
    ("d80-gqa", G.custom_projection("b80", T=61, H=256, nq=6, nkv=2, d=80), None),
    ("d256", G.custom_projection("b256", T=40, H=256, nq=2, nkv=1, d=256), None),
    ("d1024", G.custom_projection("b1k", T=9, H=256, nq=2, nkv=1, d=1024), None),
]


@pytest.mark.parametrize("name,p,flags", NR_CASES, ids=[c[0] for c in NR_CASES])
def test_norm_rope_standalone(name, p, flags):
    """Pass 2 alone on identical inputs: the oracle's rounded pass-1 output and its sums."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    fl = G.flags_of(p) if flags is None else flags
    rng = np.random.default_rng(11)
    X = rng.standard_normal((p.T, p.I)) * 1.5
    bits = codecs.f64_to_bf16(X)
    xv = codecs.bf16_to_f64(bits)
    ssq = oracle.segment_ssq(xv, p.num_heads, p.num_kv_heads, p.head_dim).astype(np.float32)
    gq, gk = synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k")
    cos, sin = synth.rope_tables(dataclassesreplace(p, rope="1d"))
    use_gk = gk if fl & q.NORM_K else None
    ref = oracle.norm_rope(bits, ssq, gq, use_gk, cos, sin, num_heads=p.num_heads,
                           num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, eps=1e-6, flags=fl)
    t = G.bf16_dev(bits, dev)
    q.qk_norm_rope_apply(t, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                         head_dim=p.head_dim, eps=1e-6, flags=fl, ssq=G.to_dev(ssq, dev),
                         q_gamma=G.bf16_dev(gq, dev) if fl & q.NORM_Q else None,
                         k_gamma=G.bf16_dev(use_gk, dev) if use_gk is not None else None,
                         cos=G.to_dev(cos, dev) if fl & q.FUSED_ROPE else None,
                         sin=G.to_dev(sin, dev) if fl & q.FUSED_ROPE else None)
    torch.cuda.synchronize()
    got = G.bf16_host(t)
    seg = (p.num_heads + p.num_kv_heads) * p.head_dim
    G.check_equal(got[:, seg:], bits[:, seg:], f"{name} V untouched")
    G.check_close(got, ref, f"{name} Q/K")
    if not (fl & q.NORM_K) and not (fl & q.FUSED_ROPE):
        G.check_equal(got[:, p.Iq:seg], bits[:, p.Iq:seg], f"{name} K untouched")


def dataclassesreplace(p, **kw):
    import dataclasses
    return dataclasses.replace(p, **kw)


# ----------------------------------------------------------------------------------------------
# end to end (pass 1 -> pass 2) at the tiny and the S=4096 self-attention shapes
# ----------------------------------------------------------------------------------------------

def end_to_end(p: synth.Projection, rows=None):
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(p)
    out, ssq, _ = run_projection(q, inp, dev)
    fl = G.flags_of(p)
    v_before = None
    seg = (p.num_heads + p.num_kv_heads) * p.head_dim
    if seg < p.I:
        v_before = out[:, seg:].clone()
    q.qk_norm_rope_apply(out, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                         head_dim=p.head_dim, eps=1e-6, flags=fl, ssq=ssq,
                         q_gamma=G.bf16_dev(inp.gq, dev) if fl & q.NORM_Q else None,
                         k_gamma=G.bf16_dev(inp.gk, dev) if fl & q.NORM_K else None,
                         cos=G.to_dev(inp.cos, dev) if inp.cos is not None else None,
                         sin=G.to_dev(inp.sin, dev) if inp.sin is not None else None)
    torch.cuda.synchronize()
    if v_before is not None:
        assert torch.equal(out[:, seg:].view(torch.int16), v_before.view(torch.int16))
    rows = np.arange(p.T) if rows is None else rows
    codes, sA = oracle.rowmx_unpack(inp.packed[rows], p.H)
    X, ssq_ref = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, None, inp.bias,
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                head_dim=p.head_dim)
    cos = inp.cos[rows] if inp.cos is not None else None
    sin = inp.sin[rows] if inp.sin is not None else None
    ref = oracle.norm_rope(None, ssq_ref, inp.gq, inp.gk if fl & q.NORM_K else None, cos, sin,
                           num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                           head_dim=p.head_dim, eps=1e-6, flags=fl, values=X)
    extra = G.propagated_bound(X, ssq_ref, inp.gq, inp.gk, p.num_heads, p.num_kv_heads,
                               p.head_dim, 1e-6, bool(fl & q.NORM_Q), bool(fl & q.NORM_K),
                               bool(fl & q.FUSED_ROPE))
    got = G.bf16_host(out)[rows]
    G.check_close(got, ref, f"{p.name} end-to-end", extra=extra)
    G.check_ssq(ssq.cpu().numpy()[rows], ssq_ref, f"{p.name} ssq")


def test_end_to_end_c1():
    end_to_end(synth.CONFIGS[1].calls[0])


def test_end_to_end_c2_sampled_rows():
    p = synth.CONFIGS[2].calls[0]
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095], rng.integers(0, p.T, 120)]))
    end_to_end(p, rows)
