"""GPU parity of the MX block-32 activation path ([RMSNORM-MX] qmx_output_dtype and
emit_norm_bf16; [QKV-CTE] projection fed with per-block activation exponents) against the CPU
oracle: the encoders bit for bit, the projection within the bf16 tolerance, on shapes with
ragged T and I, GQA, single-segment calls, both output layouts and a channel scale.  The
activations get a different power-of-two scale in every 32-element block, so each of the eight
blocks of a 256-byte K superstep carries its own exponent and a wrong pairing of exponents with
K-blocks changes the result by powers of two."""
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


def _blocky_activation(T, H, seed, spread=2):
    """N(0,1) rows with a random power of two (2^-spread .. 2^spread) per 32-element block and
    per-row gains in [0.5, 2], a zero block and a tiny block.  The spread keeps the exponents of
    neighbouring blocks apart (a misplaced exponent is off by a power of two) without the heavy
    cancellation that wide spreads produce: one FP8 MFMA sums its 64 products only to a small
    fraction of their absolute sum, so outputs that cancel below that fraction fall outside the
    plain bf16 tolerance on any input encoding.  The wide spreads (2^+-6 per block, row gains
    10^+-2) are checked in test_gpu_accumulation.py against the tolerance plus that bound."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= np.ldexp(1.0, rng.integers(-spread, spread + 1, (T, H // 32))).repeat(32, axis=1).astype(np.float32)
    x *= rng.uniform(0.5, 2.0, (T, 1)).astype(np.float32)
    x[0, 32:64] = 0.0
    if T > 1:
        x[1, :32] *= np.float32(1e-30)
    return x.astype(np.float32)


# ----------------------------------------------------------------------------------------------
# encoders (bit-exact)
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,H", [("f32", 2080), ("bf16", 2080), ("f32", 5120)])
def test_mx_block_quantize_bit_exact(dtype, H):
    import torch
    q = _lib()
    dev = G.torch_dev()
    T = 129
    x = _blocky_activation(T, H, 11, spread=6)
    x *= np.float32(50.0)
    x[5, :7] = -0.0                                   # signed zeros inside a non-zero block
    x[6, 40] = 1e6                                    # saturating element of its block
    # blocks at the E8M0 floor (largest magnitude below 2^-119, fp32 subnormals, -0.0; in bf16
    # the subnormal ones stay subnormal): exponent 0
    fb = G.floor_blocks(np.random.default_rng(12))
    for j, blk in enumerate(fb):
        x[10 + j, 64:96] = blk
    if dtype == "bf16":
        bits = synth.to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(bits)
        xd = G.bf16_dev(bits, dev)
    else:
        xd = G.to_dev(x, dev)
    codes_ref, e8_ref = oracle.mx_block_quantize(x)
    assert (e8_ref[10:10 + len(fb), 2] == 0).sum() >= 6   # the clamp is reached
    codes = torch.empty((T, H), dtype=torch.uint8, device=dev)
    e8 = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    q.mx_block_quantize(xd, codes, e8)
    torch.cuda.synchronize()
    G.check_equal(e8.cpu().numpy(), e8_ref, "exponents")
    G.check_equal(codes.cpu().numpy(), codes_ref, "codes")


@pytest.mark.parametrize("with_res,emit,Hu", [(True, True, 0), (False, True, 0), (True, False, 4000)])
def test_rmsnorm_mx_block_bit_exact(with_res, emit, Hu):
    import torch
    q = _lib()
    dev = G.torch_dev()
    T, H = 300, 5120
    hid, res, gam = synth.producer_inputs(78, T, H)
    if Hu:
        hid[:, Hu:] = 0
        res[:, Hu:] = 0
    res_ref, codes_ref, e8_ref, norm_ref, _ = oracle.rmsnorm_mx(hid, res if with_res else None,
                                                                gam, 1e-6, Hu)
    codes = torch.empty((T, H), dtype=torch.uint8, device=dev)
    e8 = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if with_res else None
    norm = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if emit else None
    q.rmsnorm_mx_block_quantize(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, codes, e8,
                                residual=G.bf16_dev(res, dev) if with_res else None,
                                residual_out=res_out, norm_out=norm, unpadded_h=Hu)
    torch.cuda.synchronize()
    if with_res:
        G.check_equal(G.bf16_host(res_out), res_ref, "residual_out")
    if emit:
        G.check_equal(G.bf16_host(norm), norm_ref, "bf16 norm output")
    G.check_equal(e8.cpu().numpy(), e8_ref, "exponents")
    G.check_equal(codes.cpu().numpy(), codes_ref, "codes")


# ----------------------------------------------------------------------------------------------
# pass 1 with MX activations
# ----------------------------------------------------------------------------------------------

MX_CASES = [
    ("C1", synth.CONFIGS[1].calls[0], "bsd", False),
    ("ragged-T-N", G.custom_projection("mrn", T=300, H=512, nq=3, nkv=1, d=128), "bsd", True),
    ("gqa-d64", G.custom_projection("mg", T=129, H=768, nq=4, nkv=2, d=64), "bsd", False),
    ("single-seg", G.custom_projection("mss", T=257, H=1024, nq=5, nkv=0, d=128, rope=None), "bsd", False),
    ("T1", G.custom_projection("mt1", T=1, H=256, nq=2, nkv=2, d=64), "bsd", False),
    ("nbsd-ragged", G.custom_projection("mnb", T=300, H=512, nq=3, nkv=1, d=48), "nbsd", True),
    ("ragged-H", G.custom_projection("mrh", T=200, H=352, nq=2, nkv=2, d=64), "bsd", False),
    ("H96", G.custom_projection("mh96", T=70, H=96, nq=1, nkv=1, d=64), "bsd", False),
]


def run_mx_projection(q, p, codes, e8, w_codes, w_e8m0, bias, dev, layout="bsd", cs=None):
    import torch
    wp = q.prepare_weight(G.to_dev(w_codes, dev), G.to_dev(w_e8m0, dev), p.H, p.I)
    shape = (p.I // p.head_dim, p.T, p.head_dim) if layout == "nbsd" else (p.T, p.I)
    out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ssq = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qkv_mx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    q.qkv_mx_project(G.to_dev(codes, dev), G.to_dev(e8, dev), wp, out, H=p.H,
                     num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                     channel_scale=None if cs is None else G.to_dev(cs, dev),
                     bias=None if bias is None else G.bf16_dev(bias, dev), ssq=ssq, workspace=ws,
                     layout=q.LAYOUT_NBSD if layout == "nbsd" else q.LAYOUT_BSD)
    return out, ssq


@pytest.mark.parametrize("name,p,layout,chan", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mx_projection_parity(name, p, layout, chan):
    import torch
    q = _lib()
    dev = G.torch_dev()
    x = _blocky_activation(p.T, p.H, 21)
    codes, e8 = oracle.mx_block_quantize(x)
    w_codes, w_e8m0 = oracle.mx_weight_quantize(synth.weight(p))
    bias = None if name == "single-seg" else synth.bias_bf16(p)
    rng = np.random.default_rng(5)
    cs = (0.5 + rng.random(p.I)).astype(np.float32) if chan else None
    X, ssq_ref = oracle.project(codes, None, w_codes, w_e8m0, cs, bias, num_heads=p.num_heads,
                                num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, a_e8m0=e8)
    out, ssq = run_mx_projection(q, p, codes, e8, w_codes, w_e8m0, bias, dev, layout, cs)
    torch.cuda.synchronize()
    got = G.bf16_host(out)
    if layout == "nbsd":
        got = oracle.nbsd_to_bsd(got)
    G.check_close(got, X, f"{name} X")
    G.check_ssq(ssq.cpu().numpy(), ssq_ref, f"{name} ssq")


def test_mx_projection_strided_rows():
    """Row strides beyond H (codes padded by 52 bytes: rows only 4-byte aligned; exponents
    padded by 3 bytes)."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    p = G.custom_projection("mst", T=200, H=512, nq=2, nkv=1, d=128)
    x = _blocky_activation(p.T, p.H, 31)
    codes, e8 = oracle.mx_block_quantize(x)
    cpad = np.zeros((p.T, p.H + 52), np.uint8)
    cpad[:, :p.H] = codes
    cpad[:, p.H:] = 0x7F                            # NaN codes outside the rows: never read
    epad = np.full((p.T, p.H // 32 + 3), 0xFF, np.uint8)
    epad[:, :p.H // 32] = e8
    w_codes, w_e8m0 = oracle.mx_weight_quantize(synth.weight(p))
    bias = synth.bias_bf16(p)
    X, ssq_ref = oracle.project(codes, None, w_codes, w_e8m0, None, bias, num_heads=p.num_heads,
                                num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, a_e8m0=e8)
    out, ssq = run_mx_projection(q, p, cpad, epad, w_codes, w_e8m0, bias, dev)
    torch.cuda.synchronize()
    G.check_close(G.bf16_host(out), X, "strided X")
    G.check_ssq(ssq.cpu().numpy(), ssq_ref, "strided ssq")


def test_mx_end_to_end_c1():
    """Producer (residual add + RMSNorm + MX block-32) -> MX projection -> norm + RoPE."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    p = synth.CONFIGS[1].calls[0]
    T, H, I = p.T, p.H, p.I
    hid, res, gam = synth.producer_inputs(1, T, H)
    w_codes, w_e8m0 = oracle.mx_weight_quantize(synth.weight(p))
    bias, gq, gk = synth.bias_bf16(p), synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k")
    cos, sin = synth.rope_tables(p)
    codes = torch.empty((T, H), dtype=torch.uint8, device=dev)
    e8 = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_block_quantize(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, codes, e8,
                                residual=G.bf16_dev(res, dev), residual_out=res_out)
    wp = q.prepare_weight(G.to_dev(w_codes, dev), G.to_dev(w_e8m0, dev), H, I)
    out = torch.empty((T, I), dtype=torch.bfloat16, device=dev)
    ssq = torch.empty((T, 2), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qkv_mx_workspace_bytes(T, H, I), dtype=torch.uint8, device=dev)
    q.qkv_mx_project(codes, e8, wp, out, H=H, num_heads=p.num_heads,
                     num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, bias=G.bf16_dev(bias, dev),
                     ssq=ssq, workspace=ws)
    q.qk_norm_rope_apply(out, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                         head_dim=p.head_dim, eps=1e-6, flags=G.flags_of(p), ssq=ssq,
                         q_gamma=G.bf16_dev(gq, dev), k_gamma=G.bf16_dev(gk, dev),
                         cos=G.to_dev(cos, dev), sin=G.to_dev(sin, dev))
    torch.cuda.synchronize()
    _, c_ref, e_ref, _, _ = oracle.rmsnorm_mx(hid, res, gam, 1e-6)
    G.check_equal(codes.cpu().numpy(), c_ref, "producer codes")
    G.check_equal(e8.cpu().numpy(), e_ref, "producer exponents")
    X, ssq_ref = oracle.project(c_ref, None, w_codes, w_e8m0, None, bias, num_heads=p.num_heads,
                                num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, a_e8m0=e_ref)
    ref = oracle.norm_rope(None, ssq_ref, gq, gk, cos, sin, num_heads=p.num_heads,
                           num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, eps=1e-6,
                           flags=G.flags_of(p), values=X)
    bound = G.propagated_bound(X, ssq_ref, gq, gk, p.num_heads, p.num_kv_heads, p.head_dim, 1e-6,
                               True, True, True)
    G.check_close(G.bf16_host(out), ref, "end-to-end", extra=bound)
