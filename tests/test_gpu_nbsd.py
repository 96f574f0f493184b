"""GPU parity of the NBSd output layout ([QKV-CTE] "Interface": output_layout NBSd
[num_heads, B, S, d_head]; "Design 2)": the apply pass under NBSd), through the C ABI.

Expected values come from the oracle (``oracle.bsd_to_nbsd`` of the fp64 projection / pass-2
results); the NBSd output must also equal the same call's BSD output, re-indexed, bit for bit
(the arithmetic is the same, only the stores differ), and the sums of squares must be identical.
Every NBSd element must be written, and nothing past the array: the buffer is pre-filled with a
NaN sentinel and followed by a guard region.
"""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth
from oracle import codecs

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1            # a bf16 NaN no kernel produces
GUARD = 4096                 # elements after the array


def _lib():
    q = __import__("rope_mxfp8_qkv_amd")
    q.lib()
    return q


def _nbsd_buffer(nh, T, d, dev):
    import torch
    buf = torch.full((nh * T * d + GUARD,), SENTINEL, dtype=torch.int16, device=dev)
    return buf, buf[:nh * T * d].view(torch.bfloat16).view(nh, T, d)


def _check_sentinels(buf, n, what):
    import torch
    body = buf[:n]
    assert not torch.any(body == SENTINEL).item(), f"{what}: NBSd elements left unwritten"
    assert torch.all(buf[n:] == SENTINEL).item(), f"{what}: writes past the NBSd array"


def _project(q, inp, dev, layout, out, chan_scale=None):
    import torch
    p = inp.p
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    ssq = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    q.qkv_rowmx_project(G.to_dev(inp.packed, dev), wp, out, H=p.H, num_heads=p.num_heads,
                        num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                        channel_scale=None if chan_scale is None else G.to_dev(chan_scale, dev),
                        bias=G.bf16_dev(inp.bias, dev), ssq=ssq, workspace=ws, layout=layout)
    return ssq


PROJ_CASES = [
    ("C1", synth.CONFIGS[1].calls[0]),
    ("ragged-T-N", G.custom_projection("nt", T=300, H=512, nq=3, nkv=1, d=128)),
    ("d48-straddle", G.custom_projection("n48", T=260, H=256, nq=5, nkv=2, d=48)),
    ("single-seg", G.custom_projection("nss", T=257, H=1024, nq=5, nkv=0, d=128, rope=None)),
]


@pytest.mark.parametrize("name,p", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_projection_nbsd(name, p):
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(p)
    nh, d = p.I // p.head_dim, p.head_dim
    cs = (0.5 + np.random.default_rng(5).random(p.I)).astype(np.float32) if name == "ragged-T-N" else None
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    X, ssq_ref = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, cs, inp.bias,
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=d)
    buf, out_n = _nbsd_buffer(nh, p.T, d, dev)
    ssq_n = _project(q, inp, dev, q.LAYOUT_NBSD, out_n, chan_scale=cs)
    out_b = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev)
    ssq_b = _project(q, inp, dev, q.LAYOUT_BSD, out_b, chan_scale=cs)
    torch.cuda.synchronize()
    _check_sentinels(buf, nh * p.T * d, name)
    got = G.bf16_host(out_n)
    G.check_close(got, oracle.bsd_to_nbsd(X, d), f"{name} NBSd X")
    G.check_equal(got, oracle.bsd_to_nbsd(G.bf16_host(out_b), d), f"{name} NBSd == BSD re-indexed")
    G.check_equal(ssq_n.cpu().numpy(), ssq_b.cpu().numpy(), f"{name} sums identical")
    G.check_ssq(ssq_n.cpu().numpy(), ssq_ref, f"{name} sums")


NR_CASES = [
    ("C1-norm-rope", synth.CONFIGS[1].calls[0], None),
    ("norm-only-d128", G.custom_projection("nno", T=130, H=256, nq=3, nkv=2, d=128, rope=None), None),
    ("rope-only-d64", G.custom_projection("nro", T=70, H=256, nq=2, nkv=2, d=64), 4),
    ("k-only", G.custom_projection("nko", T=50, H=256, nq=2, nkv=2, d=64, rope=None), 2),
    ("single-seg-d48", G.custom_projection("nsq", T=90, H=256, nq=4, nkv=0, d=48, rope=None), None),
    ("d256", G.custom_projection("n256", T=33, H=256, nq=2, nkv=1, d=256), None),
]


@pytest.mark.parametrize("name,p,flags", NR_CASES, ids=[c[0] for c in NR_CASES])
def test_norm_rope_nbsd_standalone(name, p, flags):
    """Pass 2 alone in NBSd on the oracle's rounded pass-1 output and its sums; V heads (and K
    heads when K is untouched) bit-identical."""
    import dataclasses
    import torch
    q = _lib()
    dev = G.torch_dev()
    fl = G.flags_of(p) if flags is None else flags
    d, nh = p.head_dim, p.I // p.head_dim
    rng = np.random.default_rng(12)
    bits = codecs.f64_to_bf16(rng.standard_normal((p.T, p.I)) * 1.5)
    ssq = oracle.segment_ssq(codecs.bf16_to_f64(bits), p.num_heads, p.num_kv_heads, d).astype(np.float32)
    gq, gk = synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k")
    cos, sin = synth.rope_tables(dataclasses.replace(p, rope="1d"))
    use_gk = gk if fl & q.NORM_K else None
    ref = oracle.norm_rope(bits, ssq, gq, use_gk, cos, sin, num_heads=p.num_heads,
                           num_kv_heads=p.num_kv_heads, head_dim=d, eps=1e-6, flags=fl)
    bits_n = oracle.bsd_to_nbsd(bits, d)
    t = G.bf16_dev(bits_n, dev)
    q.qk_norm_rope_apply(t, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=d,
                         eps=1e-6, flags=fl, ssq=G.to_dev(ssq, dev),
                         q_gamma=G.bf16_dev(gq, dev) if fl & q.NORM_Q else None,
                         k_gamma=G.bf16_dev(use_gk, dev) if use_gk is not None else None,
                         cos=G.to_dev(cos, dev) if fl & q.FUSED_ROPE else None,
                         sin=G.to_dev(sin, dev) if fl & q.FUSED_ROPE else None,
                         layout=q.LAYOUT_NBSD)
    torch.cuda.synchronize()
    got = G.bf16_host(t)
    nqk = p.num_heads + p.num_kv_heads
    G.check_equal(got[nqk:], bits_n[nqk:], f"{name} V heads untouched")
    G.check_close(got, oracle.bsd_to_nbsd(ref, d), f"{name} Q/K heads")
    if not (fl & q.NORM_K) and not (fl & q.FUSED_ROPE):
        G.check_equal(got[p.num_heads:nqk], bits_n[p.num_heads:nqk], f"{name} K untouched")
    assert nh == got.shape[0]


E2E_CASES = [
    ("self-attn-1d", G.custom_projection("ne", T=600, H=512, nq=4, nkv=4, d=128)),
    ("cross-attn-q", G.custom_projection("nxq", T=700, H=1024, nq=8, nkv=0, d=128, rope=None)),
]


@pytest.mark.parametrize("name,p", E2E_CASES, ids=[c[0] for c in E2E_CASES])
def test_end_to_end_nbsd(name, p):
    """Pass 1 -> pass 2 in NBSd: bit-identical to the BSD chain re-indexed, and within the
    end-to-end bound of the fp64 oracle chain."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(p)
    d, nh = p.head_dim, p.I // p.head_dim
    fl = G.flags_of(p)
    outs = {}
    for layout in (q.LAYOUT_NBSD, q.LAYOUT_BSD):
        out = (torch.empty((nh, p.T, d), dtype=torch.bfloat16, device=dev) if layout == q.LAYOUT_NBSD
               else torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev))
        ssq = _project(q, inp, dev, layout, out)
        q.qk_norm_rope_apply(out, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=d,
                             eps=1e-6, flags=fl, ssq=ssq,
                             q_gamma=G.bf16_dev(inp.gq, dev) if fl & q.NORM_Q else None,
                             k_gamma=G.bf16_dev(inp.gk, dev) if fl & q.NORM_K else None,
                             cos=G.to_dev(inp.cos, dev) if fl & q.FUSED_ROPE else None,
                             sin=G.to_dev(inp.sin, dev) if fl & q.FUSED_ROPE else None,
                             layout=layout)
        outs[layout] = out
    torch.cuda.synchronize()
    got = G.bf16_host(outs[q.LAYOUT_NBSD])
    G.check_equal(got, oracle.bsd_to_nbsd(G.bf16_host(outs[q.LAYOUT_BSD]), d), f"{name} == BSD chain")
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    X, ssq_ref = oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, None, inp.bias,
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=d)
    ref = oracle.norm_rope(None, ssq_ref, inp.gq, inp.gk if fl & q.NORM_K else None,
                           inp.cos if fl & q.FUSED_ROPE else None,
                           inp.sin if fl & q.FUSED_ROPE else None, num_heads=p.num_heads,
                           num_kv_heads=p.num_kv_heads, head_dim=d, eps=1e-6, flags=fl, values=X)
    extra = G.propagated_bound(X, ssq_ref, inp.gq, inp.gk, p.num_heads, p.num_kv_heads, d, 1e-6,
                               bool(fl & q.NORM_Q), bool(fl & q.NORM_K), bool(fl & q.FUSED_ROPE))
    G.check_close(got, oracle.bsd_to_nbsd(ref, d), f"{name} end-to-end",
                  extra=oracle.bsd_to_nbsd(extra, d))
