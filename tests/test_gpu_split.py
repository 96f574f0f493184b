"""GPU parity of the split contraction (projections with at most 128 output tiles: the K range
is cut into chunks, each (tile, chunk) unit stores fp32 partial sums to a workspace plane, and
a per-token pass adds the planes and applies the epilogue, BSD or NBSd store), and of the
unsplit path at small ragged sizes (more than 128 tiles).

qkvmx_projection_k_chunks tells which path a shape takes; the tests assert it, so a change of
the split policy cannot silently move a case to the other path.
"""
import numpy as np
import pytest

import gpu_common as G
import oracle

pytestmark = pytest.mark.gpu


def _lib():
    import rope_mxfp8_qkv_amd as q
    q.lib()
    return q


# 512 context tokens x 40 channel tiles -> 3-way factor; 7 supersteps -> chunks of 3, 3, 1
UNEVEN = G.custom_projection("split-uneven", T=512, H=1792, nq=16, nkv=12, d=128)
# 2 x 3 tiles (ragged T and I) -> 3-way factor; 2 supersteps -> 2 chunks of 1
SMALL = G.custom_projection("split-small", T=300, H=512, nq=3, nkv=1, d=128)
# 5 x 26 = 130 tiles (ragged T and I) -> no split, at a size the oracle finishes quickly
UNSPLIT = G.custom_projection("unsplit-130", T=1100, H=512, nq=45, nkv=3, d=128)


def _oracle_rowmx(inp, cs=None, bias=True):
    p = inp.p
    codes, sA = oracle.rowmx_unpack(inp.packed, p.H)
    return oracle.project(codes, sA, inp.w_codes, inp.w_e8m0, cs, inp.bias if bias else None,
                          num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                          head_dim=p.head_dim)


def _run(q, inp, dev, path, cs=None, bias=True, with_ssq=True, nbsd=False):
    """One projection call on `path` (rowmx-packed, rowmx-staged, mx-natural, mx-staged)."""
    import torch
    p = inp.p
    wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I)
    shape = (p.I // p.head_dim, p.T, p.head_dim) if nbsd else (p.T, p.I)
    out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ssq = torch.full((p.T, 2), float("nan"), dtype=torch.float32, device=dev) if with_ssq else None
    kw = dict(num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
              channel_scale=None if cs is None else G.to_dev(cs, dev),
              bias=G.bf16_dev(inp.bias, dev) if bias else None, ssq=ssq,
              layout=q.LAYOUT_NBSD if nbsd else q.LAYOUT_BSD)
    xd = G.to_dev(inp.x, dev)
    if path == "rowmx-packed":
        ws = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
        q.qkv_rowmx_project(G.to_dev(inp.packed, dev), wp, out, H=p.H, workspace=ws, **kw)
    elif path == "rowmx-staged":
        img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
        sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
        q.row_quantize_staged(xd, img, sc)
        ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
        q.qkv_rowmx_project_staged(img, sc, wp, out, H=p.H, workspace=ws, **kw)
    elif path == "mx-natural":
        codes = torch.empty((p.T, p.H), dtype=torch.uint8, device=dev)
        e8 = torch.empty((p.T, p.H // 32), dtype=torch.uint8, device=dev)
        q.mx_block_quantize(xd, codes, e8)
        ws = torch.empty(q.qkv_mx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
        q.qkv_mx_project(codes, e8, wp, out, H=p.H, workspace=ws, **kw)
    else:
        img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
        eimg = torch.empty(q.qkv_act_exp_image_bytes(p.T, p.H) // 4, dtype=torch.int32, device=dev)
        q.mx_block_quantize_staged(xd, img, eimg)
        ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
        q.qkv_mx_project_staged(img, eimg, wp, out, T=p.T, H=p.H, workspace=ws, **kw)
    return out, ssq


def _ref(inp, path, cs=None, bias=True):
    if path.startswith("rowmx"):
        return _oracle_rowmx(inp, cs, bias)
    p = inp.p
    codes, e8 = oracle.mx_block_quantize(inp.x)
    return oracle.project(codes, None, inp.w_codes, inp.w_e8m0, cs, inp.bias if bias else None,
                          num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                          head_dim=p.head_dim, a_e8m0=e8)


PATHS = ["rowmx-packed", "rowmx-staged", "mx-natural", "mx-staged"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("p,chunks", [(UNEVEN, 3), (SMALL, 2), (UNSPLIT, 1)],
                         ids=["uneven-3-chunks", "small-2-chunks", "unsplit-130-tiles"])
def test_projection_paths_match_oracle(p, chunks, path):
    import torch
    q = _lib()
    dev = G.torch_dev()
    assert q.projection_k_chunks(p.T, p.H, p.I) == chunks
    inp = G.make_inputs(p)
    X, ssq_ref = _ref(inp, path)
    out, ssq = _run(q, inp, dev, path)
    torch.cuda.synchronize()
    G.check_close(G.bf16_host(out), X, f"{p.name} {path} X")
    G.check_ssq(ssq.cpu().numpy(), ssq_ref, f"{p.name} {path} ssq")


@pytest.mark.parametrize("p", [UNEVEN, SMALL], ids=["uneven", "small"])
def test_split_staged_equals_packed(p):
    """Same codes and scales through the two hand-overs: identical bytes (ROW_MX and MX)."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(p)
    for a, b in (("rowmx-packed", "rowmx-staged"), ("mx-natural", "mx-staged")):
        o1, s1 = _run(q, inp, dev, a)
        o2, s2 = _run(q, inp, dev, b)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{a} vs {b}"
        assert torch.equal(s1, s2), f"{a} vs {b} ssq"


@pytest.mark.parametrize("path", ["rowmx-packed", "mx-staged"])
def test_split_epilogue_variants(path):
    """Channel scale without bias, and no sums requested, on the split path."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    p = SMALL
    inp = G.make_inputs(p)
    cs = (0.5 + np.random.default_rng(9).random(p.I)).astype(np.float32)
    X, _ = _ref(inp, path, cs=cs, bias=False)
    out, ssq = _run(q, inp, dev, path, cs=cs, bias=False, with_ssq=False)
    torch.cuda.synchronize()
    assert ssq is None
    G.check_close(G.bf16_host(out), X, f"{path} channel scale, no bias")


def test_split_deterministic_and_repeatable():
    import torch
    q = _lib()
    dev = G.torch_dev()
    inp = G.make_inputs(UNEVEN)
    o1, s1 = _run(q, inp, dev, "rowmx-staged")
    o2, s2 = _run(q, inp, dev, "rowmx-staged")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("path", ["rowmx-packed", "mx-staged"])
@pytest.mark.parametrize("p", [UNEVEN, SMALL], ids=["uneven", "small"])
def test_split_nbsd_equals_bsd(p, path):
    """The NBSd store of the split pass holds exactly the BSD result, re-laid per head."""
    import torch
    q = _lib()
    dev = G.torch_dev()
    assert q.projection_k_chunks(p.T, p.H, p.I, q.LAYOUT_NBSD) == q.projection_k_chunks(p.T, p.H, p.I)
    inp = G.make_inputs(p)
    o1, s1 = _run(q, inp, dev, path)
    o2, s2 = _run(q, inp, dev, path, nbsd=True)
    torch.cuda.synchronize()
    G.check_equal(oracle.nbsd_to_bsd(G.bf16_host(o2)), G.bf16_host(o1), f"{path} NBSd vs BSD")
    assert torch.equal(s1, s2)
