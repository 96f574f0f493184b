"""A whole step (producer -> projection -> across-heads norm + RoPE) captured into a HIP graph
and replayed.  The entry points launch kernels only (counters are cleared by a kernel, never by
a memset), so a caller may capture them; every replay must give the eager step's bytes, also
after the inputs were rewritten in place between replays (the graph reads the live buffers).

Between replays the test clobbers every output with eager fills and synchronises, so a replay
that skipped a node or relied on stale memory would show.
"""
import numpy as np
import pytest

import gpu_common as G
import synth

pytestmark = pytest.mark.gpu


def _lib():
    import rope_mxfp8_qkv_amd as q
    q.lib()
    return q


CASES = [("rowmx-staged", "rowmx", "staged"), ("rowmx-packed", "rowmx", "packed"),
         ("mx-staged", "mx", "staged"), ("mx-natural", "mx", "packed")]


def _setup(q, dev, act, layout):
    import torch
    p = G.custom_projection("graph", T=300, H=512, nq=3, nkv=1, d=128)
    inp = G.make_inputs(p)
    hid, res, gam = synth.producer_inputs(81, p.T, p.H)
    b = {"hid": G.bf16_dev(hid, dev), "res": G.bf16_dev(res, dev), "gam": G.bf16_dev(gam, dev),
         "wp": q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev), p.H, p.I),
         "bias": G.bf16_dev(inp.bias, dev), "gq": G.bf16_dev(inp.gq, dev),
         "gk": G.bf16_dev(inp.gk, dev), "cos": G.to_dev(inp.cos, dev),
         "sin": G.to_dev(inp.sin, dev),
         "res_out": torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev),
         "out": torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev),
         "ssq": torch.empty((p.T, 2), dtype=torch.float32, device=dev)}
    if layout == "staged":
        b["img"] = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
        b["ws"] = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
        if act == "mx":
            b["eimg"] = torch.empty(q.qkv_act_exp_image_bytes(p.T, p.H) // 4, dtype=torch.int32,
                                    device=dev)
        else:
            b["sc"] = torch.empty((p.T,), dtype=torch.float32, device=dev)
    elif act == "mx":
        b["codes"] = torch.empty((p.T, p.H), dtype=torch.uint8, device=dev)
        b["e8"] = torch.empty((p.T, p.H // 32), dtype=torch.uint8, device=dev)
        b["ws"] = torch.empty(q.qkv_mx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    else:
        b["packed"] = torch.empty((p.T, p.H + 4), dtype=torch.uint8, device=dev)
        b["ws"] = torch.empty(q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
    return p, b


def _step(q, p, b, act, layout):
    kw = dict(num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim)
    common = dict(residual=b["res"], residual_out=b["res_out"])
    if act == "mx" and layout == "staged":
        q.rmsnorm_mx_block_quantize_staged(b["hid"], b["gam"], 1e-6, b["img"], b["eimg"], **common)
        q.qkv_mx_project_staged(b["img"], b["eimg"], b["wp"], b["out"], T=p.T, H=p.H,
                                bias=b["bias"], ssq=b["ssq"], workspace=b["ws"], **kw)
    elif act == "mx":
        q.rmsnorm_mx_block_quantize(b["hid"], b["gam"], 1e-6, b["codes"], b["e8"], **common)
        q.qkv_mx_project(b["codes"], b["e8"], b["wp"], b["out"], H=p.H, bias=b["bias"],
                         ssq=b["ssq"], workspace=b["ws"], **kw)
    elif layout == "staged":
        q.rmsnorm_mx_quantize_staged(b["hid"], b["gam"], 1e-6, b["img"], b["sc"], **common)
        q.qkv_rowmx_project_staged(b["img"], b["sc"], b["wp"], b["out"], H=p.H, bias=b["bias"],
                                   ssq=b["ssq"], workspace=b["ws"], **kw)
    else:
        q.rmsnorm_mx_quantize(b["hid"], b["gam"], 1e-6, b["packed"], **common)
        q.qkv_rowmx_project(b["packed"], b["wp"], b["out"], H=p.H, bias=b["bias"], ssq=b["ssq"],
                            workspace=b["ws"], **kw)
    q.qk_norm_rope_apply(b["out"], eps=1e-6, flags=q.NORM_Q | q.NORM_K | q.FUSED_ROPE,
                         ssq=b["ssq"], q_gamma=b["gq"], k_gamma=b["gk"], cos=b["cos"],
                         sin=b["sin"], **kw)


def _outputs(b):
    return (G.bf16_host(b["out"]).copy(), G.bf16_host(b["res_out"]).copy(),
            b["ssq"].cpu().numpy().view(np.uint32).copy())


def _clobber(b):
    b["out"].fill_(float("nan"))
    b["res_out"].fill_(float("nan"))
    b["ssq"].fill_(float("nan"))
    for k in ("img", "packed", "codes", "e8", "eimg", "ws"):
        if k in b:
            b[k].fill_(0x5A)
    if "sc" in b:
        b["sc"].fill_(float("nan"))


def _compare(got, ref, what):
    for g, r, name in zip(got, ref, ("projected Q/K/V", "residual_out", "ssq")):
        G.check_equal(g, r, f"{what}: {name}")


@pytest.mark.parametrize("name,act,layout", CASES, ids=[c[0] for c in CASES])
def test_step_graph_replays_match_eager(name, act, layout):
    import torch
    q = _lib()
    dev = G.torch_dev()
    p, b = _setup(q, dev, act, layout)
    _step(q, p, b, act, layout)
    torch.cuda.synchronize()
    ref = _outputs(b)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up on the capture stream
        _step(q, p, b, act, layout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(q, p, b, act, layout)
    torch.cuda.synchronize()

    for i in range(3):
        _clobber(b)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _compare(_outputs(b), ref, f"replay {i}")

    b["hid"].mul_(-0.5)                            # new inputs in the same buffers
    b["res"].add_(0.25)
    torch.cuda.synchronize()
    _step(q, p, b, act, layout)                    # eager result on the new inputs
    torch.cuda.synchronize()
    ref2 = _outputs(b)
    assert not np.array_equal(ref2[1], ref[1])
    for i in range(2):
        _clobber(b)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _compare(_outputs(b), ref2, f"replay {i} on rewritten inputs")
