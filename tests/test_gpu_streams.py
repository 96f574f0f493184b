"""Concurrent calls on distinct streams with distinct buffers: the library keeps no mutable
global state, so two whole steps (staged producer -> projection -> norm + RoPE) enqueued
alternately on two streams, one on the split-contraction path and one unsplit, must give the
bytes each gives when run alone on the current stream.  Both streams have the default priority.
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


SHAPES = [G.custom_projection("streams-split", T=512, H=1792, nq=16, nkv=12, d=128),
          G.custom_projection("streams-unsplit", T=1100, H=512, nq=45, nkv=3, d=128)]


class Step:
    def __init__(self, q, dev, p, seed):
        import torch
        self.q, self.p = q, p
        inp = G.make_inputs(p)
        hid, res, gam = synth.producer_inputs(seed, p.T, p.H)
        self.hid, self.res, self.gam = (G.bf16_dev(hid, dev), G.bf16_dev(res, dev),
                                        G.bf16_dev(gam, dev))
        self.wp = q.prepare_weight(G.to_dev(inp.w_codes, dev), G.to_dev(inp.w_e8m0, dev),
                                   p.H, p.I)
        self.bias, self.gq, self.gk = (G.bf16_dev(inp.bias, dev), G.bf16_dev(inp.gq, dev),
                                       G.bf16_dev(inp.gk, dev))
        self.cos, self.sin = G.to_dev(inp.cos, dev), G.to_dev(inp.sin, dev)
        self.res_out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev)
        self.img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
        self.sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
        self.out = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev)
        self.ssq = torch.empty((p.T, 2), dtype=torch.float32, device=dev)
        self.ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8,
                              device=dev)

    def run(self, stream=None):
        q, p = self.q, self.p
        kw = dict(num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim)
        q.rmsnorm_mx_quantize_staged(self.hid, self.gam, 1e-6, self.img, self.sc,
                                     residual=self.res, residual_out=self.res_out, stream=stream)
        q.qkv_rowmx_project_staged(self.img, self.sc, self.wp, self.out, H=p.H, bias=self.bias,
                                   ssq=self.ssq, workspace=self.ws, stream=stream, **kw)
        q.qk_norm_rope_apply(self.out, eps=1e-6, flags=q.NORM_Q | q.NORM_K | q.FUSED_ROPE,
                             ssq=self.ssq, q_gamma=self.gq, k_gamma=self.gk, cos=self.cos,
                             sin=self.sin, stream=stream, **kw)

    def result(self):
        return (G.bf16_host(self.out).copy(), G.bf16_host(self.res_out).copy(),
                self.ssq.cpu().numpy().view(np.uint32).copy())

    def clobber(self):
        self.out.fill_(float("nan"))
        self.res_out.fill_(float("nan"))
        self.ssq.fill_(float("nan"))
        self.img.fill_(0x5A)
        self.ws.fill_(0x5A)


def test_two_streams_match_serial():
    import torch
    q = _lib()
    dev = G.torch_dev()
    assert q.projection_k_chunks(SHAPES[0].T, SHAPES[0].H, SHAPES[0].I) > 1
    assert q.projection_k_chunks(SHAPES[1].T, SHAPES[1].H, SHAPES[1].I) == 1
    steps = [Step(q, dev, p, 90 + i) for i, p in enumerate(SHAPES)]
    ref = []
    for s in steps:                               # alone, on the current stream
        s.run()
        torch.cuda.synchronize()
        ref.append(s.result())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for s in steps:
            s.clobber()
        torch.cuda.synchronize()
        for _ in range(2):                        # interleaved enqueue, twice per stream
            for s, st in zip(steps, streams):
                s.run(stream=st)
        torch.cuda.synchronize()
        for s, r in zip(steps, ref):
            for got, want, what in zip(s.result(), r, ("out", "residual_out", "ssq")):
                G.check_equal(got, want, f"{s.p.name} rep {rep}: {what}")
