"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The GPU runs every stage on the whole workload (T = 75600 tokens of the 21 x 45 x 80 video
grid, H = 5120, I = 15360, or the separate cross-attention calls); the oracle recomputes a
sample of rows one by one -- tile boundaries, the ragged last tile and random rows -- from the
same seeded inputs.  Encoded bytes (ROW_MX rows, weight codes and exponents, the residual sum)
are compared bit for bit; bf16 outputs to |gpu - ref| <= 1e-2 |ref| + 1e-3 (plus, after pass 2,
the propagated rounding of pass 1's stored bf16 output, see gpu_common).
"""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sample_rows(T, n_random=40, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 255, 256, 257, 511, 512, 4095, 4096, T // 2, T - 257, T - 256, T - 80,
             T - 2, T - 1]
    rows = np.concatenate([[r for r in fixed if 0 <= r < T], rng.integers(0, T, n_random)])
    return np.unique(rows)


class Gpu:
    """The library calls of one projection on full-size device tensors."""

    def __init__(self, q, dev):
        self.q, self.dev = q, dev

    def weight(self, w):
        import torch
        H, I = w.shape
        codes = torch.empty((H // 4, I, 4), dtype=torch.uint8, device=self.dev)
        e8 = torch.empty((H // 32, I), dtype=torch.uint8, device=self.dev)
        self.q.mx_weight_quantize(G.to_dev(w, self.dev), codes, e8)
        return codes, e8, self.q.prepare_weight(codes, e8, H, I)

    def project(self, p, packed, wp, bias):
        import torch
        out = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=self.dev)
        ssq = torch.empty((p.T, 2), dtype=torch.float32, device=self.dev)
        ws = torch.empty(self.q.qkvmx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8,
                         device=self.dev)
        self.q.qkv_rowmx_project(packed, wp, out, H=p.H, num_heads=p.num_heads,
                                 num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                                 bias=G.bf16_dev(bias, self.dev), ssq=ssq, workspace=ws)
        return out, ssq

    def project_staged(self, p, img, sc, wp, bias):
        import torch
        out = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=self.dev)
        ssq = torch.empty((p.T, 2), dtype=torch.float32, device=self.dev)
        ws = torch.empty(self.q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8,
                         device=self.dev)
        self.q.qkv_rowmx_project_staged(img, sc, wp, out, H=p.H, num_heads=p.num_heads,
                                        num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                                        bias=G.bf16_dev(bias, self.dev), ssq=ssq, workspace=ws)
        return out, ssq

    def pass2(self, p, out, ssq, gq, gk, cos, sin):
        fl = G.flags_of(p)
        if fl == 0:
            return fl
        q = self.q
        q.qk_norm_rope_apply(out, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                             head_dim=p.head_dim, eps=1e-6, flags=fl, ssq=ssq,
                             q_gamma=G.bf16_dev(gq, self.dev) if fl & q.NORM_Q else None,
                             k_gamma=G.bf16_dev(gk, self.dev) if fl & q.NORM_K else None,
                             cos=G.to_dev(cos, self.dev) if fl & q.FUSED_ROPE else None,
                             sin=G.to_dev(sin, self.dev) if fl & q.FUSED_ROPE else None)
        return fl


def check_projection(p, packed_rows_ref, w_codes, w_e8, bias, gq, gk, out, ssq, rows, fl,
                     mx_rows_ref=None):
    """Oracle on the sampled rows vs the GPU's pass-1 sums and final (pass-2) outputs.  The
    activation rows are ROW_MX packed rows, or (mx_rows_ref) MX block-32 codes and exponents."""
    W = oracle.mx_weight_decode(w_codes, w_e8)
    if mx_rows_ref is None:
        codes, sA = oracle.rowmx_unpack(packed_rows_ref, p.H)
        a_e8 = None
    else:
        (codes, a_e8), sA = mx_rows_ref, None
    X, ssq_ref = oracle.project(codes, sA, w_codes, w_e8, None, bias, num_heads=p.num_heads,
                                num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, w_dense=W,
                                a_e8m0=a_e8)
    cos, sin = synth.rope_tables(p, rows)
    if fl:
        ref = oracle.norm_rope(None, ssq_ref, gq, gk if fl & 2 else None, cos, sin,
                               num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                               head_dim=p.head_dim, eps=1e-6, flags=fl, values=X)
        extra = G.propagated_bound(X, ssq_ref, gq, gk, p.num_heads, p.num_kv_heads, p.head_dim,
                                   1e-6, bool(fl & 1), bool(fl & 2), bool(fl & 4))
    else:
        ref, extra = X, None
    ti = _idx(rows, out.device)
    G.check_close(G.bf16_host(out[ti]), ref, f"{p.name} output rows", extra=extra)
    G.check_ssq(ssq[ti].cpu().numpy(), ssq_ref, f"{p.name} sums")


def _idx(rows, device):
    import torch
    return torch.as_tensor(np.asarray(rows, dtype=np.int64), device=device)


def _run_self_attention(p, producer: bool, staged: bool = False):
    import torch
    q = __import__("rope_mxfp8_qkv_amd")
    q.lib()
    dev = G.torch_dev()
    gpu = Gpu(q, dev)
    rows = sample_rows(p.T)
    print(f"[fullsize] {p.name}: T={p.T} H={p.H} I={p.I} rows={len(rows)}", flush=True)
    if staged:
        img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
        sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
    else:
        packed = torch.empty((p.T, p.H + 4), dtype=torch.uint8, device=dev)
    if producer:
        hid, res, gam = synth.producer_inputs(p.seed_id, p.T, p.H)
        res_out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev)
        if staged:
            q.rmsnorm_mx_quantize_staged(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, img, sc,
                                         residual=G.bf16_dev(res, dev), residual_out=res_out)
        else:
            q.rmsnorm_mx_quantize(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, packed,
                                  residual=G.bf16_dev(res, dev), residual_out=res_out)
        r_ref, packed_ref, _ = oracle.rmsnorm_rowmx(hid[rows], res[rows], gam, 1e-6)
        G.check_equal(G.bf16_host(res_out[_idx(rows, dev)]), r_ref, "residual_out rows")
        del hid, res, res_out
    else:
        x = synth.activation(p)
        if staged:
            q.row_quantize_staged(G.to_dev(x, dev), img, sc)
        else:
            q.row_quantize_packed(G.to_dev(x, dev), packed)
        packed_ref = oracle.rowmx_quantize(x[rows])
        del x
    if staged:
        codes_ref, s_ref = oracle.rowmx_unpack(packed_ref, p.H)
        G.check_equal(G.unstage(img, rows, p.H), codes_ref, "staged code rows")
        G.check_equal(sc[_idx(rows, dev)].cpu().numpy().view(np.uint32),
                      s_ref.astype(np.float32).view(np.uint32), "row scales")
    else:
        G.check_equal(packed[_idx(rows, dev)].cpu().numpy(), packed_ref, "ROW_MX rows")
    w = synth.weight(p)
    codes, e8, wp = gpu.weight(w)
    w_codes, w_e8 = oracle.mx_weight_quantize(w)
    G.check_equal(e8.cpu().numpy(), w_e8, "weight exponents")
    G.check_equal(codes.cpu().numpy(), w_codes, "weight codes")
    bias, gq, gk = synth.bias_bf16(p), synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k")
    cos, sin = synth.rope_tables(p)
    if staged:
        out, ssq = gpu.project_staged(p, img, sc, wp, bias)
    else:
        out, ssq = gpu.project(p, packed, wp, bias)
    seg = (p.num_heads + p.num_kv_heads) * p.head_dim
    ti = _idx(rows, dev)
    v_before = out[ti, seg:].clone()
    fl = gpu.pass2(p, out, ssq, gq, gk, cos, sin)
    torch.cuda.synchronize()
    assert torch.equal(out[ti, seg:].view(torch.int16), v_before.view(torch.int16))
    check_projection(p, packed_ref, w_codes, w_e8, bias, gq, gk, out, ssq, rows, fl)


def test_fullsize_self_attention_video():
    """Full video shape (21 x 45 x 80 tokens, outlier channels, 3-axis RoPE)."""
    _run_self_attention(synth.CONFIGS[3].calls[0], producer=False)


def test_fullsize_producer_then_self_attention():
    """bf16 hidden + residual -> fused producer -> projection -> norm + 3-axis RoPE."""
    _run_self_attention(synth.CONFIGS[5].calls[0], producer=True)


def test_fullsize_staged_producer_then_self_attention():
    """The benchmark's default step: fused producer writing staged codes and row scales ->
    staged projection -> norm + 3-axis RoPE."""
    _run_self_attention(synth.CONFIGS[5].calls[0], producer=True, staged=True)


def test_fullsize_nbsd_step_equals_bsd_step():
    """The benchmark's default step with the NBSd output ([I / d, T, d]; the last heads' rows lie
    2.3 GB into the output): staged producer -> staged projection -> norm + 3-axis RoPE in
    NBSd gives byte for byte the BSD step's output re-indexed (every element) and the same sums;
    sampled rows also against the oracle."""
    import torch
    q = __import__("rope_mxfp8_qkv_amd")
    q.lib()
    dev = G.torch_dev()
    gpu = Gpu(q, dev)
    p = synth.CONFIGS[5].calls[0]
    rows = sample_rows(p.T)
    print(f"[fullsize] {p.name} (NBSd vs BSD): T={p.T} H={p.H} I={p.I} rows={len(rows)}", flush=True)
    hid, res, gam = synth.producer_inputs(p.seed_id, p.T, p.H)
    img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
    sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
    res_out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_quantize_staged(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, img, sc,
                                 residual=G.bf16_dev(res, dev), residual_out=res_out)
    _, packed_ref, _ = oracle.rmsnorm_rowmx(hid[rows], res[rows], gam, 1e-6)
    del hid, res, res_out
    w = synth.weight(p)
    _, _, wp = gpu.weight(w)
    w_codes, w_e8 = oracle.mx_weight_quantize(w)
    bias, gq, gk = synth.bias_bf16(p), synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k")
    cos, sin = synth.rope_tables(p)
    fl = G.flags_of(p)
    ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    d = p.head_dim
    res = {}
    for name, layout, shape in (("bsd", q.LAYOUT_BSD, (p.T, p.I)),
                                ("nbsd", q.LAYOUT_NBSD, (p.I // d, p.T, d))):
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        ssq = torch.empty((p.T, 2), dtype=torch.float32, device=dev)
        q.qkv_rowmx_project_staged(img, sc, wp, out, H=p.H, num_heads=p.num_heads,
                                   num_kv_heads=p.num_kv_heads, head_dim=d,
                                   bias=G.bf16_dev(bias, dev), ssq=ssq, workspace=ws,
                                   layout=layout)
        q.qk_norm_rope_apply(out, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                             head_dim=d, eps=1e-6, flags=fl, ssq=ssq,
                             q_gamma=G.bf16_dev(gq, dev), k_gamma=G.bf16_dev(gk, dev),
                             cos=G.to_dev(cos, dev), sin=G.to_dev(sin, dev), layout=layout)
        res[name] = (out, ssq)
    torch.cuda.synchronize()
    (bsd, ssq_b), (nbsd, ssq_n) = res["bsd"], res["nbsd"]
    assert torch.equal(ssq_b.view(torch.int32), ssq_n.view(torch.int32)), "sums differ"
    nbsd_as_bsd = nbsd.permute(1, 0, 2).reshape(p.T, p.I)
    assert torch.equal(nbsd_as_bsd.view(torch.int16), bsd.view(torch.int16)), "NBSd != BSD"
    del bsd
    check_projection(p, packed_ref, w_codes, w_e8, bias, gq, gk, nbsd_as_bsd, ssq_n, rows, fl)


@pytest.mark.parametrize("kind", [1, 2], ids=["rms", "ln-beta"])
def test_fullsize_headnorm_step(kind):
    """The benchmark's --headnorm step at the full video shape: staged producer -> staged
    projection with the per-head RMS_NORM (LAYER_NORM with beta) and 3-axis RoPE fused into its
    epilogue, no pass 2; per-head gamma / beta as the benchmark draws them (the first head_dim
    entries of the seeded segment gammas / of the bias); sampled rows against the oracle."""
    import torch
    q = __import__("rope_mxfp8_qkv_amd")
    q.lib()
    dev = G.torch_dev()
    gpu = Gpu(q, dev)
    p = synth.CONFIGS[5].calls[0]
    d = p.head_dim
    rows = sample_rows(p.T)
    print(f"[fullsize] {p.name} (per-head norm kind {kind}): T={p.T} H={p.H} I={p.I} "
          f"rows={len(rows)}", flush=True)
    hid, res, gam = synth.producer_inputs(p.seed_id, p.T, p.H)
    img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
    sc = torch.empty((p.T,), dtype=torch.float32, device=dev)
    res_out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_quantize_staged(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, img, sc,
                                 residual=G.bf16_dev(res, dev), residual_out=res_out)
    _, packed_ref, _ = oracle.rmsnorm_rowmx(hid[rows], res[rows], gam, 1e-6)
    del hid, res, res_out
    w = synth.weight(p)
    _, _, wp = gpu.weight(w)
    w_codes, w_e8 = oracle.mx_weight_quantize(w)
    bias = synth.bias_bf16(p)
    hgq, hgk = synth.gamma_bf16(p, "q")[:d], synth.gamma_bf16(p, "k")[:d]
    hbq, hbk = (bias[:d], bias[d:2 * d]) if kind == 2 else (None, None)
    cos, sin = synth.rope_tables(p)
    out = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
    opt = lambda a: None if a is None else G.bf16_dev(a, dev)
    q.qkv_rowmx_project_headnorm_staged(img, sc, wp, out, H=p.H, num_heads=p.num_heads,
                                        num_kv_heads=p.num_kv_heads, head_dim=d, norm_kind=kind,
                                        q_gamma=opt(hgq), k_gamma=opt(hgk), q_beta=opt(hbq),
                                        k_beta=opt(hbk), eps=1e-6, cos=G.to_dev(cos, dev),
                                        sin=G.to_dev(sin, dev), bias=opt(bias), workspace=ws)
    torch.cuda.synchronize()
    codes, sA = oracle.rowmx_unpack(packed_ref, p.H)
    X, _ = oracle.project(codes, sA, w_codes, w_e8, None, bias, num_heads=p.num_heads,
                          num_kv_heads=p.num_kv_heads, head_dim=d)
    ref = oracle.head_norm_rope(X, kind, hgq, hgk, 1e-6, cos[rows], sin[rows],
                                num_heads=p.num_heads, num_kv_heads=p.num_kv_heads, head_dim=d,
                                q_beta_bf16=hbq, k_beta_bf16=hbk)
    G.check_close(G.bf16_host(out[_idx(rows, dev)]), ref, f"{p.name} per-head output rows")


@pytest.mark.parametrize("staged", [False, True], ids=["natural", "staged"])
def test_fullsize_mx_producer_then_self_attention(staged):
    """MX block-32 path at the full video shape: bf16 hidden + residual -> residual add +
    RMSNorm + E4M3 codes with per-32 exponents (and the bf16 normed rows) -> projection with
    per-block activation exponents -> norm + 3-axis RoPE; natural-order codes and exponents, or
    staged in the projection's layouts (the benchmark's --act mx step)."""
    import torch
    q = __import__("rope_mxfp8_qkv_amd")
    q.lib()
    dev = G.torch_dev()
    gpu = Gpu(q, dev)
    p = synth.CONFIGS[5].calls[0]
    rows = sample_rows(p.T)
    print(f"[fullsize] {p.name} (MX block-32): T={p.T} H={p.H} I={p.I} rows={len(rows)}", flush=True)
    hid, res, gam = synth.producer_inputs(p.seed_id, p.T, p.H)
    res_out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev)
    norm = torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev)
    if staged:
        img = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
        eimg = torch.empty(q.qkv_act_exp_image_bytes(p.T, p.H) // 4, dtype=torch.int32, device=dev)
        q.rmsnorm_mx_block_quantize_staged(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, img,
                                           eimg, residual=G.bf16_dev(res, dev),
                                           residual_out=res_out, norm_out=norm)
    else:
        codes = torch.empty((p.T, p.H), dtype=torch.uint8, device=dev)
        e8 = torch.empty((p.T, p.H // 32), dtype=torch.uint8, device=dev)
        q.rmsnorm_mx_block_quantize(G.bf16_dev(hid, dev), G.bf16_dev(gam, dev), 1e-6, codes, e8,
                                    residual=G.bf16_dev(res, dev), residual_out=res_out,
                                    norm_out=norm)
    r_ref, c_ref, e_ref, n_ref, _ = oracle.rmsnorm_mx(hid[rows], res[rows], gam, 1e-6)
    del hid, res
    ti = _idx(rows, dev)
    G.check_equal(G.bf16_host(res_out[ti]), r_ref, "residual_out rows")
    G.check_equal(G.bf16_host(norm[ti]), n_ref, "bf16 norm rows")
    if staged:
        G.check_equal(G.unstage(img, rows, p.H), c_ref, "MX code rows")
        G.check_equal(G.unstage_exp(eimg, rows, p.H), e_ref, "MX exponent rows")
    else:
        G.check_equal(codes[ti].cpu().numpy(), c_ref, "MX code rows")
        G.check_equal(e8[ti].cpu().numpy(), e_ref, "MX exponent rows")
    del res_out, norm
    w = synth.weight(p)
    wcodes, we8, wp = gpu.weight(w)
    w_codes, w_e8 = oracle.mx_weight_quantize(w)
    G.check_equal(wcodes.cpu().numpy(), w_codes, "weight codes")
    bias, gq, gk = synth.bias_bf16(p), synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k")
    cos, sin = synth.rope_tables(p)
    out = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev)
    ssq = torch.empty((p.T, 2), dtype=torch.float32, device=dev)
    if staged:
        ws = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
        q.qkv_mx_project_staged(img, eimg, wp, out, T=p.T, H=p.H, num_heads=p.num_heads,
                                num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                                bias=G.bf16_dev(bias, dev), ssq=ssq, workspace=ws)
    else:
        ws = torch.empty(q.qkv_mx_workspace_bytes(p.T, p.H, p.I), dtype=torch.uint8, device=dev)
        q.qkv_mx_project(codes, e8, wp, out, H=p.H, num_heads=p.num_heads,
                         num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                         bias=G.bf16_dev(bias, dev), ssq=ssq, workspace=ws)
    seg = (p.num_heads + p.num_kv_heads) * p.head_dim
    v_before = out[ti, seg:].clone()
    fl = gpu.pass2(p, out, ssq, gq, gk, cos, sin)
    torch.cuda.synchronize()
    assert torch.equal(out[ti, seg:].view(torch.int16), v_before.view(torch.int16))
    check_projection(p, None, w_codes, w_e8, bias, gq, gk, out, ssq, rows, fl,
                     mx_rows_ref=(c_ref, e_ref))


def test_fullsize_cross_attention_separate_calls():
    """Three single-segment calls: Q (75600 latent tokens, normed, no RoPE), K (512 context
    tokens, normed as Q with K's gamma), V (512 context tokens, no pass 2)."""
    import torch
    q = __import__("rope_mxfp8_qkv_amd")
    q.lib()
    dev = G.torch_dev()
    gpu = Gpu(q, dev)
    for p in synth.CONFIGS[4].calls:
        rows = sample_rows(p.T) if p.T > 4096 else np.arange(p.T)
        print(f"[fullsize] {p.name}: T={p.T} I={p.I} rows={len(rows)}", flush=True)
        x = synth.activation(p)
        packed = torch.empty((p.T, p.H + 4), dtype=torch.uint8, device=dev)
        q.row_quantize_packed(G.to_dev(x, dev), packed)
        packed_ref = oracle.rowmx_quantize(x[rows])
        G.check_equal(packed[_idx(rows, dev)].cpu().numpy(), packed_ref, f"{p.name} ROW_MX rows")
        del x
        w = synth.weight(p)
        codes, e8, wp = gpu.weight(w)
        w_codes, w_e8 = oracle.mx_weight_quantize(w)
        G.check_equal(codes.cpu().numpy(), w_codes, f"{p.name} weight codes")
        bias, gq = synth.bias_bf16(p), synth.gamma_bf16(p, "q")
        out, ssq = gpu.project(p, packed, wp, bias)
        ti = _idx(rows, dev)
        before = out[ti].clone()
        fl = gpu.pass2(p, out, ssq, gq, None, None, None)
        torch.cuda.synchronize()
        if fl == 0:                                   # V: pass 2 must not run at all
            assert torch.equal(out[ti].view(torch.int16), before.view(torch.int16))
        check_projection(p, packed_ref, w_codes, w_e8, bias, gq, None, out, ssq, rows, fl)
