"""Pins of the oracle's per-head qk-norm (+ rotate-half RoPE): torch's rms_norm / layer_norm
on each head's slice (fp64), the normalised statistics per head, a closed form on a two-value
head, RoPE's pair-norm preservation and position-0 identity, V unchanged, and the segments'
separate gammas."""
import numpy as np
import torch

import oracle
from oracle import codecs


def _inputs(T=6, nq=3, nkv=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    I = (nq + 2 * nkv) * d
    X = rng.standard_normal((T, I)) * rng.uniform(0.1, 10, (T, 1)) + rng.standard_normal(I)
    gq = codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(d))
    gk = codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(d))
    bq = codecs.f64_to_bf16(0.1 * rng.standard_normal(d))
    bk = codecs.f64_to_bf16(0.1 * rng.standard_normal(d))
    ang = rng.uniform(0, 6.3, (T, d // 2))
    cos = np.cos(np.concatenate([ang, ang], 1)).astype(np.float32)
    sin = np.sin(np.concatenate([ang, ang], 1)).astype(np.float32)
    return X, gq, gk, bq, bk, cos, sin


def test_matches_torch_norms_per_head():
    X, gq, gk, bq, bk, _, _ = _inputs()
    nq, nkv, d = 3, 2, 8
    eps = 1e-6
    e = float(np.float32(eps))
    for kind in (oracle.RMS_NORM, oracle.LAYER_NORM):
        beta = (bq, bk) if kind == oracle.LAYER_NORM else (None, None)
        out = oracle.head_norm_rope(X, kind, gq, gk, eps, num_heads=nq, num_kv_heads=nkv,
                                    head_dim=d, q_beta_bf16=beta[0], k_beta_bf16=beta[1])
        for lo, n, g, b in ((0, nq, gq, beta[0]), (nq * d, nkv, gk, beta[1])):
            xh = torch.from_numpy(X[:, lo:lo + n * d].reshape(-1, n, d))
            gt = torch.from_numpy(codecs.bf16_to_f64(g))
            if kind == oracle.RMS_NORM:
                ref = torch.nn.functional.rms_norm(xh, (d,), weight=gt, eps=e)
            else:
                ref = torch.nn.functional.layer_norm(xh, (d,), weight=gt,
                                                     bias=torch.from_numpy(codecs.bf16_to_f64(b)), eps=e)
            np.testing.assert_allclose(out[:, lo:lo + n * d], ref.reshape(X.shape[0], -1).numpy(),
                                       rtol=1e-12, atol=1e-12)
        v0 = (nq + nkv) * d
        assert np.array_equal(out[:, v0:], X[:, v0:])


def test_normalised_statistics_and_closed_form():
    X, _, _, _, _, _, _ = _inputs(seed=1)
    nq, nkv, d = 3, 2, 8
    ones = codecs.f64_to_bf16(np.ones(d))
    r = oracle.head_norm_rope(X, oracle.RMS_NORM, ones, ones, 0.0, num_heads=nq,
                              num_kv_heads=nkv, head_dim=d)
    seg = r[:, :(nq + nkv) * d].reshape(X.shape[0], -1, d)
    np.testing.assert_allclose(np.mean(seg * seg, -1), 1.0, rtol=1e-12)
    ln = oracle.head_norm_rope(X, oracle.LAYER_NORM, ones, ones, 0.0, num_heads=nq,
                               num_kv_heads=nkv, head_dim=d)
    seg = ln[:, :(nq + nkv) * d].reshape(X.shape[0], -1, d)
    np.testing.assert_allclose(np.mean(seg, -1), 0.0, atol=1e-12)
    np.testing.assert_allclose(np.var(seg, -1), 1.0, rtol=1e-12)
    # a head of two values (a, b): RMS norm -> (a, b) / sqrt((a^2 + b^2) / 2); LayerNorm -> (-1, 1)
    x = np.array([[3.0, 4.0, 1.0, 7.0, 0.5, 0.5]])                  # nq = 1, nkv = 1, d = 2
    o2 = codecs.f64_to_bf16(np.ones(2))
    rr = oracle.head_norm_rope(x, oracle.RMS_NORM, o2, o2, 0.0, num_heads=1, num_kv_heads=1, head_dim=2)
    np.testing.assert_allclose(rr[0, :2], np.array([3, 4]) / np.sqrt(12.5), rtol=1e-15)
    lr = oracle.head_norm_rope(x, oracle.LAYER_NORM, o2, o2, 0.0, num_heads=1, num_kv_heads=1, head_dim=2)
    np.testing.assert_allclose(lr[0, :4], [-1, 1, -1, 1], rtol=1e-15)
    assert np.array_equal(lr[0, 4:], x[0, 4:])                    # V


def test_rope_after_norm():
    X, gq, gk, _, _, cos, sin = _inputs(seed=2)
    nq, nkv, d = 3, 2, 8
    a = oracle.head_norm_rope(X, oracle.RMS_NORM, gq, gk, 1e-6, num_heads=nq, num_kv_heads=nkv,
                              head_dim=d)
    b = oracle.head_norm_rope(X, oracle.RMS_NORM, gq, gk, 1e-6, cos, sin, num_heads=nq,
                              num_kv_heads=nkv, head_dim=d)
    h = d // 2
    w = (nq + nkv) * d
    an, bn = a[:, :w].reshape(-1, nq + nkv, d), b[:, :w].reshape(-1, nq + nkv, d)
    # each rotate-half pair keeps its norm, up to the fp32 tables' cos^2 + sin^2 - 1 (~1e-7)
    np.testing.assert_allclose(an[..., :h] ** 2 + an[..., h:] ** 2, bn[..., :h] ** 2 + bn[..., h:] ** 2, rtol=5e-7)
    # explicit rotation of pair (j, j + h) by the row's angle
    c, s = cos.astype(np.float64)[:, None, :h], sin.astype(np.float64)[:, None, :h]
    np.testing.assert_allclose(bn[..., :h], an[..., :h] * c - an[..., h:] * s, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bn[..., h:], an[..., h:] * c + an[..., :h] * s, rtol=1e-12, atol=1e-14)
    # position 0 (cos = 1, sin = 0) leaves the normed values
    c0 = np.ones_like(cos); s0 = np.zeros_like(sin)
    z = oracle.head_norm_rope(X, oracle.RMS_NORM, gq, gk, 1e-6, c0, s0, num_heads=nq,
                              num_kv_heads=nkv, head_dim=d)
    np.testing.assert_array_equal(z, a)
    assert np.array_equal(b[:, w:], X[:, w:])


def test_separate_segment_gammas_and_single_segment():
    X, gq, gk, _, _, _, _ = _inputs(T=3, nq=2, nkv=0, d=8, seed=3)
    out = oracle.head_norm_rope(X, oracle.RMS_NORM, gq, None, 1e-6, num_heads=2, num_kv_heads=0,
                                head_dim=8)
    xh = X.reshape(3, 2, 8)
    ref = xh / np.sqrt(np.mean(xh * xh, -1, keepdims=True) + float(np.float32(1e-6))) * codecs.bf16_to_f64(gq)
    np.testing.assert_allclose(out, ref.reshape(3, 16), rtol=1e-13)
    X2, gq2, gk2, _, _, _, _ = _inputs(seed=4)
    a = oracle.head_norm_rope(X2, oracle.RMS_NORM, gq2, gk2, 1e-6, num_heads=3, num_kv_heads=2, head_dim=8)
    b = oracle.head_norm_rope(X2, oracle.RMS_NORM, gq2, gq2, 1e-6, num_heads=3, num_kv_heads=2, head_dim=8)
    assert np.array_equal(a[:, :24], b[:, :24]) and not np.array_equal(a[:, 24:40], b[:, 24:40])
