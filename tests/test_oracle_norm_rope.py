"""Pins of the oracle's pass 2 (across-heads RMSNorm + rotate-half RoPE): a hand-worked example,
torch's RMSNorm, complex-rotation identity, invariants the pages state."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import codecs
from oracle.norm_rope import FUSED_ROPE, NORM_K, NORM_Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "norm_rope_hand_example.txt")


def _load_golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        vals[k] = np.array([float(x) for x in v])
    return vals


def test_hand_worked_example():
    g = _load_golden()
    row = np.concatenate([g["q_in"], g["k_in"], g["v_in"]])
    bits = codecs.f64_to_bf16(row)[None, :]
    assert np.array_equal(codecs.bf16_to_f64(bits)[0], row)        # exact in bf16
    ssq = np.array([[np.sum(g["q_in"] ** 2), np.sum(g["k_in"] ** 2)]])
    out = oracle.norm_rope(bits, ssq, codecs.f64_to_bf16(g["q_gamma"]),
                           codecs.f64_to_bf16(g["k_gamma"]), g["cos"][None].astype(np.float32),
                           g["sin"][None].astype(np.float32), num_heads=1, num_kv_heads=1,
                           head_dim=4, eps=0.0, flags=NORM_Q | NORM_K | FUSED_ROPE)
    assert np.allclose(out[0, :4], g["q_out"], rtol=0, atol=1e-15)
    assert np.allclose(out[0, 4:8], g["k_out"], rtol=0, atol=1e-15)
    assert np.array_equal(out[0, 8:], g["v_out"])


def _rand_case(rng, T=9, nq=3, nkv=2, d=8):
    I = (nq + 2 * nkv) * d
    x = rng.standard_normal((T, I)) * 3
    bits = codecs.f64_to_bf16(x)
    xv = codecs.bf16_to_f64(bits)
    ssq = np.stack([np.sum(xv[:, :nq * d] ** 2, 1), np.sum(xv[:, nq * d:(nq + nkv) * d] ** 2, 1)], 1)
    gq = codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(nq * d))
    gk = codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(nkv * d))
    cos, sin = synth.rope_1d(rng.integers(0, 5000, T), d)
    return bits, xv, ssq, gq, gk, cos, sin, (nq, nkv, d)


def test_position_zero_reduces_to_torch_rmsnorm():
    rng = np.random.default_rng(20)
    bits, xv, ssq, gq, gk, _, _, (nq, nkv, d) = _rand_case(rng)
    T = xv.shape[0]
    cos = np.ones((T, d), np.float32)
    sin = np.zeros((T, d), np.float32)
    eps = 1e-6
    out = oracle.norm_rope(bits, ssq, gq, gk, cos, sin, num_heads=nq, num_kv_heads=nkv,
                           head_dim=d, eps=eps, flags=NORM_Q | NORM_K | FUSED_ROPE)
    e = float(np.float32(eps))
    for lo, hi, g in ((0, nq * d, gq), (nq * d, (nq + nkv) * d, gk)):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(xv[:, lo:hi]), (hi - lo,),
                                           weight=torch.from_numpy(codecs.bf16_to_f64(g)), eps=e)
        assert np.allclose(out[:, lo:hi], ref.numpy(), rtol=1e-13, atol=1e-14)


def test_rope_equals_complex_rotation_and_v_untouched():
    rng = np.random.default_rng(21)
    bits, xv, ssq, gq, gk, cos, sin, (nq, nkv, d) = _rand_case(rng)
    out = oracle.norm_rope(bits, ssq, gq, gk, cos, sin, num_heads=nq, num_kv_heads=nkv,
                           head_dim=d, eps=1e-6, flags=NORM_Q | NORM_K | FUSED_ROPE)
    normed = oracle.norm_rope(bits, ssq, gq, gk, None, None, num_heads=nq, num_kv_heads=nkv,
                              head_dim=d, eps=1e-6, flags=NORM_Q | NORM_K)
    T = xv.shape[0]
    h = d // 2
    seg = (nq + nkv) * d
    y = normed[:, :seg].reshape(T, nq + nkv, d)
    o = out[:, :seg].reshape(T, nq + nkv, d)
    theta = np.arctan2(sin[:, :h].astype(np.float64), cos[:, :h].astype(np.float64))
    rad = np.hypot(cos[:, :h].astype(np.float64), sin[:, :h].astype(np.float64))
    z = (y[..., :h] + 1j * y[..., h:]) * (rad * np.exp(1j * theta))[:, None, :]
    assert np.allclose(o[..., :h], z.real, rtol=1e-12, atol=1e-12)
    assert np.allclose(o[..., h:], z.imag, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out[:, seg:], xv[:, seg:])            # V bit-identical
    assert np.array_equal(normed[:, seg:], xv[:, seg:])


def test_pair_norm_preserved_and_unit_rms():
    rng = np.random.default_rng(22)
    bits, xv, ssq, gq, gk, cos, sin, (nq, nkv, d) = _rand_case(rng, T=16)
    ones_q = codecs.f64_to_bf16(np.ones(nq * d))
    ones_k = codecs.f64_to_bf16(np.ones(nkv * d))
    eps = 1e-6
    out = oracle.norm_rope(bits, ssq, ones_q, ones_k, cos, sin, num_heads=nq, num_kv_heads=nkv,
                           head_dim=d, eps=eps, flags=NORM_Q | NORM_K | FUSED_ROPE)
    e = float(np.float32(eps))
    for lo, n, col in ((0, nq, 0), (nq * d, nkv, 1)):
        seg = out[:, lo:lo + n * d]
        ms = np.mean(seg ** 2, axis=1)
        m = ssq[:, col] / (n * d)
        # |cos|^2 + |sin|^2 = 1 up to the fp32 rounding of the tables
        assert np.allclose(ms, m / (m + e), rtol=1e-6)
        # per pair: out_j^2 + out_{j+d/2}^2 = r^2 (x_j^2 + x_{j+d/2}^2)
        r2 = 1.0 / (m + e)
        xs = xv[:, lo:lo + n * d].reshape(-1, n, d)
        os_ = seg.reshape(-1, n, d)
        h = d // 2
        lhs = os_[..., :h] ** 2 + os_[..., h:] ** 2
        rhs = r2[:, None, None] * (xs[..., :h] ** 2 + xs[..., h:] ** 2)
        c2 = (cos[:, :h].astype(np.float64) ** 2 + sin[:, :h].astype(np.float64) ** 2)[:, None, :]
        assert np.allclose(lhs, rhs * c2, rtol=1e-12, atol=1e-15)


def test_relative_position_property():
    """<RoPE(q, m), RoPE(k, n)> per head depends only on m - n (1-D tables)."""
    rng = np.random.default_rng(23)
    d = 16
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    row = np.concatenate([q, k, np.zeros(d)])
    bits = codecs.f64_to_bf16(row)[None]
    xv = codecs.bf16_to_f64(bits)[0]
    ssq = np.zeros((1, 2))
    dots = []
    for m, n in ((7, 3), (107, 103), (1007, 1003)):
        cm, sm = synth.rope_1d(np.array([m]), d)
        cn, sn = synth.rope_1d(np.array([n]), d)
        oq = oracle.norm_rope(bits, ssq, None, None, cm, sm, num_heads=1, num_kv_heads=1,
                              head_dim=d, eps=0.0, flags=FUSED_ROPE)[0, :d]
        ok = oracle.norm_rope(bits, ssq, None, None, cn, sn, num_heads=1, num_kv_heads=1,
                              head_dim=d, eps=0.0, flags=FUSED_ROPE)[0, d:2 * d]
        dots.append(oq @ ok)
    assert np.allclose(dots, dots[0], rtol=1e-5)
    assert not np.isclose(dots[0], xv[:d] @ xv[d:2 * d])


def test_norm_without_rope_and_single_segment():
    rng = np.random.default_rng(24)
    bits, xv, ssq, gq, gk, _, _, (nq, nkv, d) = _rand_case(rng)
    out = oracle.norm_rope(bits, ssq, gq, None, None, None, num_heads=nq, num_kv_heads=nkv,
                           head_dim=d, eps=1e-6, flags=NORM_Q)
    r = 1 / np.sqrt(ssq[:, 0] / (nq * d) + float(np.float32(1e-6)))
    assert np.allclose(out[:, :nq * d], xv[:, :nq * d] * codecs.bf16_to_f64(gq) * r[:, None],
                       rtol=1e-15)
    assert np.array_equal(out[:, nq * d:], xv[:, nq * d:])        # K untouched without NORM_K
    with pytest.raises(ValueError):
        oracle.norm_rope(bits[:, :nq * d], ssq, gq, gk, None, None, num_heads=nq,
                         num_kv_heads=0, head_dim=d, eps=1e-6, flags=NORM_K)
    with pytest.raises(ValueError):
        oracle.norm_rope(bits, ssq, gq, gk, None, None, num_heads=nq, num_kv_heads=nkv,
                         head_dim=d, eps=1e-6, flags=FUSED_ROPE)
