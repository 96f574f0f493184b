"""Pins of the oracle's projection (pass 1) and its segment sums of squares: exact rational
brute force, torch's fp8 decode + fp64 matmul, closed forms and the pages' weight layout."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes in inputs
    return c


def _to_h4i4(nat):
    """[H, I] -> the pages' [H // 4, I, 4] layout, written as the flat-address formula
    ((h // 4) * I + i) * 4 + h % 4 with explicit loops (independent of the oracle's reshape)."""
    H, I = nat.shape
    flat = np.zeros(H * I, np.uint8)
    for h in range(H):
        for i in range(I):
            flat[((h // 4) * I + i) * 4 + h % 4] = nat[h, i]
    return flat.reshape(H // 4, I, 4)


def _case(rng, T=3, H=64, nq=1, nkv=1, d=2):
    I = (nq + 2 * nkv) * d
    a = _rand_codes(rng, (T, H))
    sa = (np.abs(rng.standard_normal(T)) + 0.1).astype(np.float32)
    wn = _rand_codes(rng, (H, I))
    e = rng.integers(110, 140, (H // 32, I)).astype(np.uint8)
    c = (np.abs(rng.standard_normal(I)) + 0.5).astype(np.float32)
    b = codecs.f64_to_bf16(rng.standard_normal(I))
    return a, sa, wn, e, c, b, (nq, nkv, d)


def test_project_matches_exact_rational_brute_force():
    rng = np.random.default_rng(10)
    a, sa, wn, e, c, b, (nq, nkv, d) = _case(rng)
    X, ssq = oracle.project(a, sa, _to_h4i4(wn), e, c, b, num_heads=nq, num_kv_heads=nkv,
                            head_dim=d)
    T, H = a.shape
    I = wn.shape[1]
    dec = {k: Fraction(float(v)) for k, v in enumerate(
        torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist())
        if k & 0x7F != 0x7F}
    for s in range(T):
        exact_row = []
        for i in range(I):
            terms = [dec[int(a[s, h])] * dec[int(wn[h, i])] * Fraction(2) ** (int(e[h // 32, i]) - 127)
                     for h in range(H)]
            x = Fraction(float(sa[s])) * Fraction(float(c[i])) * sum(terms) + \
                Fraction(float(codecs.bf16_to_f64(b[i:i + 1])[0]))
            bound = 1e-12 * float(sum(abs(t) for t in terms) * Fraction(float(sa[s])) *
                                  Fraction(float(c[i]))) + 1e-300
            assert abs(X[s, i] - float(x)) <= bound
            exact_row.append(x)
        q = sum(v * v for v in exact_row[: nq * d])
        k = sum(v * v for v in exact_row[nq * d: (nq + nkv) * d])
        assert abs(ssq[s, 0] - float(q)) <= 1e-12 * float(q)
        assert abs(ssq[s, 1] - float(k)) <= 1e-12 * float(k)


def test_project_unit_scales_equal_torch_matmul():
    rng = np.random.default_rng(11)
    T, H, nq, nkv, d = 17, 96, 2, 1, 8
    I = (nq + 2 * nkv) * d
    a = _rand_codes(rng, (T, H))
    wn = _rand_codes(rng, (H, I))
    e = np.full((H // 32, I), 127, np.uint8)
    X, _ = oracle.project(a, np.ones(T, np.float32), _to_h4i4(wn), e, None, None,
                          num_heads=nq, num_kv_heads=nkv, head_dim=d)
    ta = torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    tw = torch.from_numpy(wn).view(torch.float8_e4m3fn).double()
    ref = (ta @ tw).numpy()
    assert np.allclose(X, ref, rtol=1e-13, atol=1e-13)


def test_project_one_hot_row_is_dequantised_weight_row():
    rng = np.random.default_rng(12)
    a, sa, wn, e, c, b, (nq, nkv, d) = _case(rng, T=4, H=64)
    T, H = a.shape
    a[:] = 0
    js = [0, 31, 32, 63]
    for s, j in enumerate(js):
        a[s, j] = 0x38                       # 1.0
    X, _ = oracle.project(a, sa, _to_h4i4(wn), e, c, b, num_heads=nq, num_kv_heads=nkv,
                          head_dim=d)
    wv = torch.from_numpy(wn).view(torch.float8_e4m3fn).double().numpy()
    for s, j in enumerate(js):
        expect = float(sa[s]) * c.astype(np.float64) * wv[j] * 2.0 ** (e[j // 32].astype(np.int64) - 127) \
            + codecs.bf16_to_f64(b)
        assert np.allclose(X[s], expect, rtol=1e-15, atol=0)


def test_weight_layout_single_byte_lands_at_its_column():
    """A single nonzero byte at flat address ((h // 4) * I + i) * 4 + h % 4 of the [H//4, I, 4]
    weight contributes A[:, h] to output column i only."""
    rng = np.random.default_rng(13)
    T, H, I = 5, 64, 12
    a = _rand_codes(rng, (T, H))
    av = codecs.e4m3_decode(a)
    for (h, i) in [(0, 0), (5, 7), (33, 11), (63, 3), (2, 9)]:
        flat = np.zeros(H * I, np.uint8)
        flat[((h // 4) * I + i) * 4 + h % 4] = 0x40      # 2.0
        X, _ = oracle.project(a, np.ones(T, np.float32), flat.reshape(H // 4, I, 4),
                              np.full((H // 32, I), 127, np.uint8), num_heads=2, num_kv_heads=1,
                              head_dim=3)
        expect = np.zeros((T, I))
        expect[:, i] = 2.0 * av[:, h]
        assert np.array_equal(X, expect)


def test_bias_linearity_and_channel_scale():
    rng = np.random.default_rng(14)
    a, sa, wn, e, c, b, (nq, nkv, d) = _case(rng, T=6, H=64, nq=2, nkv=1, d=4)
    w = _to_h4i4(wn)
    X0, _ = oracle.project(a, sa, w, e, c, None, num_heads=nq, num_kv_heads=nkv, head_dim=d)
    X1, _ = oracle.project(a, sa, w, e, c, b, num_heads=nq, num_kv_heads=nkv, head_dim=d)
    assert np.allclose(X1 - X0, codecs.bf16_to_f64(b)[None, :], rtol=0, atol=1e-12)
    Xn, _ = oracle.project(a, sa, w, e, None, None, num_heads=nq, num_kv_heads=nkv, head_dim=d)
    assert np.allclose(X0, Xn * c[None, :].astype(np.float64), rtol=1e-14)


def test_ssq_excludes_v_and_handles_single_segment():
    rng = np.random.default_rng(15)
    nq, nkv, d = 2, 1, 4
    a, sa, wn, e, c, b, _ = _case(rng, T=5, H=64, nq=nq, nkv=nkv, d=d)
    w = _to_h4i4(wn)
    X, ssq = oracle.project(a, sa, w, e, c, b, num_heads=nq, num_kv_heads=nkv, head_dim=d)
    wn2 = wn.copy()
    wn2[:, (nq + nkv) * d:] = _rand_codes(rng, (wn.shape[0], nkv * d))   # change V only
    X2, ssq2 = oracle.project(a, sa, _to_h4i4(wn2), e, c, b, num_heads=nq, num_kv_heads=nkv,
                              head_dim=d)
    assert not np.array_equal(X[:, (nq + nkv) * d:], X2[:, (nq + nkv) * d:])
    assert np.array_equal(ssq, ssq2)
    assert (ssq >= 0).all() and (ssq.sum(1) <= (X ** 2).sum(1) * (1 + 1e-12)).all()
    # single-segment call: the whole output is "Q", the K sum is 0
    Xq, ssq_q = oracle.project(a, sa, _to_h4i4(wn[:, :8]), e[:, :8], c[:8], b[:8],
                               num_heads=2, num_kv_heads=0, head_dim=4)
    assert np.all(ssq_q[:, 1] == 0)
    assert np.allclose(ssq_q[:, 0], (Xq ** 2).sum(1), rtol=1e-14)
    with pytest.raises(ValueError):
        oracle.project(a, sa, w, e, num_heads=3, num_kv_heads=1, head_dim=d)


def test_abs_term_sum_pins():
    """abs_term_sum: exact rational brute force of sum_h |a_h w_h| 2^(E - 127) times |sA c| on a
    tiny shape (with negative scales and MX activation exponents); equal to X - bias when every
    code is non-negative; never below |X - bias| (triangle inequality)."""
    rng = np.random.default_rng(70)
    T, H, nq, nkv, d = 3, 64, 1, 1, 2
    I = (nq + 2 * nkv) * d
    a = _rand_codes(rng, (T, H))
    wn = _rand_codes(rng, (H, I))
    ew = rng.integers(118, 136, (H // 32, I)).astype(np.uint8)
    w4 = _to_h4i4(wn)
    sA = np.array([0.75, -2.0, 1e-3], np.float32)
    cs = np.array([1.5, -0.25, 3.0, 1.0, -1.0, 0.5], np.float32)
    S = oracle.abs_term_sum(a, sA, w4, ew, cs)
    dec = {k: Fraction(float(v)) for k, v in enumerate(
        torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist())
        if k & 0x7F != 0x7F}
    for s in range(T):
        for i in range(I):
            ref = sum(abs(dec[int(a[s, h])] * dec[int(wn[h, i])]) *
                      Fraction(2) ** (int(ew[h // 32, i]) - 127) for h in range(H))
            ref *= abs(Fraction(float(sA[s]))) * abs(Fraction(float(cs[i])))
            assert abs(S[s, i] - float(ref)) <= 1e-14 * float(ref)
    # MX activation exponents enter inside the sum
    ea = rng.integers(120, 134, (T, H // 32)).astype(np.uint8)
    S2 = oracle.abs_term_sum(a, None, w4, ew, None, a_e8m0=ea)
    for s in range(T):
        i = s % I
        ref = sum(abs(dec[int(a[s, h])] * dec[int(wn[h, i])]) *
                  Fraction(2) ** (int(ew[h // 32, i]) + int(ea[s, h // 32]) - 254) for h in range(H))
        assert abs(S2[s, i] - float(ref)) <= 1e-14 * float(ref)
    # all codes non-negative: the sum of absolute terms is the contraction itself
    ap, wp4 = a & 0x7F, w4 & 0x7F
    b = codecs.f64_to_bf16(rng.standard_normal(I))
    X, _ = oracle.project(ap, np.abs(sA), wp4, ew, np.abs(cs), b, num_heads=nq,
                          num_kv_heads=nkv, head_dim=d)
    Sp = oracle.abs_term_sum(ap, np.abs(sA), wp4, ew, np.abs(cs))
    assert np.allclose(Sp, X - codecs.bf16_to_f64(b)[None, :], rtol=1e-13, atol=0)
    # triangle inequality on signed codes
    X, _ = oracle.project(a, sA, w4, ew, cs, b, num_heads=nq, num_kv_heads=nkv, head_dim=d)
    assert (S >= np.abs(X - codecs.bf16_to_f64(b)[None, :]) * (1 - 1e-13)).all()
