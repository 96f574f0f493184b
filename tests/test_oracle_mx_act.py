"""Pins of the oracle's MX block-32 activation path ([RMSNORM-MX] qmx_output_dtype /
emit_norm_bf16): the block exponent rule and codes against an independent formula and torch's
fp8 cast, the decode, the projection with per-block activation exponents against exact rational
brute force and against the ROW_MX form when every block of a row shares one exponent, and the
bf16 norm output against torch's RMSNorm."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import codecs


def test_mx_block_exponents_and_codes():
    rng = np.random.default_rng(40)
    T, H = 12, 128
    y = rng.standard_normal((T, H)).astype(np.float32)
    y[3, 32:64] = 0                                               # an all-zero block
    y[5, 64:96] *= 1e-30                                          # tiny block
    y[7] *= 300.0                                                 # large row
    codes, e8 = oracle.mx_block_quantize(y)
    assert codes.shape == (T, H) and e8.shape == (T, H // 32)
    assert e8[3, 1] == 0 and (codes[3, 32:64] == 0).all()
    blocks = y.reshape(T, H // 32, 32).astype(np.float64)
    amax = np.abs(blocks).max(2)
    nz = amax > 0
    # independent: E - 127 = floor(log2 amax) - 8, clamped to the E8M0 range
    X = np.clip(np.floor(np.log2(amax[nz])) - 8, -127, 127).astype(np.int64)
    assert np.array_equal(e8[nz].astype(np.int64) - 127, X)
    # codes = torch RNE cast of y / 2^X (saturated at 448), zero blocks zero
    scale = np.repeat(np.ldexp(1.0, np.where(nz, e8.astype(np.int64) - 127, 0)), 32, 1)
    v = (y / scale).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    big = np.abs(v) >= 464
    ref[big] = np.where(v[big] > 0, 0x7E, 0xFE)
    ref[np.repeat(~nz, 32, 1)] = 0
    assert np.array_equal(codes, ref)
    # decode = codes * 2^(E - 127) exactly; every non-zero block's largest code in [256, 448]
    dec = oracle.mx_block_decode(codes, e8)
    assert np.array_equal(dec, codecs.e4m3_decode(codes) * scale)
    mags = codecs.e4m3_decode(codes & 0x7F).reshape(T, H // 32, 32).max(2)
    assert ((mags[nz] >= 256) & (mags[nz] <= 448)).all()


def test_project_with_block_exponents_exact_rational():
    rng = np.random.default_rng(41)
    T, H, nq, nkv, d = 2, 64, 1, 1, 2
    I = (nq + 2 * nkv) * d
    a = rng.integers(0, 256, (T, H), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    ea = rng.integers(115, 135, (T, H // 32)).astype(np.uint8)
    wn = rng.integers(0, 256, (H, I), dtype=np.uint8)
    wn[(wn & 0x7F) == 0x7F] = 0x38
    ew = rng.integers(115, 135, (H // 32, I)).astype(np.uint8)
    w4 = wn.reshape(H // 4, 4, I).transpose(0, 2, 1).copy()
    b = codecs.f64_to_bf16(rng.standard_normal(I))
    X, _ = oracle.project(a, None, w4, ew, None, b, num_heads=nq, num_kv_heads=nkv, head_dim=d,
                          a_e8m0=ea)
    dec = {k: Fraction(float(v)) for k, v in enumerate(
        torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist())
        if k & 0x7F != 0x7F}
    for s in range(T):
        for i in range(I):
            terms = [dec[int(a[s, h])] * Fraction(2) ** (int(ea[s, h // 32]) - 127) *
                     dec[int(wn[h, i])] * Fraction(2) ** (int(ew[h // 32, i]) - 127) for h in range(H)]
            x = sum(terms) + Fraction(float(codecs.bf16_to_f64(b[i:i + 1])[0]))
            assert abs(X[s, i] - float(x)) <= 1e-12 * float(sum(abs(t) for t in terms)) + 1e-300


def test_project_equal_block_exponents_reduce_to_row_scale():
    rng = np.random.default_rng(42)
    T, H, nq, nkv, d = 5, 96, 2, 1, 8
    I = (nq + 2 * nkv) * d
    a = rng.integers(0, 256, (T, H), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x40
    Erow = rng.integers(110, 140, T).astype(np.uint8)
    ea = np.repeat(Erow[:, None], H // 32, 1)
    w, e = oracle.mx_weight_quantize((0.02 * rng.standard_normal((H, I))).astype(np.float32))
    X1, s1 = oracle.project(a, None, w, e, None, None, num_heads=nq, num_kv_heads=nkv, head_dim=d,
                            a_e8m0=ea)
    X2, s2 = oracle.project(a, np.ldexp(1.0, Erow.astype(np.int64) - 127).astype(np.float32), w, e,
                            None, None, num_heads=nq, num_kv_heads=nkv, head_dim=d)
    assert np.array_equal(X1, X2) and np.array_equal(s1, s2)


def test_mx_producer_norm_bf16_matches_torch_rmsnorm():
    rng = np.random.default_rng(43)
    T, H = 16, 256
    hid = codecs.f64_to_bf16(rng.standard_normal((T, H)))
    res = codecs.f64_to_bf16(0.5 * rng.standard_normal((T, H)))
    gam = codecs.f64_to_bf16(1 + 0.1 * rng.standard_normal(H))
    r_out, codes, e8, norm, y = oracle.rmsnorm_mx(hid, res, gam, 1e-6)
    # the same steps 1-4 as the ROW_MX producer
    r2, _, y2 = oracle.rmsnorm_rowmx(hid, res, gam, 1e-6)
    assert np.array_equal(r_out, r2) and np.array_equal(y, y2)
    assert np.array_equal((codes, e8)[0], oracle.mx_block_quantize(y)[0])
    # emit_norm_bf16: matches torch's fp32 RMSNorm of the bf16 sum, cast to bf16 (within one
    # bf16 step: torch sums in fp32 and multiplies in another order)
    r_t = torch.from_numpy(codecs.bf16_to_f64(r_out).astype(np.float32))
    g_t = torch.from_numpy(codecs.bf16_to_f64(gam).astype(np.float32))
    ref = torch.nn.functional.rms_norm(r_t, (H,), g_t, eps=1e-6).to(torch.bfloat16).float().numpy()
    got = codecs.bf16_to_f64(norm)
    assert (np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30).all()
    # and it is exactly the bf16 rounding of the fp32 normed value
    assert np.array_equal(norm, codecs.bf16_round_f32(y))
