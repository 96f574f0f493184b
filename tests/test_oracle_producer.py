"""Pins of the oracle's encoders: ROW_MX rows, the residual+RMSNorm producer and MX block-32
weights, against torch's casts / RMSNorm, high-precision arithmetic and the format invariants."""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import codecs


def test_rowmx_codes_equal_torch_cast_of_scaled_rows():
    rng = np.random.default_rng(30)
    y = (rng.standard_normal((64, 256)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    y[3, 17] = -0.0
    y[5] = 0.0                                                      # all-zero row
    packed = oracle.rowmx_quantize(y)
    codes, s = oracle.rowmx_unpack(packed, 256)
    amax = np.abs(y).max(1)
    assert np.array_equal(s, (torch.from_numpy(amax) / 448.0).numpy())   # fp32 IEEE division
    nz = s > 0
    v = torch.from_numpy(y[nz]) / torch.from_numpy(s[nz])[:, None]
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[nz], ref)
    assert (codes[5] == 0).all() and s[5] == 0
    # the row maximum encodes to +-448, and s >= 0
    idx = np.argmax(np.abs(y), 1)
    top = codes[np.arange(64), idx][nz]
    assert set(np.unique(top & 0x7F)) == {0x7E}
    # tail is little-endian fp32
    assert np.array_equal(packed[:, 256:].copy().view("<f4").ravel(), s)


def test_rowmx_round_trip_error_bound():
    rng = np.random.default_rng(31)
    y = (rng.standard_normal((32, 512)) * 5).astype(np.float32)
    codes, s = oracle.rowmx_unpack(oracle.rowmx_quantize(y), 512)
    deq = codecs.e4m3_decode(codes) * s[:, None].astype(np.float64)
    err = np.abs(deq - y)
    sub = (codes & 0x78) == 0
    assert (err[~sub] <= 2.0 ** -4 * np.abs(y[~sub]) * (1 + 1e-6)).all()
    assert (err[sub] <= (2.0 ** -10 * s[:, None] * np.ones_like(y))[sub] * (1 + 1e-6)).all()


def _hp_inv(ss: float, hu: int, eps32: float) -> float:
    getcontext().prec = 60
    v = Decimal(ss) / Decimal(hu) + Decimal(eps32)
    return float(1 / v.sqrt())


def test_producer_residual_norm_and_encode():
    rng = np.random.default_rng(32)
    T, H = 24, 320
    hid = synth.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    res = synth.to_bf16_bits((0.5 * rng.standard_normal((T, H))).astype(np.float32))
    gam = synth.to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    eps = 1e-6
    res_out, packed, y = oracle.rmsnorm_rowmx(hid, res, gam, eps)
    th = torch.from_numpy(hid.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(res.view(np.int16)).view(torch.bfloat16)
    ref_sum = (th.float() + tr.float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(res_out, ref_sum)                          # bit-exact
    r = codecs.bf16_to_f64(res_out)
    g = codecs.bf16_to_f64(gam)
    e32 = float(np.float32(eps))
    ref_y = torch.nn.functional.rms_norm(torch.from_numpy(r), (H,), weight=torch.from_numpy(g),
                                         eps=e32).numpy()
    assert np.allclose(y, ref_y, rtol=2.5e-7, atol=0)               # two fp32 roundings
    # inv: fp32 rounding of the exact value (high-precision decimal)
    ss = np.sum(r * r, 1)
    for t in range(T):
        inv_hp = _hp_inv(float(ss[t]), H, e32)
        inv32 = np.float32(inv_hp)
        yt = ((r[t].astype(np.float32) * inv32).astype(np.float32) * g.astype(np.float32)).astype(np.float32)
        assert np.array_equal(yt, y[t])
    codes, s = oracle.rowmx_unpack(packed, H)
    assert np.array_equal(packed, oracle.rowmx_quantize(y))
    assert (s > 0).all()


def test_producer_without_residual_and_padding():
    rng = np.random.default_rng(33)
    T, H, Hu = 8, 128, 96
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, Hu:] = 0
    hid = synth.to_bf16_bits(x)
    gam = synth.to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    ro, packed, y = oracle.rmsnorm_rowmx(hid, None, gam, 1e-6, unpadded_h=Hu)
    assert ro is None
    ro2, packed2, y2 = oracle.rmsnorm_rowmx(hid[:, :Hu], None, gam[:Hu], 1e-6)
    assert np.array_equal(y[:, :Hu], y2)                           # zero pad does not skew the mean
    assert np.array_equal(packed[:, :Hu], packed2[:, :Hu])
    with pytest.raises(ValueError):
        oracle.rmsnorm_rowmx(hid, None, gam, 1e-6, unpadded_h=H + 1)


def test_mx_weight_shared_exponent_rule():
    rng = np.random.default_rng(34)
    H, I = 128, 40
    w = (0.02 * rng.standard_normal((H, I))).astype(np.float32)
    w[32:64, 5] = 0                                                 # an all-zero block
    w[0:32, 7] *= 1e-3
    codes, e8 = oracle.mx_weight_quantize(w)
    assert codes.shape == (H // 4, I, 4) and e8.shape == (H // 32, I)
    assert e8[1, 5] == 0 and (codes[8:16, 5, :] == 0).all()
    wd = oracle.mx_weight_decode(codes, e8)
    blocks = w.reshape(H // 32, 32, I).astype(np.float64)
    amax = np.abs(blocks).max(1)
    nz = amax > 0
    X = np.floor(np.log2(amax[nz])) - 8                              # independent formula
    assert np.array_equal(e8[nz].astype(np.int64) - 127, X.astype(np.int64))
    nat = codes.transpose(0, 2, 1).reshape(H, I)
    mags = codecs.e4m3_decode(nat & 0x7F).reshape(H // 32, 32, I).max(1)
    assert ((mags[nz] >= 256) & (mags[nz] <= 448)).all()
    # codes = torch RNE cast of w / 2^X where |w / 2^X| < 464, else saturated to 448
    scale = np.repeat(np.ldexp(1.0, np.where(nz, e8.astype(np.int64) - 127, 0)), 32, 0)
    v = (w / scale).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    big = np.abs(v) >= 464
    ref[big] = np.where(v[big] > 0, 0x7E, 0xFE)
    zero_blk = np.repeat(~nz, 32, 0)
    ref[zero_blk] = 0
    assert np.array_equal(nat, ref)
    # round trip: half an E4M3 step (2^-4 relative for normal codes, 2^-10 * 2^X for subnormal)
    ok = ~zero_blk & (np.abs(v) <= 448)
    sub = (nat & 0x78) == 0
    err = np.abs(wd - w)
    assert (err[ok & ~sub] <= 2.0 ** -4 * np.abs(w[ok & ~sub])).all()
    assert (err[ok & sub] <= scale[ok & sub] * 2.0 ** -10).all()
    sat = ~zero_blk & (np.abs(v) > 448)
    assert np.array_equal(np.abs(wd[sat]), 448 * scale[sat])
