"""Pins of the oracle's number formats against torch's independent FP8 / bf16 codecs and
exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes, allow_nan=True)
    ref = torch_e4m3(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    assert np.isnan(ours[[0x7F, 0xFF]]).all() and np.isnan(ours).sum() == 2


def test_e4m3_spot_values():
    v = codecs.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x00, 0x80, 0x07], np.uint8))
    assert list(v[:5]) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0]
    assert v[5] == 0.0 and np.signbit(v[6]) and v[7] == 7 * 2.0 ** -9
    with pytest.raises(ValueError):
        codecs.e4m3_decode(np.array([0x7F], np.uint8))


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ours = codecs.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(ours, ref)
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127
    with pytest.raises(ValueError):
        codecs.e8m0_decode(np.array([255], np.uint8))


def _encode_probe_values(rng):
    pos = codecs.E4M3_VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                      # exact ties (all fp32-representable)
    vals = [pos, mids]
    for k in (1, 2, 3):                                  # just below / above each tie
        vals.append(np.nextafter(mids.astype(np.float32), np.float32(0), dtype=np.float32)
                    .astype(np.float64))
        vals.append(np.nextafter(mids.astype(np.float32), np.float32(1e9), dtype=np.float32)
                    .astype(np.float64))
    vals.append(np.abs(rng.standard_normal(20000)) * 40)
    vals.append(np.abs(rng.standard_normal(5000)) * 2.0 ** -7)   # subnormal range
    vals.append(np.array([0.0, 2.0 ** -10, 2.0 ** -10 * 1.0001, 463.9, 456.0, 460.0]))
    v = np.concatenate(vals).astype(np.float32)
    v = v[v < 464.0]                                     # torch's cast is non-saturating above
    return np.concatenate([v, -v])


def test_e4m3_encode_matches_torch_rne_below_464():
    rng = np.random.default_rng(0)
    v = _encode_probe_values(rng)
    ours = codecs.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 464.0, 470.0, 1e4, 3e38, -500.0, -1e30], np.float32)
    assert list(codecs.e4m3_encode(v)) == [0x7E] * 5 + [0xFE] * 2
    z = codecs.e4m3_encode(np.array([-0.0, -1e-6, 0.0, 1e-6], np.float32))
    assert list(z) == [0x80, 0x80, 0x00, 0x00]
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([np.nan], np.float32))


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # exact ties: low half 0x8000 with both parities of bit 16
    tie_bits = (rng.integers(0, 2 ** 16, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    t = tie_bits.view(np.float32)
    x = np.concatenate([x, t[np.isfinite(t)]]).astype(np.float32)
    ours = codecs.bf16_round_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _exact_bf16_round(x: float) -> int:
    """Brute force: nearest bf16 to the rational value of x, ties to even."""
    fx = Fraction(x)
    a = abs(fx)
    # bracket among positive bf16 patterns by bisection over the 0x0000..0x7F80 range
    def val(b):
        return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))
    lo, hi = 0, 0x7F80
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if val(mid) <= a:
            lo = mid
        else:
            hi = mid
    dl, dh = a - val(lo), val(hi) - a
    b = lo if (dl < dh or (dl == dh and lo % 2 == 0)) else hi
    return b | (0x8000 if x < 0 or (x == 0 and np.signbit(x)) else 0)


def test_f64_to_bf16_single_rounding_brute_force():
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(300) * 10.0 ** rng.integers(-20, 20, 300))
    # values 1 fp64-ulp off a bf16 tie: a double rounding through fp32 would get these wrong
    for b in (0x3F80, 0x4049, 0x3C01):
        tie = float(np.array([(b << 16) | 0x8000], np.uint32).view(np.float32)[0])
        xs += [np.nextafter(tie, 0.0), np.nextafter(tie, 1e9), tie]
    xs = np.array(xs)
    ours = codecs.f64_to_bf16(xs)
    ref = np.array([_exact_bf16_round(float(v)) for v in xs], np.uint16)
    assert np.array_equal(ours, ref)
