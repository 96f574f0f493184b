"""The ROW_MX encoders form fl32(y / s) as fl32(fl64(y * fl64(1 / s))) (one fp64 reciprocal per
row instead of an fp32 division per element).  This checks that identity on the CPU with
NumPy's IEEE arithmetic: random magnitudes, the scales the encoders actually produce
(s = fl32(amax / 448) with |y| <= amax), divisors whose significand is all ones or a power of
two, and quotients near the ends of the E4M3 range."""
import numpy as np


def _check(y, s):
    """Equal bits wherever the fp32 quotient is a finite normal number (the encoders' quotients
    are at most ~448; overflowing random pairs are skipped)."""
    with np.errstate(over="ignore", under="ignore"):
        y = np.asarray(y, np.float32)
        s = np.asarray(s, np.float32)
        ref = (y / s).astype(np.float32)                                   # IEEE fp32 divide
        got = (y.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)
    normal = np.isfinite(ref) & np.isfinite(y) & (np.abs(ref) >= np.float32(2.0 ** -126))
    bad = normal & (ref.view(np.uint32) != got.view(np.uint32))
    assert not bad.any(), (y[bad][:5], s[bad][:5])


def test_random_pairs():
    rng = np.random.default_rng(0)
    for _ in range(8):
        y = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-40, 40, 1_000_000))).astype(np.float32)
        s = np.abs(rng.standard_normal(1_000_000) * np.exp(rng.uniform(-40, 40, 1_000_000))).astype(np.float32) + np.float32(1e-30)
        _check(y, s)


def test_encoder_scales():
    rng = np.random.default_rng(1)
    for _ in range(8):
        amax = np.abs(rng.standard_normal(1_000_000) * np.exp(rng.uniform(-20, 20, 1_000_000))).astype(np.float32) + np.float32(1e-20)
        s = (amax / np.float32(448.0)).astype(np.float32)
        y = (amax * rng.uniform(-1, 1, 1_000_000)).astype(np.float32)
        _check(y, s)
        _check(amax, s)                       # the row maximum itself (quotient ~448)
        _check(-amax, s)


def test_special_significands():
    rng = np.random.default_rng(2)
    ones = np.uint32(0x007FFFFF)
    exps = rng.integers(1, 254, 200_000).astype(np.uint32) << 23
    s_all_ones = (exps | ones).view(np.float32)                          # 1.111...1 x 2^e
    s_pow2 = exps.view(np.float32)                                       # 1.0 x 2^e
    s_near = (exps | rng.integers(0x7FFF00, 0x800000, 200_000).astype(np.uint32)).view(np.float32)
    y = (rng.standard_normal(200_000) * 448).astype(np.float32)
    with np.errstate(over="ignore"):
        for s in (s_all_ones, s_pow2, s_near):
            _check(y * s / np.float32(448.0), s)
            _check(np.nextafter(y, np.float32(np.inf)) * s, s)
