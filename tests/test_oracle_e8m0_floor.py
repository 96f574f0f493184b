"""Pins of the E8M0 floor clamp in the oracle's MX encoders (weights and MX block-32
activations).

The shared exponent of a block is E = floor(log2 amax) - 8 + 127, clamped to the finite E8M0
range [0, 254] (the OCP MX v1.0 rule read for both encoders).  The lower clamp acts only for
blocks whose largest magnitude is below 2^-119, i.e. fp32 values near the bottom of the normal
range and fp32 subnormals.  The expected exponents here come from exact rational arithmetic
(the largest k with 2^k <= amax, found by repeated doubling / halving of a Fraction), not from
the oracle's frexp; the expected codes from torch's RNE E4M3 cast of the block divided by
2^(E - 127), which is exact in fp32 for every block below.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
from gpu_common import floor_blocks
from oracle import codecs


def exact_floor_log2(v: float) -> int:
    """Largest integer k with 2^k <= v, for a positive finite v, in exact rationals."""
    x = Fraction(v)
    k = 0
    while Fraction(2) ** k > x:
        k -= 1
    while Fraction(2) ** (k + 1) <= x:
        k += 1
    return k


def expected_block(vals: np.ndarray):
    """(E, codes) of one 32-element fp32 block by the rule above, independently of the oracle."""
    amax = float(np.max(np.abs(vals.astype(np.float64))))
    if amax == 0.0:
        return 0, np.zeros(32, np.uint8)
    E = min(max(exact_floor_log2(amax) - 8 + 127, 0), 254)
    # power-of-two rescale (keeps the sign of -0.0); exactness checked in rationals
    v32 = np.ldexp(vals.astype(np.float64), 127 - E).astype(np.float32)
    assert all(Fraction(float(a)) == Fraction(float(v)) / Fraction(2) ** (E - 127)
               for a, v in zip(v32, vals)), "rescale not exact"
    c = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    big = np.abs(v32) >= 464                      # torch's cast gives NaN there; satfinite clamps
    c[big] = np.where(v32[big] > 0, 0x7E, 0xFE)
    return E, c


def test_floor_log2_helper_is_exact():
    for k in (-149, -127, -126, -120, -119, -1, 0, 1, 127):
        v = float(np.float32(2.0 ** k))
        assert exact_floor_log2(v) == k
        if k > -149:
            assert exact_floor_log2(float(np.nextafter(np.float32(v), np.float32(0)))) == k - 1


def test_weight_encoder_floor_clamp():
    rng = np.random.default_rng(90)
    blocks = floor_blocks(rng)
    I = len(blocks)
    w = np.stack(blocks, axis=1).astype(np.float32)            # [32, I]: block j = column j
    w = np.concatenate([w, (0.02 * rng.standard_normal((32, I))).astype(np.float32)])  # H = 64
    codes, e8 = oracle.mx_weight_quantize(w)
    nat = codes.transpose(0, 2, 1).reshape(64, I)              # element (h, i)
    for j, blk in enumerate(blocks):
        E, c = expected_block(blk)
        assert e8[0, j] == E, (j, e8[0, j], E)
        assert np.array_equal(nat[:32, j], c), j
    # the clamp is reached: every block below 2^-119 has E = 0
    amax = np.abs(w[:32].astype(np.float64)).max(0)
    assert (e8[0][(amax > 0) & (amax < 2.0 ** -119)] == 0).all()
    assert ((amax > 0) & (amax < 2.0 ** -119)).sum() >= 5
    assert e8[0, 6] == 0 and e8[0, 8] == 1                     # 2^-119 -> 0 (exact), 2^-118 -> 1
    # decoding gives back each value to within half an E4M3 step at scale 2^-127
    dec = oracle.mx_weight_decode(codes, e8)[:32]
    err = np.abs(dec - w[:32].astype(np.float64))
    assert (err[:, e8[0] == 0] <= 2.0 ** -10 * 2.0 ** -127 + 2.0 ** -4 * np.abs(w[:32, e8[0] == 0])).all()


def test_mx_activation_encoder_floor_clamp():
    rng = np.random.default_rng(91)
    blocks = floor_blocks(rng)
    T = len(blocks)
    y = np.stack(blocks).astype(np.float32)                    # row j = block j (H = 32)
    y = np.concatenate([y, (rng.standard_normal((T, 32)) * 1e-3).astype(np.float32)], axis=1)
    codes, e8 = oracle.mx_block_quantize(y)
    for j, blk in enumerate(blocks):
        E, c = expected_block(blk)
        assert e8[j, 0] == E, (j, e8[j, 0], E)
        assert np.array_equal(codes[j, :32], c), j
    assert (e8[:, 0] == 0).sum() >= 6
    # signs survive on values that round to zero at the floor scale
    j = 2                                                      # +-2^-149 block
    neg = blocks[j] < 0
    assert (codes[j, :32][neg] == 0x80).all() and (codes[j, :32][~neg] == 0x00).all()
    # exact decode: code value times 2^(E - 127)
    dec = oracle.mx_block_decode(codes, e8)
    assert np.array_equal(dec[:, :32], codecs.e4m3_decode(codes[:, :32]) *
                          np.ldexp(1.0, e8[:, :1].astype(np.int64) - 127))
