"""The input recipe: determinism, row-subset regeneration and the rotary caches' closed forms."""
import math

import numpy as np

import synth


def test_row_subset_regenerates_same_rows():
    p = synth.CONFIGS[1].calls[0]
    full = synth.activation(p)
    idx = np.array([0, 5, 127, 64])
    assert np.array_equal(synth.activation(p, row_idx=idx), full[idx])
    assert synth.digest(full) == synth.digest(synth.activation(p))


def test_outliers_scale_fixed_channel_set():
    p = synth.CONFIGS[3].calls[0]
    ch = synth.outlier_channels(p)
    assert len(ch) == 51 and len(set(ch)) == 51
    q = synth.CONFIGS[4].calls[0]
    assert np.array_equal(synth.outlier_channels(q), ch)            # C4 latent = C3 latent
    x = synth.activation(p, row_idx=np.arange(8))
    xq = synth.activation(q, row_idx=np.arange(8))
    assert np.array_equal(x, xq)
    others = np.setdiff1d(np.arange(p.H), ch)
    assert np.abs(x[:, ch]).mean() > 10 * np.abs(x[:, others]).mean()


def test_rope_1d_textbook_values():
    d = 64
    cos, sin = synth.rope_1d(np.array([0, 1, 127]), d)
    assert np.all(cos[0] == 1) and np.all(sin[0] == 0)
    for p_i, p in enumerate([0, 1, 127]):
        for j in (0, 5, 31):
            a = p * 10000.0 ** (-2 * j / d)
            assert abs(cos[p_i, j] - math.cos(a)) < 1e-7 and abs(sin[p_i, j] - math.sin(a)) < 1e-7
            assert cos[p_i, j] == cos[p_i, j + d // 2] and sin[p_i, j] == sin[p_i, j + d // 2]
    assert np.allclose(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2, 1, atol=1e-6)


def test_rope_3d_axis_bands():
    grid = (21, 45, 80)
    d = 128
    t = np.array([0, 1, 80, 3600, 75599])
    ang = synth.rope_3d_angles(t, grid, d)
    assert ang.shape == (5, 64) and np.all(ang[0] == 0)
    # token 1 = (0,0,1): only the width band (pairs 43..63) moves
    assert np.all(ang[1, :43] == 0) and np.all(ang[1, 43:] > 0)
    # token 80 = (0,1,0): only the height band (pairs 22..42)
    assert np.all(ang[2, :22] == 0) and np.all(ang[2, 22:43] > 0) and np.all(ang[2, 43:] == 0)
    # token 3600 = (1,0,0): only the frame band (pairs 0..21)
    assert np.all(ang[3, :22] > 0) and np.all(ang[3, 22:] == 0)
    # last token (20, 44, 79); pair 0 of each band rotates by the coordinate itself
    assert ang[4, 0] == 20 and ang[4, 22] == 44 and ang[4, 43] == 79
    assert math.isclose(ang[4, 1], 20 * 10000.0 ** (-2 / 44))
    assert math.isclose(ang[4, 23], 44 * 10000.0 ** (-2 / 42))
    cos, sin = synth.rope_3d(t, grid, d)
    assert np.array_equal(cos[:, :64], cos[:, 64:])
    assert np.allclose(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2, 1, atol=1e-6)
