"""Pins of oracle.layouts: the NBSd layout ([QKV-CTE] "Interface": output_layout NBSd
[num_heads, B, S, d_head]) against its index formula, element by element."""
import numpy as np

import oracle


def test_nbsd_index_formula_brute_force():
    # distinct values everywhere, so any transposed or shifted index shows up
    T, nh, d = 5, 7, 4
    x = np.arange(T * nh * d, dtype=np.float64).reshape(T, nh * d) * 1.5 + 0.25
    y = oracle.bsd_to_nbsd(x, d)
    assert y.shape == (nh, T, d)
    flat = y.reshape(-1)
    for t in range(T):
        for h in range(nh):
            for j in range(d):
                # NBSd element (h, t, j) lives at flat offset (h * T + t) * d + j and holds BSD
                # column h * d + j of token t
                assert flat[(h * T + t) * d + j] == x[t, h * d + j]


def test_nbsd_round_trip_and_segments():
    rng = np.random.default_rng(0)
    T, nq, nkv, d = 9, 3, 2, 16
    I = (nq + 2 * nkv) * d
    x = rng.standard_normal((T, I))
    y = oracle.bsd_to_nbsd(x, d)
    assert np.array_equal(oracle.nbsd_to_bsd(y), x)
    # heads in column order: Q heads first, then K, then V
    assert np.array_equal(y[:nq].transpose(1, 0, 2).reshape(T, nq * d), x[:, :nq * d])
    assert np.array_equal(y[nq + nkv:].transpose(1, 0, 2).reshape(T, nkv * d), x[:, (nq + nkv) * d:])


def test_nbsd_rejects_partial_heads():
    import pytest
    with pytest.raises(ValueError):
        oracle.bsd_to_nbsd(np.zeros((2, 10)), 4)
