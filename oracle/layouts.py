"""Output layouts of the projection ([QKV-CTE] "Upstream behavior" and "Interface":
``output_layout`` is BSD ``[B, S, I]`` or NBSd ``[num_heads, B, S, d_head]``; "Design 2)": under
NBSd each head occupies its own block of rows with d_head contiguous).

TEST INFRASTRUCTURE ONLY (see the package docstring).

B = 1 here, so BSD is ``[T, I]``.  The I columns form I / d heads in column order (the Q heads,
then the K heads, then the V heads), and the NBSd element (h, t, j) is BSD column h * d + j of
token t: a pure re-indexing, with no arithmetic.
"""
from __future__ import annotations

import numpy as np


def bsd_to_nbsd(x: np.ndarray, head_dim: int) -> np.ndarray:
    """[T, I] -> [I / head_dim, T, head_dim] (a copy)."""
    T, I = x.shape
    if I % head_dim:
        raise ValueError("I must be a multiple of head_dim")
    return np.ascontiguousarray(x.reshape(T, I // head_dim, head_dim).transpose(1, 0, 2))


def nbsd_to_bsd(y: np.ndarray) -> np.ndarray:
    """[I / d, T, d] -> [T, I] (a copy)."""
    nh, T, d = y.shape
    return np.ascontiguousarray(y.transpose(1, 0, 2).reshape(T, nh * d))
