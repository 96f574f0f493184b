"""Seeded synthetic inputs for the fused MXFP8 QKV projection workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no arithmetic of the method itself: it only draws random
numbers (fp32 / bf16 tensors) and builds the rotary cos/sin caches, which the
method takes as *inputs* ("Interface" table of the qkv_cte kernel reference:
``cos_cache`` / ``sin_cache`` are caller-supplied ``[B, S, d_head]`` rotate-half
caches).  Quantisation to ROW_MX / MX codes is the method's arithmetic and lives
on each side separately (the oracle, and the library's own kernels).

Seeding: every tensor is drawn in row chunks of ``CHUNK_ROWS`` rows from
``numpy.random.default_rng([config_id, tensor_id, chunk])``, so any subset of
rows can be regenerated on its own (used by sampled full-size parity checks).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Sequence

import numpy as np

CHUNK_ROWS = 4096

# tensor ids (second seed word)
TID_X = 0          # activation x ~ N(0,1) fp32, [T, H]
TID_W = 1          # weight ~ N(0, 0.02) fp32, [H, I]
TID_BIAS = 2       # bias ~ N(0, 0.02) -> bf16, [I]
TID_QGAMMA = 3     # 1 + N(0, 0.1) -> bf16, [Iq]
TID_KGAMMA = 4     # 1 + N(0, 0.1) -> bf16, [Ik]
TID_OUTLIER = 5    # outlier channel set
TID_HIDDEN = 6     # producer hidden ~ N(0,1) -> bf16, [T, H]
TID_RESID = 7      # producer residual ~ N(0,0.5) -> bf16, [T, H]
TID_PGAMMA = 8     # producer gamma 1 + N(0,0.1) -> bf16, [H]


@dataclasses.dataclass(frozen=True)
class Projection:
    """One call of the projection: activations [T, H] -> [T, I]."""
    name: str
    seed_id: int              # config id used for the seeds of this call's tensors
    T: int
    H: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    rope: Optional[str]       # None, "1d" or "3d"
    norm_q: bool              # across-heads RMSNorm on the first segment
    norm_k: bool              # across-heads RMSNorm on the K segment (fused calls)
    outlier_frac: float = 0.0
    outlier_gain: float = 20.0
    grid: Optional[tuple] = None   # (F, Hh, Ww) for 3d rope
    x_seed_id: Optional[int] = None  # activations drawn with another config's seed
    x_tid: int = TID_X               # tensor id of the activations
    tid_offset: int = 0              # shifts W/bias/gamma tensor ids (separate calls)

    @property
    def I(self) -> int:
        return (self.num_heads + 2 * self.num_kv_heads) * self.head_dim

    @property
    def Iq(self) -> int:
        return self.num_heads * self.head_dim

    @property
    def Ik(self) -> int:
        return self.num_kv_heads * self.head_dim


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    calls: Sequence[Projection]
    producer: bool = False    # activations come from the residual+RMSNorm+ROW_MX stage


def _mk_configs():
    c1 = Projection("tiny-self", 1, T=128, H=256, num_heads=2, num_kv_heads=2, head_dim=64,
                    rope="1d", norm_q=True, norm_k=True)
    c2 = Projection("wan-self-S4096", 2, T=4096, H=5120, num_heads=40, num_kv_heads=40,
                    head_dim=128, rope="1d", norm_q=True, norm_k=True)
    c3 = Projection("wan-self-S75600", 3, T=75600, H=5120, num_heads=40, num_kv_heads=40,
                    head_dim=128, rope="3d", norm_q=True, norm_k=True,
                    outlier_frac=0.01, grid=(21, 45, 80))
    # cross-attention: three separate single-segment calls (num_kv_heads = 0)
    c4q = Projection("wan-cross-Q", 4, T=75600, H=5120, num_heads=40, num_kv_heads=0,
                     head_dim=128, rope=None, norm_q=True, norm_k=False,
                     outlier_frac=0.01, x_seed_id=3, tid_offset=0)
    # K and V project the same 512 context tokens with their own weights
    c4k = Projection("wan-cross-K", 4, T=512, H=5120, num_heads=40, num_kv_heads=0,
                     head_dim=128, rope=None, norm_q=True, norm_k=False,
                     x_seed_id=4, x_tid=TID_X + 10, tid_offset=10)
    c4v = Projection("wan-cross-V", 4, T=512, H=5120, num_heads=40, num_kv_heads=0,
                     head_dim=128, rope=None, norm_q=False, norm_k=False,
                     x_seed_id=4, x_tid=TID_X + 10, tid_offset=20)
    c5 = dataclasses.replace(c3, name="wan-producer+self-S75600", seed_id=5, x_seed_id=None)
    return {
        1: Config(1, "C1 tiny self-attn", [c1]),
        2: Config(2, "C2 Wan-like self-attn S=4096", [c2]),
        3: Config(3, "C3 Wan-like self-attn S=75600 (21x45x80)", [c3]),
        4: Config(4, "C4 Wan-like cross-attn separate Q/K/V", [c4q, c4k, c4v]),
        5: Config(5, "C5 producer + self-attn S=75600", [c5], producer=True),
    }


CONFIGS = _mk_configs()


def _chunks(rows: int):
    for c in range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS):
        yield c, c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)


def _normal_rows(seed: Sequence[int], rows: int, cols: int, std: float,
                 row_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """N(0, std) fp32 rows, chunk-seeded.  ``row_idx`` selects a subset of rows."""
    if row_idx is None:
        out = np.empty((rows, cols), np.float32)
        for c, r0, r1 in _chunks(rows):
            g = np.random.default_rng(list(seed) + [c])
            out[r0:r1] = g.standard_normal((r1 - r0, cols), dtype=np.float32)
    else:
        row_idx = np.asarray(row_idx, dtype=np.int64)
        out = np.empty((len(row_idx), cols), np.float32)
        for c in np.unique(row_idx // CHUNK_ROWS):
            r0 = int(c) * CHUNK_ROWS
            r1 = min(rows, r0 + CHUNK_ROWS)
            g = np.random.default_rng(list(seed) + [int(c)])
            blk = g.standard_normal((r1 - r0, cols), dtype=np.float32)
            sel = (row_idx // CHUNK_ROWS) == c
            out[sel] = blk[row_idx[sel] - r0]
    if std != 1.0:
        out *= np.float32(std)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round-to-nearest-even, via torch's cast) as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(p: Projection) -> np.ndarray:
    """Channel set scaled by ``outlier_gain``: round(frac * H) channels, drawn once per seed."""
    n = int(round(p.outlier_frac * p.H))
    if n == 0:
        return np.zeros(0, np.int64)
    sid = p.x_seed_id if p.x_seed_id is not None else p.seed_id
    g = np.random.default_rng([sid, TID_OUTLIER])
    return np.sort(g.choice(p.H, size=n, replace=False))


def activation(p: Projection, row_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """x ~ N(0,1) fp32 [T, H] (or the rows ``row_idx``), with the outlier channels x gain."""
    sid = p.x_seed_id if p.x_seed_id is not None else p.seed_id
    x = _normal_rows([sid, p.x_tid], p.T, p.H, 1.0, row_idx)
    ch = outlier_channels(p)
    if len(ch):
        x[:, ch] *= np.float32(p.outlier_gain)
    return x


def weight(p: Projection, std: float = 0.02) -> np.ndarray:
    """W ~ N(0, std) fp32 in natural [H, I] orientation."""
    return _normal_rows([p.seed_id, TID_W + p.tid_offset], p.H, p.I, std)


def bias_bf16(p: Projection) -> np.ndarray:
    g = np.random.default_rng([p.seed_id, TID_BIAS + p.tid_offset])
    return to_bf16_bits(g.standard_normal(p.I, dtype=np.float32) * np.float32(0.02))


def gamma_bf16(p: Projection, which: str) -> Optional[np.ndarray]:
    """Segment-wide gamma 1 + N(0, 0.1) as bf16 ([Iq] for 'q', [Ik] for 'k')."""
    n = p.Iq if which == "q" else p.Ik
    if n == 0:
        return None
    tid = (TID_QGAMMA if which == "q" else TID_KGAMMA) + p.tid_offset
    g = np.random.default_rng([p.seed_id, tid])
    return to_bf16_bits(np.float32(1.0) + g.standard_normal(n, dtype=np.float32) * np.float32(0.1))


def producer_inputs(cid: int, T: int, H: int, row_idx: Optional[np.ndarray] = None):
    """Producer inputs: hidden ~ N(0,1), residual ~ N(0,0.5) (both fp32 -> bf16), gamma [H]."""
    hid = to_bf16_bits(_normal_rows([cid, TID_HIDDEN], T, H, 1.0, row_idx))
    res = to_bf16_bits(_normal_rows([cid, TID_RESID], T, H, 0.5, row_idx))
    g = np.random.default_rng([cid, TID_PGAMMA])
    gam = to_bf16_bits(np.float32(1.0) + g.standard_normal(H, dtype=np.float32) * np.float32(0.1))
    return hid, res, gam


# ----------------------------------------------------------------------------------------------
# Rotary caches (caller inputs).  Rotate-half convention: lane j pairs with lane j + d/2 and
# both lanes of a pair carry the same angle ("Design 2" of the qkv_cte kernel reference).
# ----------------------------------------------------------------------------------------------

def rope_1d(positions: np.ndarray, d: int, theta: float = 1e4):
    """Textbook 1-D RoPE: pair j (j < d/2) rotates by p * theta^(-2j/d).  Returns fp32 cos, sin [P, d]."""
    pos = np.asarray(positions, dtype=np.float64)
    j = np.arange(d // 2, dtype=np.float64)
    ang = pos[:, None] * theta ** (-2.0 * j / d)[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_3d_angles(tokens: np.ndarray, grid, d: int, theta: float = 1e4):
    """Angles [P, d/2] of the 3-axis (frame, height, width) video RoPE.

    The d/2 rotation pairs are split between the axes as 22/21/21 pairs (44/42/42 dims for
    d=128: the frame axis takes d - 4*(d//6) dims, height and width 2*(d//6) each); each axis
    uses standard RoPE frequencies over its own sub-width, theta^(-2k/dim_axis).  Token t sits at
    (f, h, w) = row-major position in the (F, Hh, Ww) grid.
    """
    F, Hh, Ww = grid
    t = np.asarray(tokens, dtype=np.int64)
    f, rem = np.divmod(t, Hh * Ww)
    h, w = np.divmod(rem, Ww)
    dims = [d - 4 * (d // 6), 2 * (d // 6), 2 * (d // 6)]
    parts = []
    for coord, dim in zip((f, h, w), dims):
        k = np.arange(dim // 2, dtype=np.float64)
        parts.append(coord.astype(np.float64)[:, None] * theta ** (-2.0 * k / dim)[None, :])
    ang = np.concatenate(parts, axis=1)
    assert ang.shape[1] == d // 2
    return ang


def rope_3d(tokens: np.ndarray, grid, d: int, theta: float = 1e4):
    ang = rope_3d_angles(tokens, grid, d, theta)
    ang = np.concatenate([ang, ang], axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_tables(p: Projection, row_idx: Optional[np.ndarray] = None):
    """cos, sin fp32 [T, d] (or the rows ``row_idx``) for a projection, or (None, None)."""
    rows = np.arange(p.T) if row_idx is None else np.asarray(row_idx)
    if p.rope == "1d":
        return rope_1d(rows, p.head_dim)
    if p.rope == "3d":
        return rope_3d(rows, p.grid, p.head_dim)
    return None, None


def digest(*arrays) -> str:
    """SHA-256 of the concatenated bytes (logged to show the inputs are reproducible)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]
