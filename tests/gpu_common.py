"""Shared pieces of the GPU parity tests: inputs from the seeded recipe, expected values from the
oracle (never from the HIP path), the library calls through the C ABI, and the comparison rules.

Tolerances
  * codes, scales, residual sums, V columns: bit-exact.
  * bf16 outputs: |gpu - ref| <= 1e-2 * |ref| + 1e-3 elementwise, ref = unrounded fp64 oracle.
  * per-token sums of squares: |gpu - ref| <= 2e-3 * ref.
  * pass 2 checked end to end (from the same A and W) against the unrounded fp64 chain: the bf16
    rounding of pass 1's stored output (at most 2^-8 relative per element) enters both lanes of a
    RoPE pair, so the bound adds 2^-8 * r * (|g_j x_j| + |g_p x_p|) for lane j and its partner p.
"""
from __future__ import annotations

import dataclasses
import os
import sys
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle                      # noqa: E402
import synth                       # noqa: E402
from oracle import codecs          # noqa: E402

REL, ABS, SSQ_REL = 1e-2, 1e-3, 2e-3


def torch_dev():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def bf16_host(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_close(gpu_bits: np.ndarray, ref: np.ndarray, what: str, extra=None):
    """Elementwise |gpu - ref| <= REL |ref| + ABS (+ extra)."""
    g = codecs.bf16_to_f64(gpu_bits)
    tol = REL * np.abs(ref) + ABS
    if extra is not None:
        tol = tol + extra
    bad = np.abs(g - ref) > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first "
                             f"{[(tuple(i), g[tuple(i)], ref[tuple(i)]) for i in idx]}")


def check_ssq(gpu: np.ndarray, ref: np.ndarray, what: str):
    bad = np.abs(gpu.astype(np.float64) - ref) > SSQ_REL * np.abs(ref) + 1e-30
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} sums outside 2e-3; first "
                             f"{[(tuple(i), gpu[tuple(i)], ref[tuple(i)]) for i in idx]}")


def check_equal(gpu: np.ndarray, ref: np.ndarray, what: str):
    if not np.array_equal(gpu, ref):
        bad = np.argwhere(gpu != ref)
        idx = bad[:5]
        raise AssertionError(f"{what}: {len(bad)} mismatches; first "
                             f"{[(tuple(i), gpu[tuple(i)], ref[tuple(i)]) for i in idx]}")


def propagated_bound(X: np.ndarray, ssq: np.ndarray, gq, gk, nq, nkv, d, eps, norm_q, norm_k,
                     rope: bool) -> np.ndarray:
    """2^-8 * r * (|g_j x_j| + |g_p x_p|) over Q/K lanes (0 elsewhere); see module docstring."""
    out = np.zeros_like(X)
    h = d // 2
    for lo, n, g, col, on in ((0, nq, gq, 0, norm_q), (nq * d, nkv, gk, 1, norm_k)):
        if n == 0:
            continue
        w = n * d
        seg = X[:, lo:lo + w]
        gv = codecs.bf16_to_f64(g) if (on and g is not None) else np.ones(w)
        r = oracle.inv_rms(ssq[:, col], n, d, eps) if on else np.ones(X.shape[0])
        a = np.abs(seg * gv[None, :]) * r[:, None]
        if rope:
            ah = a.reshape(-1, n, 2, h)
            a = (ah + ah[:, :, ::-1, :]).reshape(-1, w)
        out[:, lo:lo + w] = 2.0 ** -8 * a
    return out


def floor_blocks(rng) -> list:
    """32-element fp32 blocks that reach or straddle the lower clamp of the E8M0 exponent
    (largest magnitude below 2^-119, fp32 subnormals, -0.0, exactly 2^-119 / 2^-120 / 2^-118)."""
    f32 = np.float32
    n = lambda s: (rng.standard_normal(32) * s).astype(f32)
    blocks = [
        n(1e-37),                                              # amax ~ 2^-122: E clamps to 0
        n(1e-41),                                              # fp32 subnormals only
        np.full(32, f32(2.0 ** -149)) * np.where(rng.random(32) < 0.5, 1, -1).astype(f32),
        np.zeros(32, f32),                                     # all-zero block: E = 0, codes 0
    ]
    b = np.zeros(32, f32)                                      # one subnormal among zeros and -0
    b[7] = f32(-3 * 2.0 ** -140)
    b[8] = f32(-0.0)
    blocks.append(b)
    b = n(1e-39)                                               # subnormals with a normal max
    b[3] = f32(2.0 ** -126)
    blocks.append(b)
    for e in (-119, -120, -118):                               # around the clamp boundary
        b = (rng.uniform(-1, 1, 32) * 2.0 ** e).astype(f32)
        b[0] = f32(2.0 ** e)                                   # amax exactly 2^e
        blocks.append(b)
    b = (rng.uniform(-1, 1, 32) * 2.0 ** -119).astype(f32)
    b[5] = f32(np.nextafter(f32(2.0 ** -119), f32(0)))        # just below 2^-119
    blocks.append(b)
    return blocks


@dataclasses.dataclass
class ProjInputs:
    p: synth.Projection
    x: np.ndarray              # fp32 activations [T, H]
    packed: np.ndarray         # oracle ROW_MX rows [T, H + 4]
    w_codes: np.ndarray        # [H/4, I, 4]
    w_e8m0: np.ndarray         # [H/32, I]
    bias: np.ndarray           # bf16 bits [I]
    gq: Optional[np.ndarray]
    gk: Optional[np.ndarray]
    cos: Optional[np.ndarray]
    sin: Optional[np.ndarray]


def make_inputs(p: synth.Projection, with_bias=True) -> ProjInputs:
    x = synth.activation(p)
    w = synth.weight(p)
    codes, e8 = oracle.mx_weight_quantize(w)
    cos, sin = synth.rope_tables(p)
    return ProjInputs(p, x, oracle.rowmx_quantize(x), codes, e8,
                      synth.bias_bf16(p) if with_bias else None,
                      synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k"), cos, sin)


def flags_of(p: synth.Projection) -> int:
    from rope_mxfp8_qkv_amd import NORM_Q, NORM_K, FUSED_ROPE
    f = 0
    if p.norm_q:
        f |= NORM_Q
    if p.norm_k and p.num_kv_heads > 0:
        f |= NORM_K
    if p.rope:
        f |= FUSED_ROPE
    return f


def custom_projection(name, T, H, nq, nkv, d, rope="1d", seed=99):
    return synth.Projection(name, seed, T=T, H=H, num_heads=nq, num_kv_heads=nkv, head_dim=d,
                            rope=rope, norm_q=True, norm_k=nkv > 0)


def staged_index(rows: np.ndarray, H: int) -> np.ndarray:
    """Byte offsets, in the staged activation image, of the codes of `rows` (elements 0..H-1):
    row t, element h at ((t / 256 * KS + h / 64) * 256 + t % 256) * 64
    + ((((h / 16) % 4) ^ sw(t % 256)) << 4) + h % 16, KS = 4 ceil(H / 256),
    sw(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1) (the layout include/qkvmx.h states)."""
    KS = 4 * -(-H // 256)
    t = np.asarray(rows, dtype=np.int64)[:, None]
    h = np.arange(H, dtype=np.int64)[None, :]
    r = t % 256
    sw = ((r >> 1) & 3) ^ ((r >> 3) & 1)
    return (((t // 256) * KS + h // 64) * 256 + r) * 64 + ((((h // 16) % 4) ^ sw) << 4) + h % 16


def unstage(image, rows: np.ndarray, H: int) -> np.ndarray:
    """Codes [len(rows), H] gathered from a device image (gather on the device)."""
    import torch
    idx = torch.as_tensor(staged_index(rows, H).reshape(-1), device=image.device)
    return image[idx].reshape(len(rows), H).cpu().numpy()


def staged_exp_index(rows: np.ndarray, H: int):
    """(dword, byte) positions, in the staged MX exponent image, of the exponents of `rows`
    (blocks 0..H/32-1): row t, block b = 8 s + 2 q + g at dword
    ((t / 256 * S + s) * 256 + t % 256) * 2 + g, byte q; S = ceil(H / 256) (include/qkvmx.h)."""
    S = -(-H // 256)
    t = np.asarray(rows, dtype=np.int64)[:, None]
    b = np.arange(H // 32, dtype=np.int64)[None, :]
    s, q, g = b // 8, (b % 8) // 2, b % 2
    return (((t // 256) * S + s) * 256 + t % 256) * 2 + g, q


def unstage_exp(exp_image, rows: np.ndarray, H: int) -> np.ndarray:
    """Exponents [len(rows), H / 32] from a staged exponent image (int32 device tensor)."""
    dw, q = staged_exp_index(rows, H)
    words = exp_image.view(-1).cpu().numpy().view(np.uint32)[dw]
    return ((words >> (8 * q).astype(np.uint32)) & 0xFF).astype(np.uint8)


def check_stage_padding(img, T: int, H: int):
    """Every byte of a staged activation image outside the T x H codes is zero."""
    n = img.numel()
    used = np.zeros(n, dtype=bool)
    used[staged_index(np.arange(T), H).reshape(-1)] = True
    host = img.cpu().numpy()
    assert not host[~used].any(), f"{int((host[~used] != 0).sum())} padding bytes are not zero"


def check_exp_padding(eimg, T: int, H: int):
    """Every byte of a staged exponent image outside the T x H/32 exponents is 127 (2^0)."""
    host = eimg.cpu().numpy().view(np.uint8).reshape(-1)
    used = np.zeros(host.size, dtype=bool)
    dw, qb = staged_exp_index(np.arange(T), H)
    used[(dw * 4 + qb).reshape(-1)] = True
    bad = host[~used] != 127
    assert not bad.any(), f"{int(bad.sum())} padding exponents are not 127"
