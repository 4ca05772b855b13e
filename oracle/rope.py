"""Rotary position embedding ahead of the Hadamard rotation (test infrastructure only; see oracle/__init__).

[FA3-card] "低精度优化：非相干处理" says the Hadamard rotation of incoherent
processing is bound by memory bandwidth and can be fused with the rotary
position embedding, at no extra cost.  The pages name the rotary embedding
but do not define it; the reading taken is the standard one, with the
half-split channel pairing: in the row at position n, the pair (x_i, x_{i+d/2})
(i < d/2), read as the complex number x_i + j·x_{i+d/2}, is multiplied by
e^{j·θ_{n,i}}:

    r_i       = x_i · cos θ − x_{i+d/2} · sin θ
    r_{i+d/2} = x_{i+d/2} · cos θ + x_i · sin θ

The caller supplies cos θ and sin θ as tables [N, d/2]; ``standard_tables``
gives the usual θ_{n,i} = n · base^(−2i/d), which the pins use.  In the fused
step the embedding comes first: y = H_d·(s ⊙ rope(x))/√d, then (optionally)
the per-block FP8 quantiser of ``quant``.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .quant import BLOCK, block_absmax, rotate_f32


def standard_tables(N: int, d: int, base: float = 10000.0):
    """cos, sin [N, d/2] (fp64) of θ_{n,i} = n · base^(−2i/d)."""
    inv_freq = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.arange(N, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, cos, sin) -> np.ndarray:
    """fp64 definition: x [B, N, H, d], tables [N, d/2] -> rotated rows."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float64)[None, :, None, :]
    s = np.asarray(sin, dtype=np.float64)[None, :, None, :]
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_f32(x, cos, sin) -> np.ndarray:
    """The same in fp32 with every product and sum rounded (no fused multiply-add):
    fl(fl(x_i·c) − fl(x_{i+d/2}·s)) and fl(fl(x_{i+d/2}·c) + fl(x_i·s))."""
    x = np.asarray(x, dtype=np.float32)
    h = x.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float32)[None, :, None, :]
    s = np.asarray(sin, dtype=np.float32)[None, :, None, :]
    a, b = x[..., :h], x[..., h:]
    lo = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    hi = (b * c).astype(np.float32) + (a * s).astype(np.float32)
    return np.concatenate([lo, hi], axis=-1).astype(np.float32)


def rope_rotate_f32(x, cos, sin, signs=None) -> np.ndarray:
    """fp32 fused prologue: rope_f32, then (if signs is given) quant.rotate_f32."""
    y = rope_f32(x, cos, sin)
    return rotate_f32(y, signs) if signs is not None else y


def quantize_rope(x, cos, sin, signs=None, block=BLOCK):
    """Fused prologue with the block quantiser: (codes uint8 [B, N, H, d], scales fp32 [B, H, nb]).

    The quantiser steps are those of ``quant.quantize`` applied to the fp32
    values of ``rope_rotate_f32``."""
    y = rope_rotate_f32(x, cos, sin, signs)
    amax = block_absmax(y, block)
    m448 = np.float32(e4m3.E4M3_MAX)
    with np.errstate(divide="ignore"):
        scales = np.where(amax > 0, amax / m448, np.float32(1.0)).astype(np.float32)
        inv = np.where(amax > 0, m448 / amax, np.float32(1.0)).astype(np.float32)
    N = y.shape[1]
    per_row = np.repeat(inv, block, axis=2)[:, :, :N]
    q = (y * per_row.transpose(0, 2, 1)[..., None]).astype(np.float32)
    return e4m3.encode(q), scales
