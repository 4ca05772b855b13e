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
the per-block FP8 quantiser of ``quant``, all on fp64 values.  The cos/sin
tables are the caller's numbers (fp32 on the GPU path): the definition uses
those values exactly.
"""
from __future__ import annotations

import numpy as np


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


def rope_rotate(x, cos, sin, signs=None) -> np.ndarray:
    """fp64 fused prologue without the quantiser: rope, then the rotation if signs is given."""
    from .quant import prologue_values
    return prologue_values(x, signs, (cos, sin))


def quantize_rope(x, cos, sin, signs=None):
    """Fused prologue with the block quantiser: (codes uint8 [B, N, H, d], scales fp32 [B, H, nb]),
    decided on the fp64 values of ``rope_rotate`` exactly as ``quant.quantize`` decides them."""
    from .quant import quantize
    return quantize(x, signs, rope_tables=(cos, sin))
