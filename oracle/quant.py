"""Per-block FP8 quantisation (test infrastructure only; see oracle/__init__).

[FA3-V3] §4.3 keeps a scale factor per block so a block can be mapped back to
its float range; it also mentions an offset, which is not taken: the reading
is symmetric absmax scaling with no offset.  Blocks are 64 consecutive tokens
of one (batch, head), all d channels.  Per block:

    scale = absmax / 448      (scale = 1 when the block is all zeros)
    code  = e4m3_rne_saturate(y · (448 / absmax))      (y · 1 for a zero block)

The pages do not say how the division by the scale is carried out; the
reading taken multiplies by the reciprocal 448/absmax computed once per block
(x ≈ decode(code) · scale still holds to E4M3's rounding).

Where floating point decides the integer code, the decision is taken in fp32,
the precision the kernel computes in: the optional rotation ([FA3-card]
"非相干处理"; see ``hadamard``) is the fp32 butterfly in stage order h = 1, 2,
4, ... followed by one fp32 multiply by fl32(1/sqrt(d)); ``absmax / 448`` and
``448 / absmax`` are IEEE fp32 divisions, ``y · (448/absmax)`` one fp32
multiply; the fp32 product is then rounded to the nearest E4M3FN code.  Rows past N inside the last block do not exist and do
not enter its absmax.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .hadamard import fwht

BLOCK = 64


def rotate_f32(x, signs) -> np.ndarray:
    """fp32 rotation: fl32(FWHT_fp32(s ⊙ x) · fl32(1/sqrt(d)))."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    s = np.asarray(signs, dtype=np.float32)
    inv = np.float32(1.0 / np.sqrt(d))
    return (fwht(x * s, dtype=np.float32) * inv).astype(np.float32)


def block_absmax(y, block=BLOCK) -> np.ndarray:
    """y [B, N, H, d] -> absmax [B, H, ceil(N/block)] (fp32, exact)."""
    y = np.asarray(y, dtype=np.float32)
    B, N, H, d = y.shape
    nb = -(-N // block)
    pad = np.zeros((B, nb * block, H, d), dtype=np.float32)
    pad[:, :N] = np.abs(y)
    return pad.reshape(B, nb, block, H, d).max(axis=(2, 4)).transpose(0, 2, 1).copy()


def quantize(x, signs=None, block=BLOCK):
    """x [B, N, H, d] -> (codes uint8 [B, N, H, d], scales fp32 [B, H, ceil(N/block)])."""
    y = rotate_f32(x, signs) if signs is not None else np.asarray(x, dtype=np.float32)
    amax = block_absmax(y, block)
    m448 = np.float32(e4m3.E4M3_MAX)
    with np.errstate(divide="ignore"):
        scales = np.where(amax > 0, amax / m448, np.float32(1.0)).astype(np.float32)
        inv = np.where(amax > 0, m448 / amax, np.float32(1.0)).astype(np.float32)
    B, N, H, d = y.shape
    per_row = np.repeat(inv, block, axis=2)[:, :, :N]             # [B, H, N]
    q = (y * per_row.transpose(0, 2, 1)[..., None]).astype(np.float32)
    return e4m3.encode(q), scales


def dequantize(codes, scales, block=BLOCK) -> np.ndarray:
    """codes [B, N, H, d], scales [B, H, nb] -> fp64 values."""
    vals = e4m3.decode(codes)
    N = vals.shape[1]
    per_row = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :N]
    return vals * per_row.transpose(0, 2, 1)[..., None]
