"""Per-block FP8 quantisation (test infrastructure only; see oracle/__init__).

[FA3-V3] §4.3 keeps a scale factor per block so a block can be mapped back to
its float range; it also mentions an offset, which is not taken: the reading
is symmetric absmax scaling with no offset.  Blocks are 64 consecutive tokens
of one (batch, head), all d channels.

The quantiser's input y is the fp64 value of the prologue: the rows as given,
or the random-sign Hadamard rotation of them ([FA3-card] "非相干处理";
``hadamard.rotate``), optionally after the rotary embedding (``rope.rope``).
Every decision is taken on those fp64 values, by the definition:

    absmax = max |y| over the block                 (fp64)
    scale  = fl32(absmax / 448)                      (the stored fp32 scale; 1 for an all-zero block)
    code   = e4m3_rne_saturate(y / scale)           (the quotient in fp64)

so decode(code) · scale is the E4M3 value nearest to y on the block's grid.
An implementation that evaluates the rotation in fp32 lands on the same code
except where y / scale lies within its fp32 error of a rounding boundary; the
GPU tests bound that error and check codes against this definition.  Rows past
N inside the last block do not exist and do not enter its absmax.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .hadamard import rotate

BLOCK = 64


def prologue_values(x, signs=None, rope_tables=None) -> np.ndarray:
    """fp64 y: x [B, N, H, d], then the rotary embedding (tables (cos, sin) [N, d/2]) if
    given, then the rotation y = H_d·(s ⊙ ·)/sqrt(d) if signs is given."""
    y = np.asarray(x, dtype=np.float64)
    if rope_tables is not None:
        from .rope import rope
        y = rope(y, *rope_tables)
    if signs is not None:
        y = rotate(y, signs)
    return y


def block_absmax(y, block=BLOCK) -> np.ndarray:
    """y [B, N, H, d] -> absmax [B, H, ceil(N/block)] (fp64, exact)."""
    y = np.asarray(y, dtype=np.float64)
    B, N, H, d = y.shape
    nb = -(-N // block)
    pad = np.zeros((B, nb * block, H, d))
    pad[:, :N] = np.abs(y)
    return pad.reshape(B, nb, block, H, d).max(axis=(2, 4)).transpose(0, 2, 1).copy()


def scale_rows(scales, N, block=BLOCK) -> np.ndarray:
    """Per-block scales [B, H, nb] -> per-row factors [B, N, H, 1] (fp64)."""
    per_row = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :N]
    return per_row.transpose(0, 2, 1)[..., None]


def quantize_values(y, block=BLOCK):
    """fp64 y [B, N, H, d] -> (codes uint8 [B, N, H, d], scales fp32 [B, H, ceil(N/block)])."""
    y = np.asarray(y, dtype=np.float64)
    amax = block_absmax(y, block)
    scales = np.where(amax > 0, amax / e4m3.E4M3_MAX, 1.0).astype(np.float32)
    return e4m3.encode(y / scale_rows(scales, y.shape[1], block)), scales


def quantize(x, signs=None, block=BLOCK, rope_tables=None):
    """x [B, N, H, d] -> (codes uint8 [B, N, H, d], scales fp32 [B, H, ceil(N/block)])."""
    return quantize_values(prologue_values(x, signs, rope_tables), block)


def dequantize(codes, scales, block=BLOCK) -> np.ndarray:
    """codes [B, N, H, d], scales [B, H, nb] -> fp64 values."""
    vals = e4m3.decode(codes)
    return vals * scale_rows(scales, vals.shape[1], block)
