"""Random-sign Hadamard rotation (test infrastructure only; see oracle/__init__).

[FA3-card] "低精度优化：非相干处理": each attention head's Q and K are
multiplied by a random orthogonal matrix built from a Hadamard transform and
random signs, which spreads outlier channels before FP8 quantisation.  The
pages give no formula; the reading taken is

    y = H_d · (s ⊙ x) / sqrt(d)

per row x of length d, with H_d the Sylvester Hadamard matrix (H_1 = [1],
H_2k = [[H_k, H_k], [H_k, -H_k]]) and s in {±1}^d.  The matrix M = H_d·diag(s)
/ sqrt(d) is orthogonal, so applying the same s to Q and K leaves Q·Kᵀ
unchanged: (Q Mᵀ)(K Mᵀ)ᵀ = Q Kᵀ.  V is not rotated and O needs no inverse.
"""
from __future__ import annotations

import numpy as np


def sylvester(d: int) -> np.ndarray:
    """H_d by the doubling construction (d a power of two)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x, signs) -> np.ndarray:
    """fp64 definition: rows of x [..., d] -> H_d·(s ⊙ x)/sqrt(d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    s = np.asarray(signs, dtype=np.float64)
    return ((x * s) @ sylvester(d).T) / np.sqrt(d)


def fwht(x, dtype=np.float64) -> np.ndarray:
    """Unnormalised fast Walsh–Hadamard transform along the last axis, in ``dtype``.

    Butterfly stages with partner distance h = 1, 2, 4, ..., d/2, each mapping
    a pair (a, b) at positions (i, i + h) to (a + b, a - b).  Every stage is
    one Kronecker factor of H_d, so the result equals x·H_dᵀ (= H_d·x per row);
    with ``dtype=float32`` each add is rounded to fp32 in that fixed stage order.
    """
    y = np.array(x, dtype=dtype, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        y = v.reshape(y.shape)
        h *= 2
    return y
