"""Coefficients of exp2_valu (tattn_device.hpp): 2^f on [0, 1] by the cubic
P(f) = 1 + a1·f + a2·f² + a3·f³ with P(1) = 2, chosen to minimise the largest
relative error max |P(f)/2^f − 1|, as a linear program over a dense grid of f.

    python tiled_attention_10_amd/csrc/exp2_poly.py    # prints the fp32 constants
"""
from __future__ import annotations

import numpy as np


def coefficients(grid: int = 20001) -> tuple[np.ndarray, float]:
    """(a1, a2, a3) in fp64 and the minimax relative error on the grid."""
    from scipy.optimize import linprog

    f = np.linspace(0.0, 1.0, grid)
    t = 2.0 ** f
    # variables a1, a2, a3, e: minimise e subject to ±(P(f)/2^f − 1) <= e and a1 + a2 + a3 = 1
    rows, rhs = [], []
    for s in (1.0, -1.0):
        rows.append(np.stack([s * f / t, s * f ** 2 / t, s * f ** 3 / t, -np.ones_like(f)], axis=1))
        rhs.append(s * (1.0 - 1.0 / t))
    r = linprog(np.array([0.0, 0.0, 0.0, 1.0]), A_ub=np.concatenate(rows), b_ub=np.concatenate(rhs),
                A_eq=np.array([[1.0, 1.0, 1.0, 0.0]]), b_eq=np.array([1.0]),
                bounds=[(None, None)] * 3 + [(0.0, None)])
    if not r.success:
        raise RuntimeError(r.message)
    return r.x[:3], float(r.x[3])


if __name__ == "__main__":
    a, e = coefficients()
    for i, x in enumerate(a.astype(np.float32), 1):
        mant, exp = float(x).hex().split("p")
        print(f"constexpr float kExp2A{i} = {mant.rstrip('0')}p{exp}f;  // {x:.9g}")
    print(f"// minimax relative error on the grid: {e:.4g}")
