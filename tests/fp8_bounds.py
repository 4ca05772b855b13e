"""Bounds for the FP8 attention path, derived from E4M3's rounding of the probabilities.

With Q, K, V given as E4M3 codes and block scales, the plain definition on the
dequantised values (oracle.attention) is O_dq = Σ_j p_j v_j / Σ_j p_j with
p_j = exp(s_j − m).  The FP8 path rounds each probability, after folding in
its V block's factor f_j = 2^8·sv(j)/max sv, to E4M3 (the reading of SURVEY
c10 both the kernel and the emulation follow), and divides by the sum of the
same rounded weights.  So its effective weights are p̃_j = p_j·(1 + ε_j) + a_j
with |ε_j| <= 2^-4 (E4M3's relative rounding of normals) and |a_j| <= 2^-10/f_j
(half the subnormal spacing, mapped back by f_j; a reference max below the
final one only shrinks it).  For a weighted mean with such weights:

    |O − O_dq|_c <= Σ_j (ε·p_j + a_j)·|v_jc − O_dq,c| / ((1 − ε)·Σ_j p_j − Σ_j a_j)
    |LSE − LSE_dq| <= −ln(1 − (ε·Σ p_j + Σ a_j)/Σ p_j)

ε carries a slack of 1e-3 on top of 2^-4·1.01 for what is far smaller: fp32
score and exponential errors and the matrix cores' truncated accumulation.  A
16-bit output adds its own rounding.
"""
from __future__ import annotations

import numpy as np

from oracle import quant

EPS = 1.01 * 2.0 ** -4 + 1e-3
U_OUT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def dq_reference(q8, k8, v8, sq, sk, sv, scale=None, causal=False, rows=None, heads=None, out_dtype=None):
    """Exact attention on the dequantised codes for the given rows and query heads, with the
    derived bounds.  Returns (O [B, rows, heads, d], LSE [B, heads, rows], bound_O, bound_LSE)."""
    qd, kd, vd = (quant.dequantize(c, s) for c, s in ((q8, sq), (k8, sk), (v8, sv)))
    B, N, Hq, d = qd.shape
    Hkv = kd.shape[2]
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    heads = list(range(Hq)) if heads is None else list(heads)
    sv = np.asarray(sv, dtype=np.float64)
    O = np.empty((B, len(rows), len(heads), d))
    bO = np.empty_like(O)
    lse = np.empty((B, len(heads), len(rows)))
    blse = np.empty_like(lse)
    for b in range(B):
        for hi, h in enumerate(heads):
            kv = h // g
            f = np.repeat(2.0 ** 8 * sv[b, kv] / sv[b, kv].max(), quant.BLOCK)[:N]
            a = 2.0 ** -10 / f
            step = max(1, 2 ** 25 // (N * d))        # rows per chunk: [rows, N, d] stays ~256 MB
            for r0 in range(0, len(rows), step):
                rr = rows[r0:r0 + step]
                S = scale * (qd[b, rr, h] @ kd[b, :, kv].T)
                if causal:
                    S = np.where(np.arange(N)[None, :] > rr[:, None], -np.inf, S)
                m = S.max(axis=1)
                p = np.exp(S - m[:, None])
                vis = np.isfinite(S)
                z = p.sum(axis=1)
                o = (p @ vd[b, :, kv]) / z[:, None]
                w = EPS * p + np.where(vis, a[None, :], 0.0)
                dev = np.abs(vd[b, :, kv][None, :, :] - o[:, None, :])          # [rows, N, d]
                num = np.einsum("rn,rnd->rd", w, dev)
                sa = (np.where(vis, a[None, :], 0.0)).sum(axis=1)
                den = (1 - EPS) * z - sa
                assert (den > 0).all()
                bo = num / den[:, None]
                if out_dtype is not None:
                    bo = bo + U_OUT[out_dtype] * (np.abs(o) + bo) + 1e-6
                O[b, r0:r0 + step, hi] = o
                bO[b, r0:r0 + step, hi] = bo
                lse[b, hi, r0:r0 + step] = m + np.log(z)
                blse[b, hi, r0:r0 + step] = -np.log1p(-(EPS * z + sa) / z) + 1e-5
    return O, lse, bO, blse


def check(got, want, bound, what):
    err = np.abs(np.asarray(got, dtype=np.float64) - want)
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the derived bound; first at {i}: "
                             f"|Δ| {err[i]:.4g} > {bound[i]:.4g}")
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.where(bound > 0, err / bound, 0.0).max())
