"""fp64 emulation of the FP8 attention path (test infrastructure only).

The pages give no worked FP8 result, only the qualitative claim that
incoherent processing lowers FP8 error ([FA3-card] "主要结果"), so this
emulation is a sanity reference, not a definition.  It is pinned where no step
rounds: with E4M3-exact codes, power-of-two block scales and scores whose
probabilities (times their V factor) are E4M3 powers of two, it must equal
``attention.attention`` on the dequantised values (tests/test_oracle_fp8.py).
The criterion for the FP8 path is its RMSE against ``attention.attention`` on
the unquantised 16-bit inputs, with and without rotation.

Steps (the FP8 path's own, in order):

1. Q, K, V arrive as E4M3FN codes with per-(batch, head, 64-row block) fp32
   scales (``quant.quantize``; Q and K optionally rotated with the same signs).
2. Dequantise: Qd = code·sq, Kd = code·sk (fp64).
3. S = scale · Qd·Kdᵀ, causal mask as in ``attention``; p = exp(S − m) with m
   the row max.
4. The probabilities feed the second product in FP8.  The V block scale sv and
   a power-of-two headroom are folded into them before rounding:
       p̃_ij = e4m3(p_ij · sv(block j) · 2^8 / sv_max)
   with sv_max the largest V scale of that (batch, kv head), so p̃ <= 256.
   (The kernel rounds relative to its running max tile by tile; here the final
   row max is used, which is why this is a sanity reference only.)
5. The denominator sums the same rounded probabilities, mapped back by their
   block's factor: l_i = Σ_j p̃_ij · sv_max / (sv(block j) · 2^8), so the weights
   that divide are the weights that entered the second product.
6. O = (Σ_j p̃_ij · v_code_j) · sv_max / 2^8 / l.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .quant import dequantize, BLOCK

P_HEADROOM_LOG2 = 8


def fp8_attention_emul(q8, k8, v8, sq, sk, sv, scale=None, causal=False, rows=None):
    q = dequantize(q8, sq)
    k = dequantize(k8, sk)
    vcode = e4m3.decode(v8)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    sv = np.asarray(sv, dtype=np.float64)
    out = np.empty((B, len(rows), Hq, d))
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            S = scale * (q[b, rows, h, :] @ k[b, :, kvh, :].T)
            if causal:
                S = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, S)
            m = S.max(axis=1)
            p = np.exp(S - m[:, None])
            svb = np.repeat(sv[b, kvh], BLOCK)[:N]
            svmax = sv[b, kvh].max()
            f = svb * 2.0 ** P_HEADROOM_LOG2 / svmax
            pq = e4m3.decode(e4m3.encode(p * f[None, :]))
            l = (pq / f[None, :]).sum(axis=1)
            out[b, :, h, :] = (pq @ vcode[b, :, kvh, :]) * (svmax / 2.0 ** P_HEADROOM_LOG2) / l[:, None]
    return out
