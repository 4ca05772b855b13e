"""fp64 definition of attention (test infrastructure only; see oracle/__init__).

[FA3-V3] §2 defines, for one head, S = Q·Kᵀ (N×N), P = softmax(S) row-wise and
O = P·V (N×d).  §11's ``standard_attention`` divides the scores by sqrt(d)
before the softmax; the scale is a parameter here with that default.  §11's
``_apply_causal_mask`` keeps key j for query i only when i >= j (masked scores
become -inf).  The mapping of query heads to key/value heads under grouped-query
attention is not stated on the pages; the reading taken is contiguous groups,
kv_head = q_head // (Hq / Hkv), which equals multi-head attention with K and V
repeated head-wise.

All tensors are laid out [B, N, H, d].  Inputs of any float dtype are upcast
exactly to fp64; S and P are materialised (in row blocks to bound memory) and
the softmax is the plain two-pass one: subtract the row max, exponentiate with
``exp``, divide by the row sum.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().to(dtype=__import__("torch").float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, N, H, d]")
    B, N, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, N, Hq, Hkv, d, k.shape[1]


def head_attention(qh, kh, vh, scale, causal, row_ids):
    """One head, the given query rows.  qh [R, d], kh/vh [Nk, d], fp64.

    Returns (O [R, d], lse [R]).  ``row_ids`` are the rows' positions in the
    sequence (needed by the causal mask).  A row with every key masked gets
    O = 0 and lse = -inf (cannot happen for square causal attention, where key
    0 is always visible; stated so the convention is explicit).
    """
    S = scale * (qh @ kh.T)                      # [R, Nk]   [FA3-V3] §2
    if causal:                                    # [FA3-V3] §11: keep i >= j
        cols = np.arange(kh.shape[0])
        S = np.where(cols[None, :] > np.asarray(row_ids)[:, None], -np.inf, S)
    m = S.max(axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    E = np.exp(S - m_safe[:, None])               # exp(-inf) = 0 for masked keys
    z = E.sum(axis=1)
    P = E / np.where(dead, 1.0, z)[:, None]
    O = P @ vh
    lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, z)))
    return O, lse


def attention(q, k, v, scale=None, causal=False, return_lse=False, row_block=2048):
    """Full attention forward, [B, N, Hq, d] -> [B, N, Hq, d] in fp64.

    ``lse`` (if requested) is [B, Hq, N]: the natural-log row log-sum-exp of
    the scaled, masked scores.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, N, Hq, Hkv, d, Nk = _check(q, k, v)
    if causal and Nk != N:
        raise ValueError("causal attention needs equal query and key lengths")
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    g = Hq // Hkv
    out = np.empty((B, N, Hq, d))
    lse = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            kh, vh = k[b, :, h // g, :], v[b, :, h // g, :]
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                rows = np.arange(r0, r1)
                o, l = head_attention(q[b, r0:r1, h, :], kh, vh, scale, causal, rows)
                out[b, r0:r1, h, :] = o
                lse[b, h, r0:r1] = l
    return (out, lse) if return_lse else out


def attention_rows(q, k, v, rows, scale=None, causal=False, heads=None):
    """Exact fp64 result for a subset of query rows (each row is independent).

    ``rows`` is a 1-D array of sequence positions; ``heads`` (default all) the
    query heads.  Returns O [B, len(rows), len(heads), d] and lse
    [B, len(heads), len(rows)].
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, N, Hq, Hkv, d, Nk = _check(q, k, v)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = list(range(Hq)) if heads is None else list(heads)
    rows = np.asarray(rows, dtype=np.int64)
    g = Hq // Hkv
    out = np.empty((B, len(rows), len(heads), d))
    lse = np.empty((B, len(heads), len(rows)))
    for b in range(B):
        for j, h in enumerate(heads):
            o, l = head_attention(q[b, rows, h, :], k[b, :, h // g, :], v[b, :, h // g, :],
                                  scale, causal, rows)
            out[b, :, j, :] = o
            lse[b, j, :] = l
    return out, lse


def partial_softmax_chunk(s, v):
    """Unnormalised statistics of one chunk of scores for one query row.

    s [n] scores (already scaled), v [n, d].  Returns (o, m, z): m = max(s),
    z = sum(exp(s - m)), o = sum(exp(s - m) * v) -- the per-chunk state the
    online softmax carries ([FA3-V3] §4.2 and §11's consumer loop).
    """
    s = np.asarray(s, dtype=np.float64)
    m = s.max()
    e = np.exp(s - m)
    return e @ np.asarray(v, dtype=np.float64), m, e.sum()


def merge_chunks(a, b):
    """Merge two chunk states with [FA3-V3] §4.2's rule.

    m = max(m_a, m_b); z = z_a·e^(m_a−m) + z_b·e^(m_b−m); the unnormalised
    outputs are rescaled by the same factors.  Returns (o, m, z).
    """
    oa, ma, za = a
    ob, mb, zb = b
    m = max(ma, mb)
    fa, fb = np.exp(ma - m), np.exp(mb - m)
    return oa * fa + ob * fb, m, za * fa + zb * fb
