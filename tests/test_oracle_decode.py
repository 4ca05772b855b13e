"""Pins of oracle/decode.py (decode step over an FP8 block-quantised KV cache; CPU only).

The pages print no decode example, so the oracle is pinned by what the
definition fixes and by independent routines:

* brute force with Python's ``math`` on tiny caches;
* the prefill oracle (pinned on its own in test_oracle_attention.py): a decode
  step equals the last row of causal attention over the sequence so far;
* torch's CPU scaled_dot_product_attention in float64 on the dequantised cache;
* the dequantisation itself: E4M3 values times the scale of the row's 64-row
  block (a block-boundary check and the quantiser's error bound), with planted
  mistakes (wrong block, divide instead of multiply) that must fail;
* special cases: one cached row gives O = v_0; rows past the sequence length do
  not matter; GQA equals MHA with repeated KV heads.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import decode as D
from oracle import e4m3, quant


def rng(seed):
    return np.random.default_rng(seed)


def cache(seed, B, N, H, d, scale_spread=True):
    """Quantised K, V caches from seeded normals (codes, scales) via the oracle quantiser."""
    r = rng(seed)
    k = r.standard_normal((B, N, H, d)).astype(np.float32)
    v = r.standard_normal((B, N, H, d)).astype(np.float32)
    if scale_spread:   # blocks of different magnitude, so a wrong block index shows
        nb = -(-N // 64)
        mult = np.repeat(r.uniform(0.25, 4.0, (B, nb, H)), 64, axis=1)[:, :N, :, None]
        k = (k * mult).astype(np.float32)
        v = (v * mult[..., ::-1, :] if H > 1 else v * mult).astype(np.float32)
    kc, ks = quant.quantize(k)
    vc, vs = quant.quantize(v)
    return kc, ks, vc, vs


def brute(q, kc, ks, vc, vs, seqlens, scale):
    B, Hq, d = q.shape
    Hkv = kc.shape[2]
    g = Hq // Hkv
    table = e4m3.decode_table()
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(seqlens[b])
        for h in range(Hq):
            kv = h // g
            def kval(j, c):
                return float(table[kc[b, j, kv, c]]) * float(ks[b, kv, j // 64])
            def vval(j, c):
                return float(table[vc[b, j, kv, c]]) * float(vs[b, kv, j // 64])
            s = [scale * math.fsum(float(q[b, h, c]) * kval(j, c) for c in range(d)) for j in range(L)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for c in range(d):
                out[b, h, c] = math.fsum(e[j] * vval(j, c) for j in range(L)) / z
            lse[b, h] = m + math.log(z)
    return out, lse


def test_brute_force_tiny():
    B, N, Hq, Hkv, d = 2, 70, 4, 2, 4
    kc, ks, vc, vs = cache(1, B, N, Hkv, d)
    q = rng(2).standard_normal((B, Hq, d))
    seqlens = [66, 3]
    o, lse = D.decode_attention(q, kc, ks, vc, vs, seqlens, scale=0.7, return_lse=True)
    ob, lb = brute(q, kc, ks, vc, vs, seqlens, 0.7)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def test_equals_last_row_of_causal_prefill():
    B, N, Hq, Hkv, d = 3, 200, 8, 2, 16
    kc, ks, vc, vs = cache(3, B, N, Hkv, d)
    Kd, Vd = D.dequantize(kc, ks), D.dequantize(vc, vs)
    q = rng(4).standard_normal((B, Hq, d))
    seqlens = [200, 65, 1]
    o, lse = D.decode_attention(q, kc, ks, vc, vs, seqlens, return_lse=True)
    for b, L in enumerate(seqlens):
        qf = np.zeros((1, L, Hq, d))
        qf[0, L - 1] = q[b]
        of, lf = A.attention(qf, Kd[b:b + 1, :L], Vd[b:b + 1, :L], causal=True, return_lse=True)
        np.testing.assert_allclose(o[b], of[0, L - 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], lf[0, :, L - 1], rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64():
    B, N, Hq, Hkv, d = 2, 300, 4, 4, 32
    kc, ks, vc, vs = cache(5, B, N, Hkv, d)
    Kd, Vd = D.dequantize(kc, ks), D.dequantize(vc, vs)
    q = rng(6).standard_normal((B, Hq, d))
    seqlens = [300, 129]
    o = D.decode_attention(q, kc, ks, vc, vs, seqlens)
    for b, L in enumerate(seqlens):
        qt = torch.from_numpy(q[b][:, None, :])                                   # [H, 1, d]
        kt = torch.from_numpy(np.ascontiguousarray(Kd[b, :L].transpose(1, 0, 2)))  # [H, L, d]
        vt = torch.from_numpy(np.ascontiguousarray(Vd[b, :L].transpose(1, 0, 2)))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy()[:, 0]
        np.testing.assert_allclose(o[b], ref, rtol=0, atol=1e-12)


def test_dequantize_uses_the_rows_block():
    # every code 1.0; block 0 scale 2, block 1 scale 3: row 63 is 2, row 64 is 3
    codes = np.full((1, 130, 1, 4), 0x38, dtype=np.uint8)
    scales = np.array([[[2.0, 3.0, 5.0]]], dtype=np.float32)
    x = D.dequantize(codes, scales)
    assert (x[0, :64] == 2.0).all() and (x[0, 64:128] == 3.0).all() and (x[0, 128:] == 5.0).all()


def test_dequantize_inverts_the_quantiser_within_e4m3_rounding():
    x = (rng(7).standard_normal((2, 150, 3, 64)) * rng(8).uniform(0.1, 10, (2, 150, 3, 1))).astype(np.float32)
    codes, scales = quant.quantize(x)
    y = D.dequantize(codes, scales)
    per_row = np.repeat(scales, 64, axis=2)[:, :, :150].transpose(0, 2, 1)[..., None]
    # RNE to E4M3: relative error <= 2^-4 for normals, absolute <= 2^-10 · scale below 2^-6 · scale
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * per_row) * (1 + 1e-5)
    assert (np.abs(y - x) <= bound).all()
    # planted mistakes: dividing by the scale, or taking the next row's block, fail the bound
    wrong_div = e4m3.decode(codes) / per_row
    assert not (np.abs(wrong_div - x) <= bound).all()
    nxt = np.repeat(scales, 64, axis=2)[:, :, 1:151].transpose(0, 2, 1)[..., None]
    wrong_blk = e4m3.decode(codes) * nxt
    assert not (np.abs(wrong_blk - x) <= bound).all()


def test_single_row_gives_v0():
    kc, ks, vc, vs = cache(9, 1, 64, 2, 8)
    q = rng(10).standard_normal((1, 4, 8))
    o, lse = D.decode_attention(q, kc, ks, vc, vs, [1], return_lse=True)
    Kd, Vd = D.dequantize(kc, ks), D.dequantize(vc, vs)
    for h in range(4):
        assert np.array_equal(o[0, h], Vd[0, 0, h // 2])
        assert abs(lse[0, h] - (Kd[0, 0, h // 2] @ q[0, h]) / math.sqrt(8)) < 1e-12


def test_rows_past_length_do_not_matter():
    kc, ks, vc, vs = cache(11, 1, 256, 1, 16, scale_spread=False)
    q = rng(12).standard_normal((1, 2, 16))
    L = 100
    base = D.decode_attention(q, kc, ks, vc, vs, [L])
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, L:] = 0x30
    vc2[0, L:] = 0x7E
    assert np.array_equal(D.decode_attention(q, kc2, ks, vc2, vs, [L]), base)
    kc2[0, L - 1] ^= 0x01     # a row inside the sequence does matter
    assert not np.array_equal(D.decode_attention(q, kc2, ks, vc2, vs, [L]), base)


def test_gqa_equals_mha_with_repeated_heads():
    B, N, Hq, Hkv, d = 2, 90, 6, 2, 8
    kc, ks, vc, vs = cache(13, B, N, Hkv, d)
    q = rng(14).standard_normal((B, Hq, d))
    g = Hq // Hkv
    rep = lambda a: np.repeat(a, g, axis=2)
    o1 = D.decode_attention(q, kc, ks, vc, vs, [90, 7])
    o2 = D.decode_attention(q, rep(kc), np.repeat(ks, g, axis=1), rep(vc), np.repeat(vs, g, axis=1), [90, 7])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def test_planted_wrong_kv_head_is_caught():
    # reading kv head h % Hkv instead of h // g changes the result
    B, N, Hq, Hkv, d = 1, 64, 4, 2, 8
    kc, ks, vc, vs = cache(15, B, N, Hkv, d)
    q = rng(16).standard_normal((B, Hq, d))
    o = D.decode_attention(q, kc, ks, vc, vs, [64])
    perm = [0, 2, 1, 3]    # head h of this query set reads kv head h % 2
    o_wrong = D.decode_attention(q[:, perm], kc, ks, vc, vs, [64])[:, perm]
    assert np.abs(o - o_wrong).max() > 1e-3
