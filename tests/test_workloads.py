"""The seeded input recipes (CPU): shapes, ranges and determinism of the decode
workloads and of the random E4M3 cache, as the design notes state them."""
import numpy as np

from tiled_attention_10_amd import workloads as W


def test_decode_lengths_mix():
    for w in W.DECODE_WORKLOADS.values():
        L = w.seqlens()
        assert L.dtype == np.int32 and L.shape == (w.B,)
        assert (L >= w.Nmax // 2).all() and (L <= w.Nmax).all() and L[-1] == w.Nmax
        assert np.array_equal(L, w.seqlens())                       # seeded
    big = W.DECODE_WORKLOADS["decode_fp8kv_b4_h64kv8_n131072"]
    assert big.seqlens().tolist() == [125622, 97325, 116701, 131072]


def test_decode_hbm_bytes():
    w = W.DECODE_WORKLOADS["decode_fp8kv_b4_h64kv8_n131072"]
    L = w.seqlens()
    rows = int(L.sum())
    blocks = int(((L + 63) // 64).sum())
    assert w.hbm_bytes(L) == rows * 8 * 128 * 2 + blocks * 8 * 4 * 2 + 2 * 4 * 64 * 128 * 2 == 964636416


def test_decode_cache_streams_are_per_sequence():
    w = W.DecodeWorkload("t", 9, 3, 100, 4, 2, 128, "bf16")
    k0, v0 = W.decode_cache_f32(w, 0)
    k1, _ = W.decode_cache_f32(w, 1)
    assert k0.shape == (100, 2, 128) and k0.dtype == np.float32
    assert not np.array_equal(k0, k1) and not np.array_equal(k0, v0)
    assert np.array_equal(k0, W.decode_cache_f32(w, 0)[0])


def test_random_e4m3_cache_codes_and_scales():
    codes, scales = W.random_e4m3_cache(3, 2, 4000, 2, 128)
    assert codes.dtype == np.uint8 and codes.shape == (2, 4000, 2, 128)
    u = np.unique(codes)
    assert 0x7F not in u and 0xFF not in u and u.size == 254      # every finite code, no NaN
    assert scales.dtype == np.float32 and scales.shape == (2, 2, 63)
    assert (scales >= 1 / 128).all() and (scales < 1 / 32).all()
    c2, s2 = W.random_e4m3_cache(3, 2, 4000, 2, 128)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
