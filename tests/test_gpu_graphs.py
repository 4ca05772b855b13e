"""The entry points inside a captured HIP graph.

The library launches kernels only (no allocation, copy or memset of its own),
so a caller can capture a call sequence once and replay it.  Each test captures
one sequence with torch.cuda.graph, then, three times, writes new inputs into
the captured buffers eagerly, replays, synchronises, and requires the replay's
outputs to equal bit for bit those of the same calls made eagerly on the new
inputs.  The decode test captures the entry point that allocates nothing (the
one meant for such callers) and changes the sequence lengths between replays;
its launch plan depends on the shapes alone, so the replays stay valid.
"""
import numpy as np
import pytest
import torch

import tiled_attention_10_amd as T
from tiled_attention_10_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def qkv(seed, B=2, N=900, Hq=8, Hkv=2, d=128):
    return [W.to_torch(x, "bf16").to(DEV) for x in W.random_qkv(seed, B, N, Hq, Hkv, d)]


def capture(fn):
    """Capture fn() after one eager warm-up call on a side stream; returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("causal", [False, True])
def test_attn_fwd_graph_replays(causal):
    print(f"[attn_fwd graph] causal={causal}", flush=True)
    q, k, v = qkv(60)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=DEV)
    g = capture(lambda: T.attn_fwd(q, k, v, causal=causal, out=o, return_lse=True, lse=lse))
    for r in range(3):
        nq, nk, nv = qkv(61 + r)
        q.copy_(nq); k.copy_(nk); v.copy_(nv)
        g.replay()
        torch.cuda.synchronize()
        eo, el = T.attn_fwd(nq, nk, nv, causal=causal, return_lse=True)
        torch.cuda.synchronize()
        assert bits_equal(o, eo) and bits_equal(lse, el), f"replay {r}"


def test_fp8_graph_replays():
    print("[fp8_prologue + attn_fwd_fp8 graph]", flush=True)
    q, k, v = qkv(70)
    signs = torch.from_numpy(np.where(np.random.default_rng(6).random(128) < 0.5, -1, 1).astype(np.int8)).to(DEV)
    pro = T.fp8_prologue(q, k, v, signs=signs)
    o = torch.empty_like(q)

    def seq():
        T.fp8_prologue(q, k, v, signs=signs, out=pro)
        T.attn_fwd_fp8(*pro, causal=True, out=o)

    g = capture(seq)
    for r in range(3):
        nq, nk, nv = qkv(71 + r)
        q.copy_(nq); k.copy_(nk); v.copy_(nv)
        g.replay()
        torch.cuda.synchronize()
        epro = T.fp8_prologue(nq, nk, nv, signs=signs)
        eo = T.attn_fwd_fp8(*epro, causal=True)
        torch.cuda.synchronize()
        assert all(bits_equal(a, b) for a, b in zip(pro, epro)), f"replay {r}: prologue"
        assert bits_equal(o, eo), f"replay {r}: attention"


def test_decode_noalloc_graph_replays():
    print("[attn_decode_fp8kv_noalloc graph]", flush=True)
    B, Nmax, Hq, Hkv, d = 3, 6000, 16, 2, 128
    rng = np.random.default_rng(9)
    cache = [W.to_torch(rng.standard_normal((B, Nmax, Hkv, d), dtype=np.float32), "bf16").to(DEV) for _ in range(2)]
    kc, ks = T.hadamard_rotate(cache[0], None, quantize=True)
    vc, vs = T.hadamard_rotate(cache[1], None, quantize=True)
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16, device=DEV)
    seqlens = torch.tensor([Nmax, 1, 2500], dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    g = capture(lambda: T.attn_decode_fp8kv_noalloc(q, kc, vc, ks, vs, seqlens, out=o, return_lse=True, lse=lse))
    lens = [[Nmax, 1, 2500], [17, Nmax, 0], [4097, 4096, 63]]
    for r in range(3):
        nq = W.to_torch(rng.standard_normal((B, Hq, d), dtype=np.float32), "bf16").to(DEV)
        nl = torch.tensor(lens[r], dtype=torch.int32, device=DEV)
        q.copy_(nq); seqlens.copy_(nl)
        g.replay()
        torch.cuda.synchronize()
        eo, el = T.attn_decode_fp8kv(nq, kc, vc, ks, vs, nl, return_lse=True)
        torch.cuda.synchronize()
        assert bits_equal(o, eo) and bits_equal(lse, el), f"replay {r}"
