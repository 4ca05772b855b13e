"""fp8_prologue, the one-launch FP8 prologue, through the C ABI.

It runs the same per-block arithmetic as hadamard_rotate and
rope_hadamard_rotate (whose outputs tests/test_gpu_hadamard.py and
tests/test_gpu_rope.py check against the oracle's fp64 definition), only
with Q, K and V in one grid.  So its codes and scales must equal the separate
calls' bit for bit: Q and K rotated with the same signs (and embedded with the
same tables), V quantised only.  Cases: with and without rotation and the
embedding, GQA and MHA, ragged N, both input types and head dims.
"""
import numpy as np
import pytest
import torch

import tiled_attention_10_amd as T
from tiled_attention_10_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SHAPES = [(1, 1, 2, 1, 128), (1, 100, 8, 2, 128), (2, 333, 4, 4, 64), (1, 1000, 16, 2, 128), (2, 130, 6, 3, 64)]


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}N{}H{}/{}d{}".format(*s))
def test_fp8_prologue_equals_separate_calls(shape, dtype, rotate, rope):
    B, N, Hq, Hkv, d = shape
    q, k, v = (W.to_torch(x, dtype).to(DEV) for x in W.random_qkv(400 + N + d, B, N, Hq, Hkv, d))
    signs = torch.from_numpy(W.rotation_signs(401 + N, d)).to(DEV) if rotate else None
    tables = tuple(torch.from_numpy(t).to(DEV) for t in W.rotary_tables(402 + N, N, d)) if rope else None
    print(f"[fp8_prologue] {shape} {dtype} rotate={rotate} rope={rope}", flush=True)
    got = T.fp8_prologue(q, k, v, signs, tables)
    if rope:
        want_q = T.rope_hadamard_rotate(q, *tables, signs, quantize=True)
        want_k = T.rope_hadamard_rotate(k, *tables, signs, quantize=True)
    else:
        want_q = T.hadamard_rotate(q, signs, quantize=True)
        want_k = T.hadamard_rotate(k, signs, quantize=True)
    want_v = T.hadamard_rotate(v, None, quantize=True)
    torch.cuda.synchronize()
    want = (want_q[0], want_k[0], want_v[0], want_q[1], want_k[1], want_v[1])
    for name, g, w in zip(("q8", "k8", "v8", "q_scale", "k_scale", "v_scale"), got, want):
        assert torch.equal(g, w), name


def test_fp8_prologue_into_given_outputs_then_attention():
    # the benchmark's use: outputs written in place, then attn_fwd_fp8 on them
    B, N, Hq, Hkv, d = 1, 777, 8, 2, 128
    q, k, v = (W.to_torch(x, "bf16").to(DEV) for x in W.random_qkv(410, B, N, Hq, Hkv, d))
    signs = torch.from_numpy(W.rotation_signs(411, d)).to(DEV)
    outs = T.fp8_prologue(q, k, v, signs)
    again = T.fp8_prologue(q, k, v, signs, out=tuple(torch.empty_like(o) for o in outs))
    o1 = T.attn_fwd_fp8(*outs)
    o2 = T.attn_fwd_fp8(*again)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(outs, again))
    assert torch.equal(o1, o2) and np.isfinite(o1.float().cpu().numpy()).all()
