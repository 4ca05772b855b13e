"""Scheduling variants of the 16-bit kernel (build.py VARIANTS) against the shipped library.

Every variant but those in build.ARITH_VARIANTS performs the same arithmetic per
query row in the same order:
the ring depth (3, 4 or 5 stages), the LDS read-ahead, the placement of the
tile loads and the two-group ping-pong change only when loads are issued, which
ring stage a tile lands in and which wave group runs a phase when.  So their
outputs must equal the shipped library's bit for bit.  A missing wait or
barrier in the ring (a tile read before it landed, or overwritten while still
read) would show up as a difference, because the stages a tile can race with
differ between ring depths.  Each variant is also compared with the fp64
oracle once, within the method's 16-bit tolerances; a variant whose arithmetic
differs (the scale folded into Q and rounded) adds the bound that rounding
implies: every score of a row moves by at most u·scale·Σ_i|q_i k_ji|, so each
softmax weight by a relative 2·that, and O by that times max_j |v_j − O|.
"""
import os

import numpy as np
import pytest
import torch

import tiled_attention_10_amd as T
from oracle import attention as A
from tiled_attention_10_amd import build as Bd
from tiled_attention_10_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"fp16": 2e-3, "bf16": 1e-2}

SHAPES = [  # B, N, Hq, Hkv, d, dtype
    (2, 333, 8, 8, 64, "fp16"),
    (1, 1000, 4, 1, 128, "bf16"),
    (1, 2048, 40, 8, 128, "bf16"),      # 320 items on 256 workgroups: uneven persistent shares
    (1, 8192, 64, 8, 128, "bf16"),      # the benchmark's GQA layer
    # many q tiles per workgroup with a ragged N: tile counts that are and are not
    # multiples of the ring depth
    (2, 1100, 96, 8, 128, "bf16"),
    (1, 1100, 96, 8, 64, "fp16"),
]


def _inputs(shape):
    B, N, Hq, Hkv, d, dt = shape
    return tuple(W.to_torch(x, dt) for x in W.random_qkv(90 + N, B, N, Hq, Hkv, d))


@pytest.fixture(scope="module")
def shipped():
    out = {}
    for shape in SHAPES:
        q, k, v = (x.to(DEV) for x in _inputs(shape))
        for causal in (False, True):
            print(f"[attn_fwd shipped] {shape} causal={causal}", flush=True)
            o, lse = T.attn_fwd(q, k, v, causal=causal, return_lse=True)
            out[shape, causal] = (o.cpu(), lse.cpu())
    return out


@pytest.mark.parametrize("variant", sorted(set(Bd.VARIANTS) - Bd.ARITH_VARIANTS))
def test_variant_bitwise_equals_shipped(variant, shipped):
    path = T.variant_path(variant)
    assert os.path.exists(path), f"{path} not built"
    with T.use_library(path):
        for shape in SHAPES:
            q, k, v = (x.to(DEV) for x in _inputs(shape))
            for causal in (False, True):
                print(f"[attn_fwd {variant}] {shape} causal={causal}", flush=True)
                o, lse = T.attn_fwd(q, k, v, causal=causal, return_lse=True)
                o0, lse0 = shipped[shape, causal]
                assert torch.equal(o.cpu().view(torch.int16), o0.view(torch.int16)), (shape, causal)
                assert torch.equal(lse.cpu().view(torch.int32), lse0.view(torch.int32)), (shape, causal)


@pytest.mark.parametrize("variant", sorted(Bd.VARIANTS))
def test_variant_parity_with_oracle(variant):
    B, N, Hq, Hkv, d, dt = 1, 777, 8, 2, 128, "bf16"
    q, k, v = (W.to_torch(x, dt) for x in W.random_qkv(95, B, N, Hq, Hkv, d))
    extra = 0.0
    if variant in Bd.ARITH_VARIANTS:
        qa, ka, va = (np.abs(x.double().numpy()) for x in (q, k, v))
        g = Hq // Hkv
        ds = max((qa[0, :, h] @ ka[0, :, h // g].T).max() for h in range(Hq)) * d ** -0.5 * 2.0 ** -8
        extra = 2.1 * ds * 2 * va.max()
    with T.use_library(T.variant_path(variant)):
        for causal in (False, True):
            o = T.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal).float().cpu().numpy()
            err = np.abs(o - A.attention(q, k, v, None, causal)).max()
            print(f"{variant} causal={causal}: max|dO| {err:.3e} (bound {TOL[dt] + extra:.3e})")
            assert err <= TOL[dt] + extra
