"""GPU checks of rope_hadamard_rotate (through the C ABI) against the oracle.

The fused prologue (rotary embedding, then the optional random-sign Hadamard
rotation, then either the 16-bit output or the FP8 block quantiser) is
decided by the oracle on fp64 values (oracle/rope.py, oracle/quant.py).  The
kernel computes in fp32, so its outputs must equal the oracle's except where
an fp64 value lies within the fp32 evaluation's error bound of a rounding
boundary (tests/prologue_bounds.py); every output must lie in its bounded
interval, and the open elements are counted and held to a small fraction.
The end-to-end test checks that attention on the fused prologue's output
approximates the exact attention of the rotary-embedded inputs.
"""
import math

import numpy as np
import pytest
import torch

import prologue_bounds as PB
import tiled_attention_10_amd as T
from oracle import attention as A
from oracle import rope as R
from tiled_attention_10_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}

SHAPES = [(1, 1, 1, 64), (1, 63, 2, 128), (2, 65, 3, 64), (1, 200, 4, 128), (2, 130, 2, 128)]


def inputs(shape, dtype, seed):
    B, N, H, d = shape
    x = W.to_torch(W.normal(seed, 0, (B, N, H, d)), dtype)
    c, s = W.rotary_tables(seed, N, d)
    sg = W.rotation_signs(seed, d)
    return x, c, s, sg


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}N{}H{}d{}".format(*s))
def test_rope_16bit_output_matches_definition(shape, rotate, dtype):
    x, c, s, sg = inputs(shape, dtype, 300 + sum(shape))
    print(f"[rope_hadamard_rotate] {shape} {dtype} rotate={rotate}", flush=True)
    sig = torch.from_numpy(sg).to(DEV) if rotate else None
    y = T.rope_hadamard_rotate(x.to(DEV), torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV), sig)
    torch.cuda.synchronize()
    yr, e = PB.prologue_error(x.double().numpy(), sg if rotate else None, (c, s))
    n_open, n = PB.check_16bit(y.cpu().double().numpy(), yr, e, dtype)
    print(f"open roundings {n_open}/{n}")
    assert n_open <= {"bf16": 0.02, "fp16": 0.08}[dtype] * n


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}N{}H{}d{}".format(*s))
def test_rope_quantiser_matches_definition(shape, rotate):
    x, c, s, sg = inputs(shape, "bf16", 400 + sum(shape))
    sig = torch.from_numpy(sg).to(DEV) if rotate else None
    codes, scales = T.rope_hadamard_rotate(x.to(DEV), torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV),
                                           sig, quantize=True)
    torch.cuda.synchronize()
    yr, e = PB.prologue_error(x.double().numpy(), sg if rotate else None, (c, s))
    n_open, n = PB.check_codes(codes.cpu().numpy(), scales.cpu().numpy(), yr, e)
    print(f"open codes {n_open}/{n}")
    assert n_open <= 0.01 * n


def test_identity_tables_reduce_to_hadamard_rotate():
    x, c, s, sg = inputs((1, 96, 2, 128), "bf16", 501)
    ones, zeros = np.ones_like(c), np.zeros_like(s)
    xd, sig = x.to(DEV), torch.from_numpy(sg).to(DEV)
    a = T.rope_hadamard_rotate(xd, torch.from_numpy(ones).to(DEV), torch.from_numpy(zeros).to(DEV), sig, quantize=True)
    b = T.hadamard_rotate(xd, sig, quantize=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_attention_after_fused_prologue():
    B, N, H, d = 1, 1024, 4, 128
    q, k, v = (W.to_torch(x, "bf16") for x in W.random_qkv(77, B, N, H, H, d))
    c, s = W.rotary_tables(77, N, d)
    sg = torch.from_numpy(W.rotation_signs(77, d)).to(DEV)
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    q8, sq = T.rope_hadamard_rotate(q.to(DEV), cd, sd, sg, quantize=True)
    k8, sk = T.rope_hadamard_rotate(k.to(DEV), cd, sd, sg, quantize=True)
    v8, sv = T.hadamard_rotate(v.to(DEV), None, quantize=True)
    o = T.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True).float().cpu().numpy()
    qr, kr = R.rope(q.float().numpy(), c, s), R.rope(k.float().numpy(), c, s)
    exact = A.attention(qr, kr, v.float().numpy(), None, True)
    err = math.sqrt(float(np.mean((o - exact) ** 2)))
    print(f"RMSE fp8 attention after the fused prologue: {err:.3e} (std of O {np.std(exact):.3e})")
    assert err < 0.1 * np.std(exact)


def test_binding_checks_tables():
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16, device=DEV)
    good = torch.zeros(8, 32, device=DEV)
    with pytest.raises(ValueError):
        T.rope_hadamard_rotate(x, torch.zeros(8, 31, device=DEV), good)
    with pytest.raises(ValueError):
        T.rope_hadamard_rotate(x, good.double(), good)
