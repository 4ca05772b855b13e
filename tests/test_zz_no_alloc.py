"""attn_decode_fp8kv_noalloc, the decode entry point that allocates nothing, through the C ABI.

It runs the same kernels with the same plan as attn_decode_fp8kv, only with the
library's fixed per-device scratch in place of the caller's workspace, so its
output and log-sum-exp must equal attn_decode_fp8kv's bit for bit.  Two calls
run back to back, the second with smaller sizes: the scratch keeps the first
call's partials, and the second must not read them.  (Sizes beyond the scratch
are rejected on the host; tests/test_abi.py checks that without a GPU.)
"""
import numpy as np
import pytest
import torch

import tiled_attention_10_amd as T
from tiled_attention_10_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(seed, B, Nmax, Hq, Hkv, seqlens, dtype):
    q, k, v = W.random_qkv(seed, B, 1, Hq, Hkv, 128, Nk=Nmax)
    q16 = W.to_torch(q[:, 0], dtype).to(DEV)
    kc, ks = T.hadamard_rotate(W.to_torch(k, dtype).to(DEV), None, quantize=True)
    vc, vs = T.hadamard_rotate(W.to_torch(v, dtype).to(DEV), None, quantize=True)
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    return q16, kc, vc, ks, vs, sl


def _both(args):
    q16 = args[0]
    B, Hq, d = q16.shape
    Nmax, Hkv = args[1].shape[1], args[1].shape[2]
    need = T.decode_workspace_size(B, Nmax, Hq, Hkv, d)
    assert 0 < need <= T.TATTN_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o_ref, lse_ref = T.attn_decode_fp8kv(*args, workspace=ws, return_lse=True)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    torch.cuda.synchronize()
    print(f"[attn_decode_fp8kv_noalloc] q{tuple(q16.shape)} cache{tuple(args[1].shape)} "
          f"seqlens={args[5].tolist()[:8]}", flush=True)
    r = T.attn_decode_fp8kv_noalloc(*args, out=o, lse=lse)
    torch.cuda.synchronize()
    assert r[0] is o and r[1] is lse
    return o.cpu(), lse.cpu(), o_ref.cpu(), lse_ref.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_noalloc_equals_workspace_entry_point_twice(dtype):
    # first call: several chunks per sequence (split and merge kernels), ragged lengths
    a = _case(81, 4, 20000, 64, 8, [20000, 13001, 1, 7777], dtype)
    o, lse, o_ref, lse_ref = _both(a)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
    # second call, smaller: fewer sequences, heads and keys; the scratch still holds the
    # first call's partials
    b = _case(82, 2, 3000, 8, 2, [3000, 17], dtype)
    o, lse, o_ref, lse_ref = _both(b)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
    assert np.isfinite(o.float().numpy()).all()
