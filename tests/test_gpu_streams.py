"""Every entry point runs on the stream its caller passes.

The binding passes torch's current stream through the C ABI.  Here the inputs
of each call are produced on a side stream right after a kernel that keeps that
stream busy for tens of milliseconds; a call that launched on any other stream
would read its inputs before they exist.  The outputs must equal, bit for bit,
those of the same call made on the default stream (the kernels are
deterministic), and the side stream is only synchronised at the end.
"""
import numpy as np
import pytest
import torch

import tiled_attention_10_amd as T
from tiled_attention_10_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SPIN = 50_000_000   # cycles of the delaying kernel (tens of milliseconds)


def inputs(seed=41, B=2, N=700, Hq=8, Hkv=2, d=128):
    return [W.to_torch(x, "bf16") for x in W.random_qkv(seed, B, N, Hq, Hkv, d)]


def on_side_stream(fn, *host):
    """fn(*device tensors) on a fresh side stream, with the inputs derived there after a
    delay; returns the outputs copied there, read after synchronising that stream."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dev = [x.to(DEV) for x in host]
        torch.cuda._sleep(SPIN)
        late = [x + 1 if x.is_floating_point() else x.clone() for x in dev]
        outs = fn(*late)
        outs = [o.clone() for o in (outs if isinstance(outs, (tuple, list)) else (outs,))]
    s.synchronize()
    return [o.cpu() for o in outs]


def on_default_stream(fn, *host):
    late = [x.to(DEV) + 1 if x.is_floating_point() else x.to(DEV) for x in host]
    outs = fn(*late)
    outs = outs if isinstance(outs, (tuple, list)) else (outs,)
    torch.cuda.synchronize()
    return [o.cpu() for o in outs]


def same(a, b):
    """Bit-equal outputs (compared as bytes, so that -inf and NaN patterns count too)."""
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and x.shape == y.shape
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


@pytest.mark.parametrize("causal", [False, True])
def test_attn_fwd_on_callers_stream(causal):
    print(f"[attn_fwd side stream] causal={causal}", flush=True)
    fn = lambda q, k, v: T.attn_fwd(q, k, v, causal=causal, return_lse=True)
    same(on_side_stream(fn, *inputs()), on_default_stream(fn, *inputs()))


def test_fp8_path_on_callers_stream():
    print("[fp8_prologue + attn_fwd_fp8 side stream]", flush=True)
    signs = torch.from_numpy(np.where(np.random.default_rng(5).random(128) < 0.5, -1, 1).astype(np.int8))

    def fn(q, k, v, sg):
        q8, k8, v8, qs, ks, vs = T.fp8_prologue(q, k, v, signs=sg)
        o, lse = T.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, causal=True, return_lse=True)
        return q8, k8, v8, qs, ks, vs, o, lse

    same(on_side_stream(fn, *inputs(), signs), on_default_stream(fn, *inputs(), signs))


def test_decode_on_callers_stream():
    print("[attn_decode_fp8kv side stream]", flush=True)
    B, Nmax, Hq, Hkv, d = 3, 9000, 16, 2, 128
    rng = np.random.default_rng(8)
    q = W.to_torch(rng.standard_normal((B, Hq, d), dtype=np.float32), "bf16")
    k = W.to_torch(rng.standard_normal((B, Nmax, Hkv, d), dtype=np.float32), "bf16")
    v = W.to_torch(rng.standard_normal((B, Nmax, Hkv, d), dtype=np.float32), "bf16")
    seqlens = torch.tensor([9000, 4500, 1], dtype=torch.int32)

    def fn(q, k, v, sl):
        kc, ks = T.hadamard_rotate(k, None, quantize=True)
        vc, vs = T.hadamard_rotate(v, None, quantize=True)
        return T.attn_decode_fp8kv(q, kc, vc, ks, vs, sl, return_lse=True)

    same(on_side_stream(fn, q, k, v, seqlens), on_default_stream(fn, q, k, v, seqlens))
