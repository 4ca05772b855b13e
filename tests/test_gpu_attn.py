"""GPU parity of attn_fwd (fp16/bf16) against the fp64 CPU oracle, through the C ABI.

Tolerances are the ones the method's target states for inputs ~ N(0,1):
max |ΔO| <= 2e-3 for fp16 and <= 1e-2 for bf16.  Small shapes are compared
element by element (several tiles plus ragged tails); the large workloads are
compared on sampled rows that the oracle computes exactly, in the same launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import tiled_attention_10_amd as T
from oracle import attention as A
from tiled_attention_10_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1e-2}
# Unit roundoff of the input type (round to nearest, 11 and 8 significand bits).
U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
DEV = "cuda:0"


def lse_tol(q, k, dtype, scale=None, rows=None, heads=None, causal=False):
    """Bound on |ΔLSE| per (batch, head, row), derived from the kernel's arithmetic.

    The scores are exact products of the 16-bit inputs summed in fp32 by the
    matrix cores from zero (at most 8 accumulation steps, each rounding at most
    2^-24 of a partial sum below scale·Σ_i|q_i k_ji| in natural-log units), and
    one fused multiply-add forms c·s − m_ref (one more such rounding).  The softmax denominator sums the probabilities rounded to the input
    type (the values that enter P·V): each has relative error <= u, so
    |Δ ln z| <= u/(1-u); in fp16 a probability below 2^-14 is subnormal and
    rounds with an absolute error of at most 2^-25, against z >= 1 (the row's
    largest probability is at least 1 under the kernel's reference max).  fp32
    accumulation of z adds at most (tiles + 40)·2^-24, and the final log 1e-6
    relative to the LSE.
    """
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = d ** -0.5 if scale is None else scale
    rows = np.arange(N) if rows is None else np.asarray(rows)
    heads = list(range(Hq)) if heads is None else list(heads)
    qa = np.abs(q.double().numpy())[:, rows][:, :, heads]
    kn = np.abs(k.double().numpy())
    u = U[dtype]
    worst = np.empty((B, len(rows), len(heads)))
    for b in range(B):
        for i, h in enumerate(heads):
            worst[b, :, i] = scale * (qa[b, :, i] @ kn[b, :, h // (Hq // Hkv)].T).max(axis=1)
    sub = N * 2.0 ** -25 if dtype == "fp16" else 0.0
    tol = 1.01 * u / (1 - u) + sub + 16 * 2.0 ** -24 * worst + (N / 64 + 40) * 2.0 ** -24
    return tol.transpose(0, 2, 1)                                              # [B, heads, rows]


def check_lse(got, want, tol, what=""):
    """Every log-sum-exp within its derived bound; prints the largest error and its share of the bound."""
    err = np.abs(got - want)
    bound = tol + 1e-6 * np.abs(want)
    print(f"LSE {what}: max|dLSE| = {err.max():.3e}, largest share of the bound {(err / bound).max():.3f}")
    assert (err <= bound).all()


def run(q, k, v, causal, scale=None, lse=False):
    print(f"[attn_fwd] q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} causal={causal}", flush=True)
    r = T.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, softmax_scale=scale, return_lse=lse)
    torch.cuda.synchronize()
    if lse:
        return r[0].float().cpu().numpy(), r[1].cpu().numpy()
    return r.float().cpu().numpy()


SMALL = [
    (1, 1, 1, 1, 64), (1, 3, 2, 1, 128), (1, 64, 1, 1, 128), (2, 127, 4, 2, 64), (1, 128, 2, 2, 128),
    (1, 129, 2, 2, 128), (2, 333, 8, 8, 64), (1, 1000, 4, 1, 128), (1, 700, 6, 3, 64),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}N{}H{}/{}d{}".format(*s))
def test_small_shapes_elementwise(shape, causal, dtype):
    B, N, Hq, Hkv, d = shape
    q, k, v = (W.to_torch(x, dtype) for x in W.random_qkv(sum(shape), B, N, Hq, Hkv, d))
    o, lse = run(q, k, v, causal, lse=True)
    ref, ref_lse = A.attention(q, k, v, None, causal, return_lse=True)
    err = np.abs(o - ref).max()
    assert err <= TOL[dtype], err
    check_lse(lse, ref_lse, lse_tol(q, k, dtype, causal=causal), f"{shape} {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_tiny_workload(dtype):
    w = W.WORKLOADS["tiny_h1_n128_d64"]
    q, k, v = (W.to_torch(x, dtype) for x in W.qkv_f32(w))
    o = run(q, k, v, False)
    # the oracle runs on the same rounded values the GPU receives
    assert np.abs(o - A.attention(q, k, v)).max() <= TOL[dtype]
    # and the rounding of the fp32 inputs themselves moves the result by far less than the tolerance
    q32, k32, v32 = W.qkv_f32(w)
    assert np.abs(A.attention(q32, k32, v32) - A.attention(q, k, v)).max() < 5 * TOL[dtype]


@pytest.mark.parametrize("causal", [False, True])
def test_mha_fp16_full(causal):
    w = W.WORKLOADS["mha_fp16_b4_h16_n2048"]
    q, k, v = (W.to_torch(x, "fp16") for x in W.qkv_f32(w))
    o = run(q, k, v, causal)
    ref = A.attention(q, k, v, None, causal)
    assert np.abs(o - ref).max() <= TOL["fp16"]


def sample_rows(N, seed, n=160, bm=128):
    rng = np.random.default_rng(seed)
    edges = [0, 1, N - 1] + [x for t in range(bm, N, bm * max(1, N // (bm * 16))) for x in (t - 1, t)]
    return np.unique(np.concatenate([edges, rng.integers(0, N, n)]))


@pytest.mark.parametrize("name,causal", [("gqa_bf16_h64kv8_n8192", True), ("gqa_bf16_h64kv8_n8192", False),
                                         ("long_bf16_h8kv1_n131072", True), ("long_bf16_h8kv1_n131072", False)])
def test_large_workloads_sampled_rows(name, causal):
    w = W.WORKLOADS[name]
    q, k, v = (W.to_torch(x, "bf16") for x in W.qkv_f32(w))
    o, lse = run(q, k, v, causal, lse=True)
    rows = sample_rows(w.N, w.wid, n=96 if w.N > 100000 else 160)
    heads = list(range(0, w.Hq, max(1, w.Hq // 8)))
    ref, ref_lse = A.attention_rows(q, k, v, rows, None, causal, heads=heads)
    err = np.abs(o[:, rows][:, :, heads] - ref).max()
    print(f"{name} causal={causal}: {len(rows)} rows x {len(heads)} heads, max|dO| = {err:.3e}")
    assert err <= TOL["bf16"]
    tol = lse_tol(q, k, "bf16", rows=rows, heads=heads, causal=causal)
    check_lse(lse[:, heads][:, :, rows], ref_lse, tol, f"{name} causal={causal}")
    assert np.isfinite(o).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_long_sequence_d64(dtype):
    # d = 64 at 64k keys, causal, GQA 4/2: sampled rows at tile and item boundaries.
    N = 65536
    q, k, v = (W.to_torch(x, dtype) for x in W.random_qkv(44, 1, N, 4, 2, 64))
    o, lse = run(q, k, v, True, lse=True)
    rows = sample_rows(N, 44, n=64, bm=256)
    ref, ref_lse = A.attention_rows(q, k, v, rows, None, True)
    err = np.abs(o[:, rows] - ref).max()
    print(f"d=64 N={N} {dtype}: max|dO| = {err:.3e}")
    assert err <= TOL[dtype] and np.isfinite(o).all()
    tol = lse_tol(q, k, dtype, rows=rows, causal=True)
    check_lse(lse[:, :, rows], ref_lse, tol, f"d=64 N={N} {dtype}")


@pytest.mark.parametrize("causal,N", [(False, 2048), (True, 4096)])
def test_uneven_persistent_shares(causal, N):
    # 320 work items on a 256-workgroup grid with the XCD-contiguous dealing on: some
    # workgroups walk two items, the others one; every row of every 4th head is checked
    # at item boundaries and at random.
    q, k, v = (W.to_torch(x, "bf16") for x in W.random_qkv(41, 1, N, 40, 8, 128))
    o = run(q, k, v, causal)
    rows = sample_rows(N, 41, n=96, bm=256)
    heads = list(range(0, 40, 4)) + [39]
    ref, _ = A.attention_rows(q, k, v, rows, None, causal, heads=heads)
    err = np.abs(o[:, rows][:, :, heads] - ref).max()
    print(f"uneven shares causal={causal}: max|dO| = {err:.3e}")
    assert err <= TOL["bf16"] and np.isfinite(o).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "fp16")])
def test_many_tasks_per_workgroup_ragged(d, dtype, causal):
    # 960 (non-causal) or 576 (causal) q tiles on 256 workgroups with N = 1100: each
    # workgroup walks several, and the tile counts (4, 8, 12, 16, 18 tiles of 64 keys) are
    # and are not multiples of the ring depth, so the ring's stage sequence restarts at
    # every phase.  Every row of every 8th head is checked.
    B, N, Hq, Hkv = 2, 1100, 96, 8
    q, k, v = (W.to_torch(x, dtype) for x in W.random_qkv(48 + d, B, N, Hq, Hkv, d))
    o, lse = run(q, k, v, causal, lse=True)
    heads = list(range(0, Hq, 8)) + [Hq - 1]
    rows = np.arange(N)
    ref, ref_lse = A.attention_rows(q, k, v, rows, None, causal, heads=heads)
    err = np.abs(o[:, :, heads] - ref).max()
    print(f"many tasks d={d} {dtype} causal={causal}: max|dO| = {err:.3e}")
    assert err <= TOL[dtype] and np.isfinite(o).all()
    tol = lse_tol(q, k, dtype, rows=rows, heads=heads, causal=causal)
    check_lse(lse[:, heads], ref_lse, tol, f"many tasks d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_causal_row0_is_v0_bit_exact(dtype):
    q, k, v = (W.to_torch(x, dtype) for x in W.random_qkv(31, 2, 300, 4, 2, 128))
    o = T.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True).cpu()
    for h in range(4):
        assert torch.equal(o[:, 0, h], v[:, 0, h // 2])


def test_deterministic_and_gqa_equals_repeated_mha():
    q, k, v = (W.to_torch(x, "bf16").to(DEV) for x in W.random_qkv(32, 1, 777, 8, 2, 128))
    a = T.attn_fwd(q, k, v, causal=True)
    b = T.attn_fwd(q, k, v, causal=True)
    c = T.attn_fwd(q, k.repeat_interleave(4, dim=2).contiguous(), v.repeat_interleave(4, dim=2).contiguous(),
                   causal=True)
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_move_the_reference_max(dtype, causal):
    # Keys whose magnitude ramps along the sequence make a row's scores climb by
    # ~65 in log2 units from the first tile to the last, so the kernel must move
    # its reference max (and rescale O and z) several times: each move happens
    # before a tile's probabilities could leave the 16-bit operand range.
    rng = np.random.default_rng(77)
    B, N, Hq, Hkv, d = 1, 700, 2, 1, 128
    q = 1.0 + 0.1 * rng.standard_normal((B, N, Hq, d))
    ramp = np.linspace(-1.0, 3.0, N)[None, :, None, None]
    k = ramp + 0.1 * rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    q, k, v = (W.to_torch(x.astype(np.float32), dtype) for x in (q, k, v))
    o, lse = run(q, k, v, causal, lse=True)
    ref, ref_lse = A.attention(q, k, v, None, causal, return_lse=True)
    assert np.isfinite(o).all()
    assert np.abs(o - ref).max() <= TOL[dtype]
    check_lse(lse, ref_lse, lse_tol(q, k, dtype, causal=causal), f"ramp {dtype} causal={causal}")


def test_scale_argument_is_used():
    q, k, v = (W.to_torch(x, "fp16") for x in W.random_qkv(33, 1, 200, 2, 2, 64))
    o = run(q, k, v, False, scale=0.37)
    assert np.abs(o - A.attention(q, k, v, 0.37)).max() <= TOL["fp16"]


def test_binding_rejects_bad_calls():
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        T.attn_fwd(q, q[:, :32].contiguous(), q)
    with pytest.raises(TypeError):
        T.attn_fwd(q.float(), q.float(), q.float())
    q96 = torch.zeros(1, 64, 2, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(T.TattnError) as e:
        T.attn_fwd(q96, q96, q96)
    assert e.value.status == 2


def exact_16bit_inputs(seed, B, N, Hq, Hkv, d, dtype):
    """Integer Q, K, V on which the 16-bit path rounds nothing before the output.

    Each query row has at most 4 nonzero entries of 1 or 2, K entries are 0/1 and
    V entries integers in [-8, 8], all exact in bf16 and fp16.  With softmax
    scale ln 2 the kernel's factor c = fl32(scale·log2(e)) is exactly 1, so a
    score in log2 units is an integer in [0, 8].  Key 0 has all-one K, so it
    holds every row's maximum in the first key tile, where the reference max is
    set and never moves.  Every probability is then a power of two between 2^-8
    and 1, exact in both types, and every P·V product and partial sum (up to
    4096 keys) lies on a 2^-8 grid below 2^15, which fp32 accumulation keeps
    exactly even when the matrix cores truncate small terms.
    """
    rng = np.random.default_rng(seed)
    q = np.zeros((B, N, Hq, d))
    np.put_along_axis(q, rng.integers(0, d, (B, N, Hq, 4)), 1.0, axis=-1)
    q *= rng.integers(1, 3, (B, N, Hq, d))
    k = rng.integers(0, 2, (B, N, Hkv, d)).astype(np.float64)
    k[:, 0] = 1.0
    v = rng.integers(-8, 9, (B, N, Hkv, d)).astype(np.float64)
    tt = tuple(W.to_torch(x.astype(np.float32), dtype) for x in (q, k, v))
    for a, x in zip(tt, (q, k, v)):
        assert np.array_equal(a.double().numpy(), x)
    check_rows = rng.choice(N, min(N, 64), replace=False)
    for b in range(B):
        for h in range(Hq):
            s = q[b, check_rows, h] @ k[b, :, h // (Hq // Hkv)].T      # log2-unit scores
            assert s.min() >= 0 and s.max() <= 8 and (s == s.round()).all() and (s.max(axis=1) == s[:, 0]).all()
    return tt, (q, k, v)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1000, 8, 2, 128), (2, 4096, 8, 1, 128), (1, 777, 4, 4, 64)],
                         ids=lambda s: "B{}N{}H{}/{}d{}".format(*s))
def test_equals_exact_attention_when_nothing_rounds(shape, causal, dtype):
    # With exact inputs and exactly representable probabilities the kernel is
    # exact attention up to the one rounding of the output to the input type.
    import math
    B, N, Hq, Hkv, d = shape
    (qt, kt, vt), (q, k, v) = exact_16bit_inputs(70 + N, B, N, Hq, Hkv, d, dtype)
    scale = math.log(2.0)
    o, lse = run(qt, kt, vt, causal, scale=scale, lse=True)
    rows = np.arange(N) if N <= 1000 else np.unique(np.concatenate(
        [np.arange(0, 70), np.arange(N - 70, N), np.random.default_rng(N).choice(N, 200, replace=False)]))
    want, want_lse = A.attention_rows(q, k, v, rows, scale, causal)
    got = o[:, rows]
    err = np.abs(got - want)
    tol = 1.01 * U[dtype] * np.abs(want) + 1e-6
    bad = np.argwhere(err > tol)
    detail = [(int(rows[r]), int(h), int(c), float(got[b, r, h, c]), float(want[b, r, h, c]))
              for b, r, h, c in bad[:8]]
    assert len(bad) == 0, f"{len(bad)} elements off, max err {err.max():.3g}; (row, head, ch, got, want): {detail}"
    np.testing.assert_allclose(lse[:, :, rows], want_lse, rtol=1e-5, atol=1e-5)
