"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds none of the attention arithmetic: it only draws numbers and
rounds them to the storage dtype.  Every tensor is laid out [B, N, H, d].

Recipe: ``np.random.default_rng([workload_id, tensor_id])`` draws standard
normals in fp32 (tensor 0 = Q, 1 = K, 2 = V, 3 = rotation signs, 4 = outlier
channels, 5 = rotary angles); the values are then rounded to nearest-even into
fp16 or bf16.  The
FP8 workload first multiplies one seeded channel per head of Q and K by 20
(0.5 % of d = 128 channels rounds up to one channel per head).

Decode workloads draw the query from tensor 0, each sequence's K and V cache
rows from the streams [workload_id, 1, b] and [workload_id, 2, b], and the
sequence lengths (a mix between Nmax/2 and Nmax, the last one full) from
tensor 6; the cache rows are rounded to the query's 16-bit type and stored as
E4M3 codes with 64-row block scales, made by the block quantiser from these
values.  ``random_e4m3_cache`` instead draws the codes themselves (every finite
E4M3FN code equally likely) and the block scales, for edge cases that must
cover all codes.

The workloads follow the shapes the pages discuss: the tiny single-head check,
multi-head fp16 (the B=2, N=2048, d=128 benchmark of the FA3 deep-dive page,
widened to 4 × 16 heads), one layer of a 70B-class model with grouped KV heads,
the 128k-token single-layer prefill of the tile-pipeline page taken as one
GPU's 8-head share, and FP8 with activation outliers.  No public dataset is
involved: the synthetic tensors stand in for activations.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed namespace
    B: int
    N: int
    Hq: int
    Hkv: int
    d: int
    dtype: str          # storage dtype of Q, K, V: "fp32", "fp16", "bf16"
    causal: tuple       # causal settings exercised
    outlier_scale: float = 0.0
    fp8: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self, causal: bool) -> float:
        f = 4.0 * self.B * self.N * self.N * self.d * self.Hq
        return f / 2 if causal else f


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_h1_n128_d64", 1, 1, 128, 1, 1, 64, "fp32", (False,)),
        Workload("mha_fp16_b4_h16_n2048", 2, 4, 2048, 16, 16, 128, "fp16", (False, True)),
        Workload("gqa_bf16_h64kv8_n8192", 3, 1, 8192, 64, 8, 128, "bf16", (True, False)),
        Workload("long_bf16_h8kv1_n131072", 4, 1, 131072, 8, 1, 128, "bf16", (True,)),
        Workload("fp8_outlier_b2_h16_n4096", 5, 2, 4096, 16, 16, 128, "bf16", (False,),
                 outlier_scale=20.0, fp8=True),
    ]
}

HEADLINE = "gqa_bf16_h64kv8_n8192"       # run non-causal for the headline figure


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: B sequences, each with one new query token [B, Hq, d]
    attending to its own cached K/V [B, Nmax, Hkv, d] (the first seqlens[b] rows)."""
    name: str
    wid: int
    B: int
    Nmax: int
    Hq: int
    Hkv: int
    d: int
    dtype: str          # storage dtype of the query and the output

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def seqlens(self) -> np.ndarray:
        """Length mix: uniform integers in [Nmax/2, Nmax] (tensor 6), the last
        sequence full; int32 [B]."""
        L = _rng(self.wid, 6).integers(self.Nmax // 2, self.Nmax + 1, size=self.B)
        L[-1] = self.Nmax
        return L.astype(np.int32)

    def hbm_bytes(self, seqlens) -> int:
        """Bytes a decode step must move at least: the valid cache rows (one byte
        per K and V element), their block scales, the query and the output."""
        rows = int(np.sum(np.asarray(seqlens, dtype=np.int64)))
        blocks = int(np.sum((np.asarray(seqlens, dtype=np.int64) + 63) // 64))
        return rows * self.Hkv * self.d * 2 + blocks * self.Hkv * 4 * 2 + 2 * self.B * self.Hq * self.d * 2


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        DecodeWorkload("decode_fp8kv_b3_h8kv2_n1000", 6, 3, 1000, 8, 2, 128, "bf16"),
        DecodeWorkload("decode_fp8kv_b4_h64kv8_n131072", 7, 4, 131072, 64, 8, 128, "bf16"),
    ]
}


def decode_query_f32(w: DecodeWorkload) -> np.ndarray:
    """fp32 query [B, Hq, d] of a decode workload (tensor 0)."""
    return normal(w.wid, 0, (w.B, w.Hq, w.d))


def decode_cache_f32(w: DecodeWorkload, b: int):
    """fp32 K and V cache rows [Nmax, Hkv, d] of sequence b (tensors 1 and 2, one
    stream per sequence so a sequence is drawn without the others)."""
    k = np.random.default_rng([w.wid, 1, b]).standard_normal(size=(w.Nmax, w.Hkv, w.d), dtype=np.float32)
    v = np.random.default_rng([w.wid, 2, b]).standard_normal(size=(w.Nmax, w.Hkv, w.d), dtype=np.float32)
    return k, v


def random_e4m3_cache(seed: int, B: int, N: int, H: int, d: int):
    """Random finite E4M3FN codes (uint8 [B, N, H, d]; the two NaN codes 0x7f and
    0xff are never drawn) and block scales (fp32 [B, H, ceil(N/64)], uniform in
    [1/128, 1/32))."""
    r = np.random.default_rng([2000 + seed, 7])
    codes = r.integers(0, 254, size=(B, N, H, d), dtype=np.int64)
    codes = codes + (codes >= 0x7F)              # skip 0x7f; 0xfe is the largest drawn, so 0xff never appears
    scales = r.uniform(1 / 128, 1 / 32, size=(B, H, -(-N // 64))).astype(np.float32)
    return codes.astype(np.uint8), scales


def _rng(wid: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([wid, tensor])


def normal(wid: int, tensor: int, shape) -> np.ndarray:
    return _rng(wid, tensor).standard_normal(size=shape, dtype=np.float32)


def rotation_signs(wid: int, d: int) -> np.ndarray:
    """Seeded ±1 vector (int8) of length d."""
    return np.where(_rng(wid, 3).integers(0, 2, size=d) == 1, 1, -1).astype(np.int8)


def rotary_tables(wid: int, N: int, d: int):
    """Seeded rotary tables: cos and sin (fp32 [N, d/2]) of angles drawn uniformly
    in [-pi, pi) (tensor 5).  Any angles are valid inputs of the rotary step."""
    ang = _rng(wid, 5).uniform(-np.pi, np.pi, size=(N, d // 2))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def outlier_channels(wid: int, H: int, d: int) -> np.ndarray:
    """One seeded channel per head: ceil(0.005·d) = 1 for d = 128."""
    return _rng(wid, 4).integers(0, d, size=H)


def qkv_f32(w: Workload):
    """fp32 Q, K, V of workload ``w`` before rounding to its storage dtype."""
    q = normal(w.wid, 0, (w.B, w.N, w.Hq, w.d))
    k = normal(w.wid, 1, (w.B, w.N, w.Hkv, w.d))
    v = normal(w.wid, 2, (w.B, w.N, w.Hkv, w.d))
    if w.outlier_scale:
        ch = outlier_channels(w.wid, w.Hq, w.d)
        for h in range(w.Hq):
            q[:, :, h, ch[h]] *= np.float32(w.outlier_scale)
        chk = ch[:: w.Hq // w.Hkv]
        for h in range(w.Hkv):
            k[:, :, h, chk[h]] *= np.float32(w.outlier_scale)
    return q, k, v


def random_qkv(seed: int, B: int, N: int, Hq: int, Hkv: int, d: int, Nk: int | None = None):
    """fp32 Q, K, V for ad-hoc shapes (edge cases, ragged tails)."""
    Nk = N if Nk is None else Nk
    base = 1000 + seed
    return (normal(base, 0, (B, N, Hq, d)), normal(base, 1, (B, Nk, Hkv, d)),
            normal(base, 2, (B, Nk, Hkv, d)))


def to_torch(x: np.ndarray, dtype: str):
    """Round an fp32 array to the storage dtype (nearest-even) as a CPU torch tensor."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to({"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype])
