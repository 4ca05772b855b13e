"""The C ABI on the CPU: the library loads, exports every function declared in
include/tattn.h, and rejects bad arguments with the documented status codes
before any HIP call (so these run without a GPU and make no compute call)."""
import ctypes
import os
import re
import subprocess

import pytest

import tiled_attention_10_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tattn.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, HIP = 0, 1, 2, 3, 4
P = 0x100000          # a 16-byte aligned fake address: never dereferenced, every call below is rejected
BAD = 0x100001        # misaligned fake address


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(T.LIB_PATH):
        from tiled_attention_10_amd.build import build
        build()
    return T.lib()


def test_header_declares_the_three_operations():
    fns = declared_functions()
    for name in ("attn_fwd", "attn_fwd_fp8", "hadamard_rotate", "rope_hadamard_rotate", "attn_decode_fp8kv",
                 "attn_decode_fp8kv_workspace_size", "tattn_status_string", "tattn_last_error"):
        assert name in fns


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", T.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings(L):
    for code, text in ((OK, b"ok"), (INVALID, b"invalid argument"), (MISALIGNED, b"misaligned pointer"),
                       (HIP, b"HIP runtime error"), (99, b"unknown status")):
        assert L.tattn_status_string(code) == text
    assert b"unsupported" in L.tattn_status_string(UNSUPPORTED)


def fwd(L, q=P, k=P, v=P, o=P, lse=None, B=1, N=128, Hq=2, Hkv=1, d=128, scale=0.125, causal=0, dtype=2):
    return L.attn_fwd(q, k, v, o, lse, B, N, Hq, Hkv, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(B=0), INVALID), (dict(N=0), INVALID),
    (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID), (dict(Hq=3, Hkv=2), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(dtype=0), UNSUPPORTED),
    (dict(dtype=3), UNSUPPORTED), (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID), (dict(causal=2), INVALID),
    (dict(q=BAD), MISALIGNED), (dict(v=BAD), MISALIGNED), (dict(o=P + 8), MISALIGNED),
    (dict(lse=P + 2), MISALIGNED), (dict(B=1 << 20, N=1 << 20, Hq=64, Hkv=8), INVALID),
    # 64 key rows of 2^18 KV heads of 256 bytes span 4 GiB: past the kernels' 32-bit tile offsets
    (dict(Hq=1 << 18, Hkv=1 << 18, N=1), INVALID),
])
def test_attn_fwd_rejects(L, kw, status):
    assert fwd(L, **kw) == status
    assert L.tattn_last_error() != b""


def fp8(L, d=128, out_dtype=2, scales=P, causal=0, q8=P, N=128, Hq=2, Hkv=2):
    return L.attn_fwd_fp8(q8, P, P, scales, P, P, P, None, 1, N, Hq, Hkv, d, 0.1, causal, out_dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), UNSUPPORTED), (dict(out_dtype=7), UNSUPPORTED), (dict(scales=None), INVALID),
    (dict(causal=-1), INVALID), (dict(q8=BAD), MISALIGNED), (dict(scales=P + 1), MISALIGNED),
    (dict(q8=None), INVALID), (dict(N=-5), INVALID), (dict(N=262145), UNSUPPORTED),
    (dict(Hq=1 << 19, Hkv=1 << 19, N=1), INVALID),
])
def test_attn_fwd_fp8_rejects(L, kw, status):
    assert fp8(L, **kw) == status


def rot(L, x=P, y=P, signs=None, scales=None, B=1, N=64, H=1, d=128, dtype=2):
    return L.hadamard_rotate(x, y, signs, scales, B, N, H, d, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(d=32), UNSUPPORTED), (dict(dtype=9), UNSUPPORTED),
    (dict(N=0), INVALID), (dict(x=BAD), MISALIGNED), (dict(scales=P + 3), MISALIGNED),
])
def test_hadamard_rotate_rejects(L, kw, status):
    assert rot(L, **kw) == status


def rope_rot(L, x=P, y=P, cos=P, sin=P, signs=None, scales=None, B=1, N=64, H=1, d=128, dtype=2):
    return L.rope_hadamard_rotate(x, y, cos, sin, signs, scales, B, N, H, d, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cos=None), INVALID), (dict(sin=None), INVALID), (dict(cos=P + 4), MISALIGNED),
    (dict(sin=P + 8), MISALIGNED), (dict(x=None), INVALID), (dict(d=32), UNSUPPORTED),
    (dict(dtype=9), UNSUPPORTED), (dict(N=0), INVALID), (dict(y=BAD), MISALIGNED),
])
def test_rope_hadamard_rotate_rejects(L, kw, status):
    assert rope_rot(L, **kw) == status
    assert L.tattn_last_error() != b""


def decode(L, q=P, kc=P, vc=P, ks=P, vs=P, sl=P, o=P, lse=None, ws=P, wsb=1 << 30, B=2, Nmax=1000, Hq=8, Hkv=2,
           d=128, scale=0.1, dtype=2):
    return L.attn_decode_fp8kv(q, kc, vc, ks, vs, sl, o, lse, ws, wsb, B, Nmax, Hq, Hkv, d, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(vs=None), INVALID), (dict(sl=None), INVALID),
    (dict(o=None), INVALID), (dict(ws=None), INVALID), (dict(B=0), INVALID), (dict(Nmax=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(Hkv=0), INVALID), (dict(d=64), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED),
    (dict(scale=0.0), INVALID), (dict(scale=float("inf")), INVALID), (dict(q=BAD), MISALIGNED),
    (dict(vc=P + 4), MISALIGNED), (dict(ws=P + 8), MISALIGNED), (dict(ks=P + 2), MISALIGNED),
    (dict(sl=P + 1), MISALIGNED), (dict(lse=P + 3), MISALIGNED), (dict(wsb=16), INVALID),
    (dict(B=1 << 20, Nmax=1 << 20, Hq=64, Hkv=8), INVALID), (dict(B=65536, Nmax=8), INVALID),
    (dict(Hq=65537 * 2, Hkv=65537, Nmax=8), INVALID), (dict(Hq=4, Hkv=4, d=0), UNSUPPORTED),
])
def test_attn_decode_fp8kv_rejects(L, kw, status):
    assert decode(L, **kw) == status
    assert L.tattn_last_error() != b""


def test_decode_workspace_size(L):
    f = L.attn_decode_fp8kv_workspace_size
    # B·Hq·ceil(Nmax/chunk)·(d + 2)·4 bytes; the chunk is a multiple of 256 keys
    n = f(2, 1000, 8, 2, 128)
    assert n > 0 and n % (2 * 8 * 130 * 4) == 0 and n // (2 * 8 * 130 * 4) == 4   # chunk 256
    big = f(4, 131072, 64, 8, 128)
    nc = big // (4 * 64 * 130 * 4)
    assert big % (4 * 64 * 130 * 4) == 0 and 131072 % nc == 0 and (131072 // nc) % 256 == 0
    for bad in ((0, 10, 8, 2, 128), (1, 10, 8, 3, 128), (1, 10, 8, 2, 64), (1, 0, 8, 2, 128)):
        assert f(*bad) == 0
    # the Python binding hands over exactly this size
    assert T.decode_workspace_size(2, 1000, 8, 2, 128) == n
    # a workspace one byte short of it is rejected before any HIP call
    assert decode(L, wsb=n - 1) == INVALID
    assert b"workspace" in L.tattn_last_error()


def test_python_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(T, "_lib", None)
    monkeypatch.setattr(T, "LIB_PATH", "/nonexistent/libtattn.so")
    with pytest.raises(ImportError):
        T.lib()


def test_clock_probe_library():
    # the benchmark's clock probe is a library of its own, outside the attention ABI
    path = os.path.join(os.path.dirname(T.LIB_PATH), "libtattn_clock.so")
    if not os.path.exists(path):
        from tiled_attention_10_amd.build import build_probe
        build_probe()
    P = ctypes.CDLL(path)
    u64 = ctypes.c_ulonglong
    P.tattn_clock_probe.argtypes = [u64, u64, ctypes.c_void_p, ctypes.c_void_p]
    # rejected before any launch
    assert P.tattn_clock_probe(0, 10, ctypes.c_void_p(0x100000), None) == 1
    assert P.tattn_clock_probe(10, 10, None, None) == 1
    out = subprocess.run(["nm", "-D", "--defined-only", T.LIB_PATH], capture_output=True, text=True).stdout
    assert "tattn_clock_probe" not in out


def decode_noalloc(L, q=P, kc=P, vc=P, ks=P, vs=P, sl=P, o=P, lse=None, B=2, Nmax=1000, Hq=8, Hkv=2, d=128,
                   scale=0.1, dtype=2):
    return L.attn_decode_fp8kv_noalloc(q, kc, vc, ks, vs, sl, o, lse, B, Nmax, Hq, Hkv, d, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(sl=None), INVALID), (dict(B=0), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED), (dict(scale=0.0), INVALID),
    (dict(q=BAD), MISALIGNED), (dict(ks=P + 2), MISALIGNED),
    # needs more than the fixed scratch: rejected before any HIP call
    (dict(B=64, Nmax=131072, Hq=64, Hkv=8), INVALID),
])
def test_attn_decode_fp8kv_noalloc_rejects(L, kw, status):
    assert decode_noalloc(L, **kw) == status
    assert L.tattn_last_error() != b""


def test_noalloc_scratch_limit_against_workspace_sizes(L):
    limit = 16 << 20
    assert L.attn_decode_fp8kv_workspace_size(64, 131072, 64, 8, 128) > limit
    # the benchmark's decode workload fits
    assert 0 < L.attn_decode_fp8kv_workspace_size(4, 131072, 64, 8, 128) <= limit
    decode_noalloc(L, B=64, Nmax=131072, Hq=64, Hkv=8)
    assert b"scratch" in L.tattn_last_error()


def prologue(L, q=P, k=P, v=P, signs=P, rc=None, rs=None, q8=P, k8=P, v8=P, sq=P, sk=P, sv=P, B=1, N=100,
             Hq=4, Hkv=2, d=128, dtype=2):
    return L.fp8_prologue(q, k, v, signs, rc, rs, q8, k8, v8, sq, sk, sv, B, N, Hq, Hkv, d, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(v8=None), INVALID), (dict(sk=None), INVALID), (dict(rc=P), INVALID),
    (dict(rs=P), INVALID), (dict(B=0), INVALID), (dict(Hq=3, Hkv=2), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED), (dict(k=BAD), MISALIGNED), (dict(q8=P + 8), MISALIGNED),
    (dict(sv=P + 2), MISALIGNED), (dict(rc=P + 4, rs=P), MISALIGNED),
    (dict(B=1 << 20, N=1 << 20, Hq=64, Hkv=8), INVALID),
])
def test_fp8_prologue_rejects(L, kw, status):
    assert prologue(L, **kw) == status
    assert L.tattn_last_error() != b""
