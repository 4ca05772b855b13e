"""tiled_attention_10_amd — fused attention forward for MI355X (gfx950).

A thin ctypes binding over ``libtattn.so`` (see ``include/tattn.h``).  The
functions here only check and marshal arguments; every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device
memory and the current stream.  If the library has not been built, every call
raises: there is no fallback implementation.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

__all__ = ["attn_fwd", "attn_fwd_fp8", "hadamard_rotate", "rope_hadamard_rotate", "fp8_prologue", "attn_decode_fp8kv",
           "decode_workspace_size", "TattnError", "lib", "LIB_PATH", "TATTN_F16", "TATTN_BF16",
           "use_library", "variant_path", "attn_decode_fp8kv_noalloc", "TATTN_NOALLOC_SCRATCH_BYTES"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtattn.so")

TATTN_F16 = 1
TATTN_BF16 = 2
TATTN_NOALLOC_SCRATCH_BYTES = 16 << 20     # the fixed decode scratch of attn_decode_fp8kv_noalloc
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "misaligned", 4: "HIP error"}

_lib = None


class TattnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"tattn status {status} ({_STATUS.get(status, '?')}): {detail}")
        self.status = status


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m tiled_attention_10_amd.build`")
    L = ctypes.CDLL(path)
    _declare(L)
    return L


def lib() -> ctypes.CDLL:
    """Load libtattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def variant_path(name: str) -> str:
    """Path of a scheduling variant of the library (``libtattn_<name>.so``, built by build.py)."""
    return os.path.join(os.path.dirname(LIB_PATH), f"libtattn_{name}.so")


@contextlib.contextmanager
def use_library(path: str):
    """Route this module's calls through another build of the same ABI (a scheduling
    variant of the kernels) for the duration of the block."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _declare(L: ctypes.CDLL) -> None:
    """Argument and result types of the exported functions."""
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd_fp8.restype = i
    L.hadamard_rotate.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    L.hadamard_rotate.restype = i
    L.rope_hadamard_rotate.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    L.rope_hadamard_rotate.restype = i
    L.fp8_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    L.fp8_prologue.restype = i
    L.attn_decode_fp8kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                     i, i, i, i, i, f, i, vp]
    L.attn_decode_fp8kv.restype = i
    L.attn_decode_fp8kv_workspace_size.argtypes = [i, i, i, i, i]
    L.attn_decode_fp8kv_workspace_size.restype = ctypes.c_size_t
    L.attn_decode_fp8kv_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_decode_fp8kv_noalloc.restype = i
    L.tattn_status_string.argtypes = [i]
    L.tattn_status_string.restype = ctypes.c_char_p
    L.tattn_last_error.argtypes = []
    L.tattn_last_error.restype = ctypes.c_char_p


def _check(status: int) -> None:
    if status != 0:
        raise TattnError(status, lib().tattn_last_error().decode(errors="replace"))


def _torch():
    import torch

    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float16:
        return TATTN_F16
    if dt == torch.bfloat16:
        return TATTN_BF16
    raise TypeError(f"unsupported dtype {dt} (float16 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one device")
    return dev


def _stream(dev):
    return ctypes.c_void_p(_torch().cuda.current_stream(dev).cuda_stream)


def _shape4(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, N, H, d]")
    B, N, Hq, d = q.shape
    if tuple(k.shape) != tuple(v.shape) or k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    return B, N, Hq, k.shape[2], d


def _out(out, shape, dtype, dev, name):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype:
        raise ValueError(f"{name} must be {tuple(shape)} {dtype}")
    _dev(out)
    return out


def attn_fwd(q, k, v, causal: bool = False, softmax_scale: float | None = None, out=None,
             return_lse: bool = False, lse=None):
    """O = softmax(scale·QKᵀ + mask)·V for fp16/bf16 [B, N, H, d] tensors."""
    B, N, Hq, Hkv, d = _shape4(q, k, v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    dev = _dev(q, k, v)
    code = _dtype_code(q.dtype)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = _out(out, (B, N, Hq, d), q.dtype, dev, "out")
    if return_lse or lse is not None:
        lse = _out(lse, (B, Hq, N), _torch().float32, dev, "lse")
    _check(lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, N, Hq, Hkv, d,
                          scale, int(bool(causal)), code, _stream(dev)))
    return (out, lse) if lse is not None else out


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False,
                 softmax_scale: float | None = None, out_dtype=None, out=None,
                 return_lse: bool = False, lse=None):
    """Attention on E4M3FN codes (uint8 [B, N, H, d]) with fp32 [B, H, ceil(N/64)] scales."""
    torch = _torch()
    B, N, Hq, Hkv, d = _shape4(q8, k8, v8)
    for t in (q8, k8, v8):
        if t.dtype != torch.uint8:
            raise TypeError("q8, k8, v8 must be uint8 E4M3FN codes")
    nb = (N + 63) // 64
    for t, h, name in ((q_scale, Hq, "q_scale"), (k_scale, Hkv, "k_scale"), (v_scale, Hkv, "v_scale")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, h, nb):
            raise ValueError(f"{name} must be float32 {(B, h, nb)}")
    dev = _dev(q8, k8, v8, q_scale, k_scale, v_scale)
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    code = _dtype_code(out_dtype)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = _out(out, (B, N, Hq, d), out_dtype, dev, "out")
    if return_lse or lse is not None:
        lse = _out(lse, (B, Hq, N), torch.float32, dev, "lse")
    _check(lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale),
                              _ptr(v_scale), _ptr(out), _ptr(lse), B, N, Hq, Hkv, d, scale,
                              int(bool(causal)), code, _stream(dev)))
    return (out, lse) if lse is not None else out


def hadamard_rotate(x, signs=None, quantize: bool = False, out=None, scales=None):
    """Rotate rows of x [B, N, H, d] by H_d·diag(signs)/sqrt(d) (signs None: no rotation).

    quantize=False: returns the rotated tensor in x's dtype.
    quantize=True:  returns (uint8 E4M3FN codes [B, N, H, d], fp32 scales [B, H, ceil(N/64)]).
    """
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [B, N, H, d]")
    B, N, H, d = x.shape
    code = _dtype_code(x.dtype)
    if signs is not None:
        if signs.dtype != torch.int8 or tuple(signs.shape) != (d,):
            raise ValueError(f"signs must be int8 [{d}]")
    dev = _dev(x, signs)
    if quantize:
        out = _out(out, (B, N, H, d), torch.uint8, dev, "out")
        scales = _out(scales, (B, H, (N + 63) // 64), torch.float32, dev, "scales")
    else:
        out = _out(out, (B, N, H, d), x.dtype, dev, "out")
        scales = None
    _check(lib().hadamard_rotate(_ptr(x), _ptr(out), _ptr(signs), _ptr(scales), B, N, H, d, code,
                                 _stream(dev)))
    return (out, scales) if quantize else out


def rope_hadamard_rotate(x, rope_cos, rope_sin, signs=None, quantize: bool = False, out=None, scales=None):
    """Rotary embedding of x [B, N, H, d] by the fp32 tables rope_cos/rope_sin [N, d/2]
    (channel pairs (i, i + d/2)), then exactly ``hadamard_rotate`` in the same pass."""
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [B, N, H, d]")
    B, N, H, d = x.shape
    code = _dtype_code(x.dtype)
    for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        if t.dtype != torch.float32 or tuple(t.shape) != (N, d // 2) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32 [{N}, {d // 2}]")
    if signs is not None:
        if signs.dtype != torch.int8 or tuple(signs.shape) != (d,):
            raise ValueError(f"signs must be int8 [{d}]")
    dev = _dev(x, rope_cos, rope_sin, signs)
    if quantize:
        out = _out(out, (B, N, H, d), torch.uint8, dev, "out")
        scales = _out(scales, (B, H, (N + 63) // 64), torch.float32, dev, "scales")
    else:
        out = _out(out, (B, N, H, d), x.dtype, dev, "out")
        scales = None
    _check(lib().rope_hadamard_rotate(_ptr(x), _ptr(out), _ptr(rope_cos), _ptr(rope_sin), _ptr(signs),
                                      _ptr(scales), B, N, H, d, code, _stream(dev)))
    return (out, scales) if quantize else out


def fp8_prologue(q, k, v, signs=None, rope=None, out=None):
    """The FP8 prologue of one attention call in one launch: q [B, N, Hq, d] and k, v
    [B, N, Hkv, d] (fp16/bf16); Q and K rotated with ``signs`` (int8 [d], None: no rotation)
    after the rotary embedding ``rope`` = (cos, sin) fp32 [N, d/2] (None: none), and all
    three block-quantised.  Returns (q8, k8, v8, q_scale, k_scale, v_scale), the arguments
    of ``attn_fwd_fp8``; ``out`` may give those six tensors to write into."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, N, H, d]")
    B, N, Hq, d = q.shape
    if tuple(k.shape) != tuple(v.shape) or k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    Hkv = k.shape[2]
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    code = _dtype_code(q.dtype)
    if signs is not None and (signs.dtype != torch.int8 or tuple(signs.shape) != (d,)):
        raise ValueError(f"signs must be int8 [{d}]")
    rc, rs = (None, None) if rope is None else rope
    for name, t in (("rope cos", rc), ("rope sin", rs)):
        if rope is not None and (t.dtype != torch.float32 or tuple(t.shape) != (N, d // 2) or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 [{N}, {d // 2}]")
    dev = _dev(q, k, v, signs, rc, rs)
    nb = (N + 63) // 64
    shapes = [((B, N, Hq, d), torch.uint8), ((B, N, Hkv, d), torch.uint8), ((B, N, Hkv, d), torch.uint8),
              ((B, Hq, nb), torch.float32), ((B, Hkv, nb), torch.float32), ((B, Hkv, nb), torch.float32)]
    names = ["q8", "k8", "v8", "q_scale", "k_scale", "v_scale"]
    outs = [None] * 6 if out is None else list(out)
    if len(outs) != 6:
        raise ValueError("out must hold six tensors (q8, k8, v8, q_scale, k_scale, v_scale)")
    outs = [_out(o, shp, dt, dev, n) for o, (shp, dt), n in zip(outs, shapes, names)]
    _check(lib().fp8_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(signs), _ptr(rc), _ptr(rs), *(_ptr(o) for o in outs),
                              B, N, Hq, Hkv, d, code, _stream(dev)))
    return tuple(outs)


def decode_workspace_size(B: int, Nmax: int, Hq: int, Hkv: int, d: int) -> int:
    """Bytes of device workspace ``attn_decode_fp8kv`` needs (0 for invalid sizes)."""
    return int(lib().attn_decode_fp8kv_workspace_size(B, Nmax, Hq, Hkv, d))


def attn_decode_fp8kv(q, k_cache, v_cache, k_scale, v_scale, seqlens, softmax_scale: float | None = None,
                      out=None, return_lse: bool = False, lse=None, workspace=None):
    """One decode step: q [B, Hq, d] (fp16/bf16) against an E4M3 KV cache (uint8 [B, Nmax, Hkv, d],
    fp32 block scales [B, Hkv, ceil(Nmax/64)]) holding seqlens[b] (int32, on the device) rows per
    sequence.  Returns O [B, Hq, d] in q's dtype (and LSE [B, Hq], fp32).  ``workspace`` is a
    uint8 device tensor of at least ``decode_workspace_size`` bytes (allocated here if None)."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the caches [B, Nmax, Hkv, d]")
    B, Hq, d = q.shape
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, v {tuple(v_cache.shape)}")
    Nmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    for t in (k_cache, v_cache):
        if t.dtype != torch.uint8:
            raise TypeError("caches must be uint8 E4M3FN codes")
    nb = (Nmax + 63) // 64
    for t, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, Hkv, nb):
            raise ValueError(f"{name} must be float32 {(B, Hkv, nb)}")
    if seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,):
        raise ValueError(f"seqlens must be int32 [{B}]")
    code = _dtype_code(q.dtype)
    dev = _dev(q, k_cache, v_cache, k_scale, v_scale, seqlens)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = _out(out, (B, Hq, d), q.dtype, dev, "out")
    if return_lse or lse is not None:
        lse = _out(lse, (B, Hq), torch.float32, dev, "lse")
    need = decode_workspace_size(B, Nmax, Hq, Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _dev(workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().attn_decode_fp8kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                   _ptr(seqlens), _ptr(out), _ptr(lse), _ptr(workspace), nbytes,
                                   B, Nmax, Hq, Hkv, d, scale, code, _stream(dev)))
    return (out, lse) if lse is not None else out


def attn_decode_fp8kv_noalloc(q, k_cache, v_cache, k_scale, v_scale, seqlens, softmax_scale: float | None = None,
                              out=None, return_lse: bool = False, lse=None):
    """``attn_decode_fp8kv`` through the entry point that allocates nothing: the library's
    fixed per-device scratch (TATTN_NOALLOC_SCRATCH_BYTES) replaces the workspace.  Pass
    ``out`` (and ``lse``) to keep this call free of allocations as well; calls that overlap
    in time on one GPU race on the shared scratch."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the caches [B, Nmax, Hkv, d]")
    B, Hq, d = q.shape
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, v {tuple(v_cache.shape)}")
    Nmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    for t in (k_cache, v_cache):
        if t.dtype != torch.uint8:
            raise TypeError("caches must be uint8 E4M3FN codes")
    nb = (Nmax + 63) // 64
    for t, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, Hkv, nb):
            raise ValueError(f"{name} must be float32 {(B, Hkv, nb)}")
    if seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,):
        raise ValueError(f"seqlens must be int32 [{B}]")
    code = _dtype_code(q.dtype)
    dev = _dev(q, k_cache, v_cache, k_scale, v_scale, seqlens)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = _out(out, (B, Hq, d), q.dtype, dev, "out")
    if return_lse or lse is not None:
        lse = _out(lse, (B, Hq), torch.float32, dev, "lse")
    _check(lib().attn_decode_fp8kv_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                           _ptr(seqlens), _ptr(out), _ptr(lse), B, Nmax, Hq, Hkv, d, scale, code,
                                           _stream(dev)))
    return (out, lse) if lse is not None else out
