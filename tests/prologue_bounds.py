"""Error bounds for comparing an fp32 evaluation of the FP8 prologue with the oracle.

The oracle (oracle/quant.py, oracle/rope.py) decides every output from fp64
values by the definition.  A GPU kernel evaluates the same steps in fp32, so
its outputs may differ where an fp64 value lies within the fp32 evaluation's
error of a rounding boundary.  The functions here bound that error element by
element, rigorously, for ANY fp32 evaluation of this shape:

* rotary embedding: each output is one sum of two products of exact fp32
  numbers, each operation rounded at most once (a fused multiply-add only
  lowers the error): |err| <= u·(|p1| + |p2| + |r|) <= 2.01·u·(|p1| + |p2|);
* rotation: each output of the unnormalised transform is a depth-log2(d)
  tree of additions of the inputs, so |err| <= γ_L·Σ|x| (γ_L = L·u/(1 − L·u),
  L = log2 d), plus the propagated input error Σ e_in; then one product with
  fl32(1/sqrt(d)), adding 2u·|y|;
* quantiser: codes of fl32(y·fl32(448/absmax)) against y / fl32(absmax_64/448),
  with the block absmax itself known to within the block's largest error E.

A value rounds (monotonically) into [round(v − δ), round(v + δ)]; outside the
elements where those two differ the result must equal the oracle's exactly.
u is fp32's unit roundoff 2^-24.
"""
from __future__ import annotations

import numpy as np

from oracle import e4m3
from oracle import hadamard as Hd
from oracle import quant

U32 = 2.0 ** -24


def rope_error(x, cos, sin):
    """fp64 values and per-element error bound of an fp32 rotary embedding of exact x."""
    from oracle import rope as R
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float64)[None, :, None, :]
    s = np.asarray(sin, dtype=np.float64)[None, :, None, :]
    a, b = np.abs(x[..., :h]), np.abs(x[..., h:])
    mag = np.concatenate([a * np.abs(c) + b * np.abs(s), b * np.abs(c) + a * np.abs(s)], axis=-1)
    return R.rope(x, cos, sin), 2.01 * U32 * mag


def rotation_error(y_in, e_in, signs):
    """fp64 rotation of y_in and the per-element error bound of an fp32 rotation of values
    known to within e_in of y_in."""
    y_in = np.asarray(y_in, dtype=np.float64)
    d = y_in.shape[-1]
    L = int(np.log2(d))
    gamma = L * U32 / (1 - L * U32)
    e_in = np.zeros_like(y_in) if e_in is None else np.asarray(e_in, dtype=np.float64)
    e_t = e_in.sum(axis=-1, keepdims=True) + gamma * (np.abs(y_in) + e_in).sum(axis=-1, keepdims=True)
    y = Hd.rotate(y_in, signs)
    return y, 1.01 * (e_t / np.sqrt(d) + 2 * U32 * np.abs(y))


def prologue_error(x, signs=None, rope_tables=None):
    """fp64 prologue values (as the oracle's quantiser sees them) and their fp32 error bound."""
    y = np.asarray(x, dtype=np.float64)
    e = np.zeros_like(y)
    if rope_tables is not None:
        y, e = rope_error(y, *rope_tables)
    if signs is not None:
        y, e = rotation_error(y, e, signs)
    return y, e


def round_to(x, dtype):
    """Round fp64 values to nearest-even on the bf16 or fp16 grid, exactly, back as fp64."""
    mbits, emin = {"bf16": (7, -126), "fp16": (10, -14)}[dtype]
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    spacing = np.exp2(np.maximum(e, emin) - mbits)
    return np.rint(x / spacing) * spacing


def check_16bit(got, y, e_y, dtype):
    """got: GPU 16-bit values (as fp64); y, e_y: fp64 values and error bounds.  Returns
    (number of elements whose rounding the bound leaves open, total); raises on a violation."""
    got = np.asarray(got, dtype=np.float64)
    lo, hi = round_to(y - e_y, dtype), round_to(y + e_y, dtype)
    bad = (got < lo) | (got > hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{int(bad.sum())} outputs outside [round(y-δ), round(y+δ)]; first at {i}: "
                             f"got {got[i]!r}, y {y[i]!r}, δ {e_y[i]!r}")
    return int((lo != hi).sum()), got.size


def code_bounds(y, e_y, block=quant.BLOCK):
    """Oracle codes and scales of fp64 values y, and for each element the interval of E4M3
    values an fp32 quantiser within the error bounds e_y can produce, plus the scale bound."""
    codes, scales = quant.quantize_values(y, block)
    amax = quant.block_absmax(y, block)
    emax = quant.block_absmax(e_y, block)
    N = y.shape[1]
    A = quant.scale_rows(amax, N, block)
    E = quant.scale_rows(emax, N, block)
    if np.any((A > 0) & (A <= 2 * E)):
        raise ValueError("error bound too large against the block absmax")
    r = y / quant.scale_rows(scales, N, block)
    with np.errstate(divide="ignore", invalid="ignore"):
        delta = np.where(A > 0, 1.01 * 448.0 / A * (e_y + np.abs(y) * (E / (A - E) + 4 * U32)), 0.0)
    lo = e4m3.decode(e4m3.encode(r - delta))
    hi = e4m3.decode(e4m3.encode(r + delta))
    ulp = np.exp2(np.floor(np.log2(scales.astype(np.float64))) - 23)
    scale_tol = 1.01 * emax / 448.0 + ulp
    return codes, scales, lo, hi, scale_tol


def check_codes(got_codes, got_scales, y, e_y, block=quant.BLOCK):
    """Checks a GPU quantiser's codes and scales against the definition on fp64 values y.
    Returns (number of elements whose code the bound leaves open, total)."""
    codes, scales, lo, hi, scale_tol = code_bounds(y, e_y, block)
    got_scales = np.asarray(got_scales, dtype=np.float64)
    serr = np.abs(got_scales - scales.astype(np.float64))
    if not (serr <= scale_tol).all():
        i = tuple(np.argwhere(serr > scale_tol)[0])
        raise AssertionError(f"scale {i}: got {got_scales[i]!r}, oracle {scales[i]!r}, bound {scale_tol[i]!r}")
    v = e4m3.decode(np.asarray(got_codes, dtype=np.uint8))
    bad = (v < lo) | (v > hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{int(bad.sum())} codes outside the bound; first at {i}: got {v[i]!r}, "
                             f"allowed [{lo[i]!r}, {hi[i]!r}], oracle {e4m3.decode(codes[i])!r}")
    open_ = lo != hi
    same = e4m3.decode(codes) == v
    assert same[~open_].all()
    return int(open_.sum()), v.size
