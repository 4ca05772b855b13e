"""exp2_valu, the VALU-pipe 2^x of the kernels (tattn_device.hpp), on the CPU.

The kernels' device sequence is emulated step by step in fp32: f = fract(x),
n = floor(x), Horner's rule with one rounding per fused multiply-add, and
ldexp.  Checked against fp64 2^x: the relative error stays within the minimax
bound its coefficients were derived for, integers are exact, and the constants
in the header are the ones the derivation gives.
"""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "tiled_attention_10_amd", "csrc", "tattn_device.hpp")


def header_coefficients():
    text = open(HEADER).read()
    return [np.float32(float.fromhex(re.search(rf"kExp2A{i} = (0x[0-9a-f.]+p-?\d+)f;", text).group(1)))
            for i in (1, 2, 3)]


def fma32(a, b, c):
    # a·b is exact in fp64 for fp32 operands; one rounding of the sum to fp32
    return (a.astype(np.float64) * b + c).astype(np.float32)


def exp2_valu(x):
    a1, a2, a3 = header_coefficients()
    x = np.asarray(x, dtype=np.float32)
    fl = np.floor(x)
    f = (x - fl).astype(np.float32)          # exact for fp32 x
    p = fma32(np.full_like(f, a3), f, a2)
    p = fma32(p, f, a1)
    p = fma32(p, f, np.float32(1.0))
    return np.ldexp(p.astype(np.float64), fl.astype(np.int64)).astype(np.float32)


def test_header_constants_are_the_derived_minimax_cubic():
    pytest.importorskip("scipy")
    import importlib.util
    spec = importlib.util.spec_from_file_location("exp2_poly", os.path.join(ROOT, "tiled_attention_10_amd", "csrc",
                                                                             "exp2_poly.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    a, err = mod.coefficients()
    assert np.array_equal(a.astype(np.float32), np.array(header_coefficients(), dtype=np.float32))
    assert err < 1.04e-4


def test_relative_error_within_minimax_bound():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-120, 15, 2_000_000), np.linspace(-3, 3, 600_001)]).astype(np.float32)
    got = exp2_valu(x).astype(np.float64)
    want = np.exp2(x.astype(np.float64))
    rel = np.abs(got / want - 1)
    assert rel.max() <= 1.05e-4, rel.max()


def test_exact_at_integers_and_continuous_across_them():
    n = np.arange(-125, 20, dtype=np.float32)
    assert np.array_equal(exp2_valu(n), np.exp2(n.astype(np.float64)).astype(np.float32))
    # just below an integer f is close to 1, where P(1) = 2 makes the error vanish
    below = np.nextafter(n, np.float32(-np.inf))
    assert (np.abs(exp2_valu(below) / np.exp2(below.astype(np.float64)) - 1) < 1e-6).all()


def test_underflow_and_overflow_like_v_exp():
    assert exp2_valu(np.float32(-200.5)) == 0.0
    assert np.isinf(exp2_valu(np.float32(130.25)))
