"""Pins of oracle/rope.py against properties the rotary embedding must have.

The pages give no worked rotary-embedding values, so the oracle is pinned by
what a rotation by θ of each channel pair fixes: identity at θ = 0, norm
preservation, composition of angles, the complex-number form, and the
relative-position property of the standard tables (the score between
positions m and n depends on m − n only).  A planted sign error must fail.
"""
import numpy as np
import pytest

from oracle import rope as R
from oracle import hadamard as Hd
from oracle import quant


def rng(seed):
    return np.random.default_rng(seed)


def random_tables(seed, N, d):
    ang = rng(seed).uniform(-np.pi, np.pi, (N, d // 2))
    return np.cos(ang), np.sin(ang), ang


def test_identity_at_angle_zero():
    x = rng(1).standard_normal((2, 5, 3, 16))
    c, s = np.ones((5, 8)), np.zeros((5, 8))
    assert np.array_equal(R.rope(x, c, s), x)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_pair_and_row_norms_preserved(d):
    x = rng(2).standard_normal((1, 7, 2, d))
    c, s, _ = random_tables(3, 7, d)
    y = R.rope(x, c, s)
    h = d // 2
    assert np.allclose(x[..., :h] ** 2 + x[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2, rtol=0, atol=1e-12)
    assert np.allclose(np.linalg.norm(x, axis=-1), np.linalg.norm(y, axis=-1), rtol=1e-13)


def test_complex_number_form():
    # pair (x_i, x_{i+d/2}) as x_i + j·x_{i+d/2}, multiplied by e^{jθ}
    d, N = 32, 9
    x = rng(4).standard_normal((2, N, 3, d))
    c, s, ang = random_tables(5, N, d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * ang)[None, :, None, :]
    want = np.concatenate([z.real, z.imag], axis=-1)
    assert np.allclose(R.rope(x, c, s), want, rtol=0, atol=1e-12)


def test_angles_compose():
    d, N = 16, 4
    x = rng(6).standard_normal((1, N, 1, d))
    c1, s1, a1 = random_tables(7, N, d)
    c2, s2, a2 = random_tables(8, N, d)
    twice = R.rope(R.rope(x, c1, s1), c2, s2)
    once = R.rope(x, np.cos(a1 + a2), np.sin(a1 + a2))
    assert np.allclose(twice, once, rtol=0, atol=1e-12)


def test_standard_tables_values():
    c, s = R.standard_tables(6, 8, base=10000.0)
    assert c.shape == (6, 4)
    assert np.array_equal(c[0], np.ones(4)) and np.array_equal(s[0], np.zeros(4))
    assert np.allclose(np.arctan2(s[:, 0], c[:, 0])[:4], np.arange(4.0))       # frequency base^0 = 1
    assert np.isclose(np.arctan2(s[1, 3], c[1, 3]), 10000.0 ** (-6 / 8))       # last pair: base^(-(d-2)/d)


def _scores_at(q, k, m, n, d, N=64):
    """q at position m, k at position n, standard tables: rope(q)·rope(k)."""
    c, s = R.standard_tables(N, d)
    X = np.zeros((1, N, 2, d))
    X[0, m, 0] = q
    X[0, n, 1] = k
    Y = R.rope(X, c, s)
    return float(Y[0, m, 0] @ Y[0, n, 1])


def test_relative_position_property():
    d = 64
    q, k = rng(9).standard_normal((2, d))
    for m, n in ((3, 1), (10, 7), (20, 20), (5, 30)):
        base = _scores_at(q, k, m, n, d)
        for t in (1, 9, 17):
            assert abs(_scores_at(q, k, m + t, n + t, d) - base) <= 1e-9 * max(1.0, abs(base))
    # and it does depend on the offset
    assert abs(_scores_at(q, k, 5, 1, d) - _scores_at(q, k, 5, 2, d)) > 1e-3


def test_planted_sign_error_breaks_relative_position():
    # r_i = x_i·cos + x_{i+d/2}·sin (wrong sign) is not a rotation: it fails the pins above
    def bad_rope(x, c, s):
        h = x.shape[-1] // 2
        a, b = x[..., :h], x[..., h:]
        return np.concatenate([a * c[None, :, None] + b * s[None, :, None], b * c[None, :, None] + a * s[None, :, None]], -1)
    d, N = 64, 40
    q, k = rng(10).standard_normal((2, d))
    c, s = R.standard_tables(N, d)

    def score(f, m, n):
        X = np.zeros((1, N, 2, d))
        X[0, m, 0], X[0, n, 1] = q, k
        Y = f(X, c, s)
        return float(Y[0, m, 0] @ Y[0, n, 1])
    assert abs(score(bad_rope, 12, 4) - score(bad_rope, 20, 12)) > 1e-3
    assert abs(score(R.rope, 12, 4) - score(R.rope, 20, 12)) < 1e-9


def test_hadamard_after_rope_keeps_scores():
    d, N = 128, 12
    c, s = R.standard_tables(N, d)
    q = R.rope(rng(11).standard_normal((1, N, 1, d)), c, s)
    k = R.rope(rng(12).standard_normal((1, N, 1, d)), c, s)
    signs = np.where(rng(13).random(d) < 0.5, -1.0, 1.0)
    sq = Hd.rotate(q, signs)[0, :, 0] @ Hd.rotate(k, signs)[0, :, 0].T
    assert np.allclose(sq, q[0, :, 0] @ k[0, :, 0].T, rtol=0, atol=1e-10)


def test_fused_quantiser_is_the_quantiser_of_the_embedded_rows():
    # the fused route decides on the same fp64 values as embedding first, then quantising
    d, N = 128, 130
    x = rng(16).standard_normal((1, N, 2, d)).astype(np.float32)
    c, s, _ = random_tables(17, N, d)
    c32, s32 = c.astype(np.float32), s.astype(np.float32)
    signs = np.where(rng(18).random(d) < 0.5, -1, 1).astype(np.int8)
    codes, scales = R.quantize_rope(x, c32, s32, signs)
    codes2, scales2 = quant.quantize(R.rope(x, c32, s32), signs)
    assert np.array_equal(codes, codes2) and np.array_equal(scales, scales2)
    np.testing.assert_array_equal(R.rope_rotate(x, c32, s32, signs), Hd.rotate(R.rope(x, c32, s32), signs))
    # a rotation by the wrong angle (sin negated) moves the codes
    codes3, _ = R.quantize_rope(x, c32, -s32, signs)
    assert (codes3 != codes).mean() > 0.5
