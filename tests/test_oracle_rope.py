"""Pins of the rotary embedding of the oracle (``oracle.fp8.rope``).

* position 0 is the identity; each (i, i + d/2) pair keeps its length;
* d = 2 is the plane rotation by t radians (closed form, written out here);
* the relative-position property: q at position t1 against k at position t2
  gives the same dot product as at t1 + s, t2 + s (float64 tables of the
  definition);
* composition: turning by the tables of t1 then t2 equals the tables of t1 + t2
  (angle addition);
* prepare with RoPE equals RoPE'd inputs through prepare without it.
"""
import numpy as np

from oracle import fp8 as F


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_position_zero_is_identity_and_pairs_keep_length():
    x = _rand((2, 9, 16), 1)
    c, s = F.rope_tables(9, 16)
    y = F.rope(x, c, s)
    np.testing.assert_allclose(y[:, 0], x[:, 0], rtol=0, atol=0)
    n0 = x[..., :8] ** 2 + x[..., 8:] ** 2
    n1 = y[..., :8] ** 2 + y[..., 8:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13, atol=1e-13)


def test_d2_is_plane_rotation_by_t_radians():
    x = _rand((5, 2), 2)
    c, s = F.rope_tables(5, 2)      # base^0 = 1: angle t
    y = F.rope(x, c, s)
    for t in range(5):
        a, b = x[t]
        np.testing.assert_allclose(y[t], [a * np.cos(t) - b * np.sin(t), a * np.sin(t) + b * np.cos(t)],
                                   rtol=0, atol=1e-15)


def test_scores_depend_on_relative_position_only():
    d, N = 32, 40
    c, s = F.rope_tables(N, d)
    q, k = _rand(d, 3), _rand(d, 4)
    Q = F.rope(np.tile(q, (N, 1)), c, s)
    K = F.rope(np.tile(k, (N, 1)), c, s)
    for t1, t2, sh in ((3, 7, 10), (20, 2, 15), (5, 5, 30)):
        assert abs(Q[t1] @ K[t2] - Q[t1 + sh] @ K[t2 + sh]) < 1e-11


def test_angle_addition():
    d = 8
    c, s = F.rope_tables(12, d)
    x = _rand((1, d), 5)
    for t1, t2 in ((2, 3), (4, 7)):
        once = F.rope(F.rope(x, c[t1:t1 + 1], s[t1:t1 + 1]), c[t2:t2 + 1], s[t2:t2 + 1])
        np.testing.assert_allclose(once, F.rope(x, c[t1 + t2:t1 + t2 + 1], s[t1 + t2:t1 + t2 + 1]),
                                   rtol=0, atol=1e-13)


def test_prepare_with_rope_equals_roped_inputs():
    q, k, v = _rand((1, 2, 130, 128), 6), _rand((1, 1, 130, 128), 7), _rand((1, 1, 130, 128), 8)
    signs = np.where(_rand(128, 9) < 0, -1, 1)
    c, s = F.rope_tables(130, 128)
    a = F.prepare(q, k, v, signs, rope_cos=c, rope_sin=s)
    b = F.prepare(F.rope(q, c, s), F.rope(k, c, s), v, signs)
    for n in ("q", "k", "v"):
        np.testing.assert_array_equal(a[n][0], b[n][0])
        np.testing.assert_array_equal(a[n][1], b[n][1])
