"""Pins of oracle/rope.py: invariants, closed forms and special cases."""

import numpy as np

from oracle import rope


def _x(n, H, D, seed=0):
    return np.random.default_rng(seed).standard_normal((n, H, D))


def test_positions_match_explicit_loops():
    t0, F, gh, gw = 7, 3, 4, 6
    t, h, w = rope.video_positions(t0, F, gh, gw)
    i = 0
    for f in range(F):
        for r in range(gh):
            for c in range(gw):
                assert (t[i], h[i], w[i]) == (t0 + f, r, c)
                i += 1


def test_pair_norms_preserved():                      # P1
    x = _x(50, 3, 64)
    t, h, w = rope.video_positions(11, 2, 5, 5)
    y = rope.rope3d(x, t, h, w, 16, 24, 24)
    nx = np.hypot(x[..., 0::2], x[..., 1::2])
    ny = np.hypot(y[..., 0::2], y[..., 1::2])
    assert np.max(np.abs(nx - ny) / nx) < 1e-14


def test_inverse_by_negated_angle():                  # P2
    x = _x(96, 2, 128, 1)
    t, h, w = rope.video_positions(88, 1, 8, 12)
    y = rope.rope3d(x, t, h, w, 32, 48, 48)
    z = rope.rope3d(y, t, h, w, 32, 48, 48, sign=-1.0)
    assert np.max(np.abs(z - x)) < 1e-13


def test_zero_position_is_identity():                 # P3
    x = _x(4, 2, 64, 2)
    zero = np.zeros(4, np.int64)
    assert np.array_equal(rope.rope3d(x, zero, zero, zero, 16, 24, 24), x)


def test_one_axis_is_complex_multiplication():        # P3: 1-D RoFormer closed form
    # with d_h = d_w = 0 the map is z_j -> z_j * exp(i t theta^(-2j/D)) on the
    # complex numbers z_j = x[2j] + i x[2j+1]
    D = 64
    x = _x(10, 2, D, 3)
    t = np.arange(10) * 3 + 1
    y = rope.rope3d(x, t, np.zeros(10, int), np.zeros(10, int), D, 0, 0)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    j = np.arange(D // 2)
    rot = np.exp(1j * t[:, None] * 10000.0 ** (-2.0 * j / D))
    want = z * rot[:, None, :]
    assert np.max(np.abs(y[..., 0::2] - want.real)) < 1e-13
    assert np.max(np.abs(y[..., 1::2] - want.imag)) < 1e-13


def test_band_layout_unit_vectors():
    # a unit vector in channel off+2j comes out as (cos phi, sin phi) in
    # (off+2j, off+2j+1) with phi set by that band's axis only
    d_t, d_h, d_w = 16, 24, 24
    t, h, w = np.array([5]), np.array([3]), np.array([2])
    for off, width, pos in ((0, d_t, 5), (d_t, d_h, 3), (d_t + d_h, d_w, 2)):
        for j in range(width // 2):
            x = np.zeros((1, 1, 64))
            x[0, 0, off + 2 * j] = 1.0
            y = rope.rope3d(x, t, h, w, d_t, d_h, d_w)
            phi = pos * 10000.0 ** (-2.0 * j / width)
            want = np.zeros(64)
            want[off + 2 * j] = np.cos(phi)
            want[off + 2 * j + 1] = np.sin(phi)
            assert np.max(np.abs(y[0, 0] - want)) < 1e-15


def test_relative_shift_invariance():                 # P4
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for _ in range(20):
        p = rng.integers(0, 100, 3)
        pk = rng.integers(0, 100, 3)
        delta = rng.integers(-50, 50, 3)
        def dot(a, b):
            qa = rope.rope3d(q, *[np.array([c]) for c in a], 32, 48, 48)
            kb = rope.rope3d(k, *[np.array([c]) for c in b], 32, 48, 48)
            return float(np.sum(qa * kb))
        assert abs(dot(p + delta, pk + delta) - dot(p, pk)) < 1e-11
