"""Pins of the QKV-projection oracle (oracle/qkv.py)."""

import numpy as np

from oracle import formats, qkv, rope


def _bf(shape, seed, scale=1.0):
    return formats.to_bf16(scale * np.random.default_rng(seed).standard_normal(shape))


def test_brute_force_projection():
    # the matrix product against explicit sums over the hidden dimension
    x, w = _bf((5, 24), 1), _bf((3 * 2 * 4, 24), 2)
    q, k, v = qkv.qkv_projection(x, w, 2, 4)
    y = np.concatenate([t.reshape(5, -1) for t in (q, k, v)], 1)
    for i in range(5):
        for c in range(24):
            assert y[i, c] == formats.to_bf16(sum(x[i, j] * w[c, j] for j in range(24)))


def test_identity_weights_give_rope_of_the_input():
    # W = [I; I; I] (hidden = H*D): q = k = RoPE(x) on video rows, v = x
    H, D, gh, gw, F = 2, 64, 2, 3, 2
    n = F * gh * gw + 4
    x = _bf((n, H * D), 3)
    w = np.concatenate([np.eye(H * D)] * 3, 0)
    r = dict(t0=5, n_frames=F, grid_h=gh, grid_w=gw, d_t=16, d_h=24, d_w=24)
    q, k, v = qkv.qkv_projection(x, w, H, D, n_video=F * gh * gw, rope=r)
    xr = x.reshape(n, H, D)
    want = formats.to_bf16(rope.rope3d_segment(xr[:F * gh * gw], 5, F, gh, gw, 16, 24, 24))
    assert np.array_equal(q[:F * gh * gw], want) and np.array_equal(k[:F * gh * gw], want)
    assert np.array_equal(q[F * gh * gw:], xr[F * gh * gw:]) and np.array_equal(v, xr)


def test_rotation_preserves_pair_norms_and_values_are_unrotated():
    H, D, gh, gw, F = 2, 128, 3, 4, 2
    nv = F * gh * gw
    x, w = _bf((nv + 3, 256), 4), _bf((3 * H * D, 256), 5, 0.06)
    r = dict(t0=7, n_frames=F, grid_h=gh, grid_w=gw, d_t=32, d_h=48, d_w=48)
    q, k, v = qkv.qkv_projection(x, w, H, D, n_video=nv, rope=r)
    q0, k0, v0 = qkv.qkv_projection(x, w, H, D)
    assert np.array_equal(v, v0) and np.array_equal(q[nv:], q0[nv:])
    pn = lambda t: np.sqrt(t[..., 0::2] ** 2 + t[..., 1::2] ** 2)
    assert np.max(np.abs(pn(q[:nv]) - pn(q0[:nv])) / (pn(q0[:nv]) + 1e-3)) < 2 ** -6


def test_one_rounding_after_the_rotation():
    # the rotated video-row q, k lie within half a bf16 ulp of the rotation of
    # the exact product: the product is rounded once, after RoPE (a rounding
    # before the rotation as well can land a full ulp away)
    H, D, gh, gw, F = 1, 64, 4, 4, 2
    nv = F * gh * gw
    x, w = _bf((nv, 48), 6), _bf((3 * H * D, 48), 7, 0.15)
    r = dict(t0=3, n_frames=F, grid_h=gh, grid_w=gw, d_t=16, d_h=24, d_w=24)
    q, k, _ = qkv.qkv_projection(x, w, H, D, n_video=nv, rope=r)
    y = x @ w.T
    for got, blk in ((q, 0), (k, 1)):
        exact = rope.rope3d_segment(y[:, blk * H * D:(blk + 1) * H * D].reshape(nv, H, D), 3, F, gh, gw, 16, 24, 24)
        assert np.all(np.abs(got - exact) <= 0.5 * formats.bf16_ulp(got) * (1 + 1e-12))
