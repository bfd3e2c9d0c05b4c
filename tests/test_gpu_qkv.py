"""GPU parity of the fused QKV projection + 3D RoPE (nomas_qkv_projection with a
nomas_rope3d_table) against the fp64 oracle (oracle/qkv.py).

Bound per element: one bf16 rounding of the exact value (half an ulp) plus the
float32 accumulation over the hidden dimension, at most hidden * 2^-24 of
sum|x||w| for each of the (up to two, rotated) channels, plus float32 angle
error: |got - ref| <= ulp(ref) + 2^-12 * max over the pair of sum|x||w|."""

import numpy as np
import pytest
import torch

from oracle import formats, qkv
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _data(n, hidden, n_ch, seed):
    xb = synth.normal_bf16((n, 1, hidden), 95, seed, 0, 0)[:, 0]
    # weights ~ N(0, 1/hidden): unit-scale outputs
    w = np.random.default_rng(seed).standard_normal((n_ch, hidden)).astype(np.float32) / np.sqrt(hidden)
    wb = synth._round_bf16_bits(w)
    return xb, wb


def _run(H, D, hidden, F, gh, gw, T, t0, band, rows=None, seed=0):
    nv = F * gh * gw
    n = nv + T
    n_ch = 3 * H * D
    xb, wb = _data(n, hidden, n_ch, seed)
    say(f"qkv: H={H} D={D} hidden={hidden} rows={n} (video {nv})")
    table = nomas.nomas_rope3d_table(D, t0, F, gh, gw, band)
    y = nomas.nomas_qkv_projection(dev_bf16(xb), dev_bf16(wb), H, D, n_video=nv, rope_table=table)
    torch.cuda.synchronize()
    got = host_f64(y)
    x, w = synth.bf16_bits_to_f64(xb), synth.bf16_bits_to_f64(wb)
    sel = np.arange(n) if rows is None else np.asarray(rows)
    r = dict(t0=t0, n_frames=F, grid_h=gh, grid_w=gw, d_t=band[0], d_h=band[1], d_w=band[2])
    # the oracle on the selected rows: RoPE needs the rows' positions, so run it
    # on all video rows when any video row is selected
    q, k, v = qkv.qkv_projection(x, w, H, D, n_video=nv, rope=r)
    ref = np.concatenate([t.reshape(n, -1) for t in (q, k, v)], 1)[sel]
    mag = (np.abs(x) @ np.abs(w).T)[sel]
    pair = np.maximum(mag, mag.reshape(len(sel), -1, 2)[:, :, ::-1].reshape(len(sel), -1))
    tol = formats.bf16_ulp(ref) + 2.0 ** -12 * pair
    diff = np.abs(got[sel] - ref)
    assert np.all(diff <= tol), f"max excess {np.max(diff - tol):.3e} at {np.unravel_index(np.argmax(diff - tol), diff.shape)}"
    return diff, ref


def test_small_ragged():
    # 2 heads of 64, hidden 256, 2 frames of 4x6 + 17 text rows (row and channel tails)
    diff, ref = _run(2, 64, 256, 2, 4, 6, 17, 3, (16, 24, 24))
    assert np.mean(diff) < 2 ** -9 * np.mean(np.abs(ref)) + 1e-6


@pytest.mark.parametrize("H", [1, 3])
def test_odd_heads_key_value_boundary_inside_a_block(H):
    # head dim 64 with an odd head count: 2*H*64 is not a multiple of the
    # 256-channel block, so one block holds both key and value channels; only
    # the key channels may be rotated
    _run(H, 64, 128, 1, 4, 6, 9, 2, (16, 24, 24), seed=5 + H)


def test_mid_head128():
    # 4 heads of 128, hidden 512, 2 frames of 12x20 + 220 text rows
    _run(4, 128, 512, 2, 12, 20, 220, 18, (32, 48, 48), seed=1)


def test_full_shape_sampled_rows():
    # 16 x 128 heads, hidden 2,048, 8 frames of 24x40 + 256 text rows (7,936 rows)
    rng = np.random.default_rng(2)
    rows = np.unique(np.r_[0, 255, 256, 7679, 7680, 7935, rng.integers(0, 7936, 20)])
    _run(16, 128, 2048, 8, 24, 40, 256, 18, (32, 48, 48), rows=rows, seed=2)


def test_no_table_is_plain_projection():
    H, D, hidden, n = 2, 128, 128, 300
    xb, wb = _data(n, hidden, 3 * H * D, 3)
    y = nomas.nomas_qkv_projection(dev_bf16(xb), dev_bf16(wb), H, D)
    torch.cuda.synchronize()
    x, w = synth.bf16_bits_to_f64(xb), synth.bf16_bits_to_f64(wb)
    ref = formats.to_bf16(x @ w.T)
    tol = formats.bf16_ulp(ref) + 2.0 ** -12 * (np.abs(x) @ np.abs(w).T)
    assert np.all(np.abs(host_f64(y) - ref) <= tol)


def test_table_matches_rope_kernel():
    # the fused rotation and the in-place RoPE kernel use the same angles: rotating
    # with identity weights equals nomas_rope3d of x (bit for bit: both round once
    # from float32 with the same operations)
    H, D, F, gh, gw, T = 2, 128, 2, 4, 6, 8
    nv, n = F * gh * gw, F * gh * gw + T
    hidden = H * D
    xb = synth.normal_bf16((n, 1, hidden), 96, 0, 0, 0)[:, 0]
    wb = synth._round_bf16_bits(np.concatenate([np.eye(hidden, dtype=np.float32)] * 3, 0))
    table = nomas.nomas_rope3d_table(D, 5, F, gh, gw, (32, 48, 48))
    y = nomas.nomas_qkv_projection(dev_bf16(xb), dev_bf16(wb), H, D, n_video=nv, rope_table=table)
    q = dev_bf16(xb).view(n, H, D).clone()
    nomas.nomas_rope3d(q, None, 5, F, gh, gw, (32, 48, 48), H, D)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :hidden].reshape(n, H, D), q)
