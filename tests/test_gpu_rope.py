"""GPU parity of nomas_rope3d against the fp64 oracle (oracle/rope.py).

Bound: the kernel evaluates the angle pos*omega, its sine/cosine and the rotation
in float32 and rounds once to bf16; the oracle rotates exactly (fp64) and the
test rounds that to bf16. With E the float32 error of the rotated value,
|gpu - to_bf16(exact)| <= ulp(y) + E, where, for a pair of norm r and angle phi,
E <= r * (|phi| * 2^-22 + 2^-20) covers the rounding of omega (2^-24 rel.), of
the product pos*omega (2^-24 rel.), sincosf (a few ulp) and the two products of
the rotation. ulp(y) is the bf16 spacing at max(|gpu|, |ref|).
"""

import numpy as np
import pytest
import torch

from oracle import formats, rope
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _bound(x, ref_exact, got, pos_max):
    r = np.repeat(np.hypot(x[..., 0::2], x[..., 1::2]), 2, axis=-1)
    E = r * (pos_max * 2.0 ** -22 + 2.0 ** -20)
    ulp = formats.bf16_ulp(np.maximum(np.abs(got), np.abs(formats.to_bf16(ref_exact))))
    return ulp + E


@pytest.mark.parametrize("name", ["tiny", "layer_bf16", "long_bf16", "layer_880"])
def test_rope_matches_oracle(name):
    wl = synth.WORKLOADS[name]
    say(f"rope parity: {name}")
    q_bits, k_bits, _ = synth.current_qkv(wl)
    nv = wl.n_video
    q, k = dev_bf16(q_bits), dev_bf16(k_bits)
    nomas.nomas_rope3d(q, k, wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split, wl.n_heads, wl.head_dim)
    torch.cuda.synchronize()
    for bits, got in ((q_bits, host_f64(q)), (k_bits, host_f64(k))):
        x = synth.bf16_bits_to_f64(bits)
        assert np.array_equal(got[nv:], x[nv:])                  # text rows untouched
        ref = rope.rope3d_segment(x[:nv], wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, *wl.rope_split)
        err = np.abs(got[:nv] - formats.to_bf16(ref))
        bound = _bound(x[:nv], ref, got[:nv], wl.t0 + wl.seg_frames + max(wl.grid_h, wl.grid_w))
        assert np.all(err <= bound), (err.max(), np.argmax(err - bound))
        exact = np.mean(err == 0)
        assert exact > 0.99, exact
        # norm preservation of every pair, up to the two bf16 roundings
        nx = np.hypot(x[:nv, :, 0::2], x[:nv, :, 1::2])
        ng = np.hypot(got[:nv, :, 0::2], got[:nv, :, 1::2])
        assert np.all(np.abs(ng - nx) <= nx * 2.0 ** -7 + 1e-30)


@pytest.mark.parametrize("name", ["tiny", "layer_bf16"])
def test_rope_inverse_restores_input(name):
    wl = synth.WORKLOADS[name]
    say(f"rope inverse: {name}")
    q_bits, k_bits, _ = synth.current_qkv(wl)
    nv = wl.n_video
    q, k = dev_bf16(q_bits), dev_bf16(k_bits)
    args = (wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split, wl.n_heads, wl.head_dim)
    nomas.nomas_rope3d(q, k, *args)
    nomas.nomas_rope3d(q, k, *args, inverse=True)
    torch.cuda.synchronize()
    for bits, got in ((q_bits, host_f64(q)), (k_bits, host_f64(k))):
        x = synth.bf16_bits_to_f64(bits)[:nv]
        r = np.repeat(np.hypot(x[..., 0::2], x[..., 1::2]), 2, axis=-1)
        # two rotations, each within ulp + E of exact, and exact rotations compose to identity
        bound = 2 * (formats.bf16_ulp(np.maximum(np.abs(got[:nv]), np.abs(x))) +
                     r * ((wl.t0 + wl.seg_frames + 40) * 2.0 ** -22 + 2.0 ** -20)) + r * 2.0 ** -7
        assert np.all(np.abs(got[:nv] - x) <= bound)


def test_rope_strided_views_and_q_only():
    wl = synth.WORKLOADS["tiny"]
    say("rope strided views")
    q_bits, k_bits, _ = synth.current_qkv(wl)
    H, D = wl.n_heads, wl.head_dim
    args = (wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split, H, D)
    q, k = dev_bf16(q_bits), dev_bf16(k_bits)
    nomas.nomas_rope3d(q, k, *args)
    # the same rows as views of one fused [rows, 3*H*D + 8] buffer
    fused = torch.zeros((wl.n_q, 3 * H * D + 8), dtype=torch.bfloat16, device="cuda")
    fused[:, :H * D] = dev_bf16(q_bits).reshape(wl.n_q, H * D)
    fused[:, H * D:2 * H * D] = dev_bf16(k_bits).reshape(wl.n_q, H * D)
    sentinel = fused[:, 2 * H * D:].clone()
    nomas.nomas_rope3d(fused[:, :H * D], fused[:, H * D:2 * H * D], *args)
    q_only = dev_bf16(q_bits)
    nomas.nomas_rope3d(q_only, None, *args)
    torch.cuda.synchronize()
    assert torch.equal(fused[:, :H * D].reshape(q.shape), q)
    assert torch.equal(fused[:, H * D:2 * H * D].reshape(k.shape), k)
    assert torch.equal(fused[:, 2 * H * D:], sentinel)
    assert torch.equal(q_only, q)


def test_rope_is_deterministic():
    wl = synth.WORKLOADS["layer_bf16"]
    say("rope determinism")
    q_bits, k_bits, _ = synth.current_qkv(wl)
    outs = []
    for _ in range(2):
        q, k = dev_bf16(q_bits), dev_bf16(k_bits)
        nomas.nomas_rope3d(q, k, wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split, wl.n_heads,
                           wl.head_dim)
        outs.append((q, k))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
