"""GPU parity of nomas_segment_attention_frames: attention against a chosen range
of the retained frames (the range may wrap round the ring), and the segment's
values given transposed.

The reference is the oracle's segment attention (oracle/attention.py) over the
frames of that range as the ring model (oracle/ring.py) holds them, dequantised
by oracle/quant.py for INT8; tolerance as for every attention path
(max|diff| <= 1e-2 * max|ref|, mean|diff| <= 1e-3, every row of every head).
With all retained frames the call must reproduce nomas_segment_attention bit for
bit, and a V^T input must give the same bits as the row-major values."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, quant
from oracle.ring import RingModel
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import Guarded, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _filled(H, D, tpf, cap, n_frames, int8, seed):
    """A cache of capacity ``cap`` after appends of n_frames frames in chunks of
    3 (wrapping when n_frames > cap), and its ring model with the frames as the
    cache holds them (dequantised for INT8)."""
    cache = nomas.KVCache(H, D, tpf, cap, int8)
    ring = RingModel(cap)
    k = synth.normal_bf16((n_frames * tpf, H, D), 71, seed, 0, 1)
    v = synth.normal_bf16((n_frames * tpf, H, D), 71, seed, 0, 2)
    f = 0
    while f < n_frames:
        n = min(3, n_frames - f)
        sl = slice(f * tpf, (f + n) * tpf)
        cache.nomas_kvcache_append(dev_bf16(k[sl]), dev_bf16(v[sl]), n)
        fr = []
        for i in range(f, f + n):
            kf = synth.bf16_bits_to_f64(k[i * tpf:(i + 1) * tpf])
            vf = synth.bf16_bits_to_f64(v[i * tpf:(i + 1) * tpf])
            if int8:
                kf, vf = quant.dequantise(*quant.quantise(kf)), quant.dequantise(*quant.quantise(vf))
            fr.append((kf, vf))
        ring.append(fr)
        f += n
    return cache, ring


def _window(ring, first, n):
    frames = [p for f, p in ring.retained() if first <= f < first + n]
    assert len(frames) == n
    if not frames:
        return None, None
    return np.concatenate([p[0] for p in frames], 0), np.concatenate([p[1] for p in frames], 0)


def _vt_of(v, n_q, H, D, pad):
    """V^T [H*D][ld_vt] of rows [0, n_q) of v [n, H, D], NaN in the pad columns
    (values past n_q must never reach the result)."""
    ld = (n_q + 127) // 128 * 128 + pad
    vt = torch.full((H * D, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    vt[:, :n_q] = v[:n_q].reshape(n_q, H * D).t()
    return vt


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_frame_ranges_match_oracle(D, int8, splits):
    """Capacity 5 after 8 frames (retained [3, 8) in slots 3, 4, 0, 1, 2): ranges
    that wrap, that do not, single frames and the empty range; 40 tokens per
    frame, so every run ends in a partial key tile."""
    H, tpf, cap = 2, 40, 5
    cache, ring = _filled(H, D, tpf, cap, 8, int8, seed=D + int8)
    assert cache.frames_written == 8
    nv, nt = 2 * tpf, 19
    n_q = nv + nt
    qb = synth.normal_bf16((n_q, H, D), 72, D, 0, 0)
    kb = synth.normal_bf16((n_q, H, D), 72, D, 0, 1)
    vb = synth.normal_bf16((n_q, H, D), 72, D, 0, 2)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    x = [synth.bf16_bits_to_f64(t) for t in (qb, kb, vb)]
    scale = 1.0 / math.sqrt(D)
    vt = _vt_of(v, n_q, H, D, pad=24)
    for first, n in [(3, 5), (3, 3), (4, 2), (4, 4), (5, 3), (7, 1), (3, 1), (6, 0)]:
        say(f"frames: D={D} int8={int8} splits={splits} range [{first}, {first + n})")
        g_out = Guarded(2 * n_q * H * D)
        g_lse = Guarded(4 * H * n_q)
        out = nomas.nomas_segment_attention_frames(q, k, v, nv, nt, cache, first, n,
                                                   out=g_out.view(torch.bfloat16, (n_q, H, D)),
                                                   lse=g_lse.view(torch.float32, (H * n_q,)), n_splits=splits)
        lse = g_lse.view(torch.float32, (H * n_q,))
        out_t = nomas.nomas_segment_attention_frames(q, k, None, nv, nt, cache, first, n, v_t=vt, n_splits=splits)
        g_out.check("frames out")
        g_lse.check("frames lse")
        torch.cuda.synchronize()
        assert torch.equal(out, out_t), f"[{first}, {first + n}): V^T input changed the result"
        kp, vp = _window(ring, first, n)
        ref, ref_lse = attention.segment_attention(x[0], x[1], x[2], kp, vp, scale)
        got = host_f64(out)
        diff = np.abs(got - ref)
        assert diff.max() <= 1e-2 * np.abs(ref).max() and diff.mean() <= 1e-3, \
            f"[{first}, {first + n}): max|diff| {diff.max():.3e}, mean {diff.mean():.3e}"
        assert np.max(np.abs(lse.cpu().numpy().reshape(H, n_q) - ref_lse)) <= 2.0 ** -8
        if n == 5:
            plain = nomas.nomas_segment_attention(q, k, v, nv, nt, cache, n_splits=splits)
            torch.cuda.synchronize()
            assert torch.equal(out, plain), "all retained frames: differs from nomas_segment_attention"
    assert cache.frames_written == 8


@pytest.mark.parametrize("int8", [False, True])
def test_layer_shape_window_before_segment(int8):
    """The final-step use at the layer shape: a cache of 18 + 8 frames holding 26
    (the newest 8 being the segment), attention to the 18 before them (a range
    that wraps), current values as V^T; every row of every head against the
    oracle over the ring model's frames."""
    H, D, tpf, W, F, nt = 16, 128, 960, 18, 8, 256
    cache, ring = _filled(H, D, tpf, W + F, W + F + 10, int8, seed=5)
    fw = cache.frames_written
    first = fw - F - W
    assert (first % (W + F)) + W > W + F, "the range must wrap round the ring"
    nv = F * tpf
    n_q = nv + nt
    qb = synth.normal_bf16((n_q, H, D), 73, 0, 0, 0)
    kb = synth.normal_bf16((n_q, H, D), 73, 0, 0, 1)
    vb = synth.normal_bf16((n_q, H, D), 73, 0, 0, 2)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    vt = _vt_of(v, n_q, H, D, pad=128)
    say(f"frames: layer shape int8={int8} range [{first}, {first + W})")
    out = nomas.nomas_segment_attention_frames(q, k, None, nv, nt, cache, first, W, v_t=vt)
    torch.cuda.synchronize()
    kp, vp = _window(ring, first, W)
    x = [synth.bf16_bits_to_f64(t) for t in (qb, kb, vb)]
    say("frames: oracle on every row")
    ref, _ = attention.segment_attention(x[0], x[1], x[2], kp, vp, 1.0 / math.sqrt(D))
    diff = np.abs(host_f64(out) - ref)
    assert diff.max() <= 1e-2 * np.abs(ref).max() and diff.mean() <= 1e-3, (diff.max(), diff.mean())
