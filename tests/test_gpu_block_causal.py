"""GPU parity of nomas_block_causal_attention (several segments in one call,
block-causal visibility inside the kernel) against the fp64 oracle's
whole-sequence block-causal attention (oracle/attention.py block_causal_full).
Same tolerance as the cached call: max|diff| <= 1e-2 * max|ref|, mean|diff| <=
1e-3; log-sum-exp within 2^-8."""

import math

import numpy as np
import pytest
import torch

from oracle import attention
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import Guarded, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu

LSE_TOL = 2.0 ** -8


def _inputs(segments, tpf, H, D, seed):
    """Seeded N(0,1) bf16 rows for each segment; returns (joint q, k, v bits,
    oracle segment dicts)."""
    qs, ks, vs, segs = [], [], [], []
    for i, (nv, nt, t0) in enumerate(segments):
        n = nv + nt
        q = synth.normal_bf16((n, H, D), 50 + seed, i, 0, 0)
        k = synth.normal_bf16((n, H, D), 50 + seed, i, 0, 1)
        v = synth.normal_bf16((n, H, D), 50 + seed, i, 0, 2)
        qs.append(q), ks.append(k), vs.append(v)
        segs.append(dict(q=synth.bf16_bits_to_f64(q), k=synth.bf16_bits_to_f64(k), v=synth.bf16_bits_to_f64(v),
                         t0=t0, n_frames=nv // tpf, tpf=tpf))
    return np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), segs


def _check(got, ref, what):
    diff = np.abs(got - ref)
    mx, mean, lim = diff.max(), diff.mean(), 1e-2 * np.abs(ref).max()
    assert mx <= lim and mean <= 1e-3, f"{what}: max|diff| {mx:.3e} (limit {lim:.3e}), mean {mean:.3e}"


def _run(segments, tpf, window, H, D, seed=0, rows=None):
    say(f"block causal: {len(segments)} segments tpf={tpf} window={window} H={H} D={D}")
    qb, kb, vb, segs = _inputs(segments, tpf, H, D, seed)
    n_rows = qb.shape[0]
    # out, lse and the workspace sit between sentinel bands, checked after the call
    g_out, g_lse = Guarded(2 * n_rows * H * D), Guarded(4 * H * n_rows)
    g_ws = Guarded(max(256, nomas.nomas_block_causal_attention_workspace_bytes(segments, tpf, H, D)))
    lse = g_lse.view(torch.float32, (H * n_rows,))
    out = nomas.nomas_block_causal_attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), segments, tpf,
                                             -1 if window is None else window, H, D,
                                             out=g_out.view(torch.bfloat16, (n_rows, H, D)), lse=lse,
                                             workspace=g_ws.view(torch.uint8, (g_ws.nbytes,)))
    for g, what in ((g_out, "block-causal out"), (g_lse, "block-causal lse"), (g_ws, "block-causal workspace")):
        g.check(what)
    torch.cuda.synchronize()
    got, g_lse = host_f64(out), lse.cpu().numpy().reshape(H, n_rows)
    ref, ref_lse = attention.block_causal_full(segs, window_frames=window, rows=rows, return_lse=True)
    r0 = 0
    for i, (nv, nt, _) in enumerate(segments):
        sel = np.arange(nv + nt) if rows is None or rows[i] is None else np.asarray(rows[i])
        _check(got[r0 + sel], ref[i], f"segment {i}")
        assert np.max(np.abs(g_lse[:, r0 + sel] - ref_lse[i])) <= LSE_TOL
        r0 += nv + nt
    return out


@pytest.mark.parametrize("window", [None, 4, 3, 0])
@pytest.mark.parametrize("D", [64, 128])
def test_session_all_rows(D, window):
    # 4 segments of 2 frames (4x6 grid) + 16 text rows, frames 0..7
    tpf = 24
    segments = [(2 * tpf, 16, 2 * s) for s in range(4)]
    _run(segments, tpf, window, 2, D, seed=D)


def test_ragged_segments():
    # unequal segments, a text-only one, one without text; rows not tile multiples
    tpf = 40
    segments = [(3 * tpf, 0, 0), (1 * tpf, 7, 3), (0, 5, 4), (4 * tpf, 33, 4), (2 * tpf, 1, 8)]
    for window in (None, 2, 5):
        _run(segments, tpf, window, 3, 128, seed=7)


def test_single_segment_is_plain_attention():
    # one segment: every row sees every row (the cached call with an empty cache)
    tpf = 24
    segments = [(3 * tpf, 20, 0)]
    _run(segments, tpf, None, 2, 128, seed=3)


def test_agrees_with_cached_calls():
    """Segment s's rows of one block-causal call equal the cached call of segment
    s against a bf16 ring cache of the window, built by appending the earlier
    segments' video K/V (GPU against GPU, to fp32 accumulation order)."""
    H, D, tpf, F, T, W = 2, 128, 48, 2, 16, 3
    segments = [(F * tpf, T, F * s) for s in range(4)]
    qb, kb, vb, _ = _inputs(segments, tpf, H, D, 11)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    say("block causal vs cached calls")
    full = host_f64(nomas.nomas_block_causal_attention(q, k, v, segments, tpf, W, H, D))
    cache = nomas.KVCache(H, D, tpf, W, False)
    r0 = 0
    for nv, nt, _ in segments:
        out = nomas.nomas_segment_attention(q[r0:r0 + nv + nt], k[r0:r0 + nv + nt], v[r0:r0 + nv + nt], nv, nt, cache)
        cache.nomas_kvcache_append(k[r0:r0 + nv], v[r0:r0 + nv], nv // tpf)
        torch.cuda.synchronize()
        ref = full[r0:r0 + nv + nt]
        assert np.max(np.abs(host_f64(out) - ref)) <= 2.0 ** -7 * max(1.0, np.abs(ref).max())
        r0 += nv + nt


def test_training_shape_sampled_rows():
    """3 segments of 8 frames on the 24x40 grid + 256 text rows each, 16x128
    heads, 18-frame window: 23,808 rows in one call; sampled rows vs the oracle."""
    H, D, tpf, F, T = 16, 128, 960, 8, 256
    segments = [(F * tpf, T, F * s) for s in range(3)]
    rng = np.random.default_rng(5)
    rows = [np.unique(np.r_[0, 255, 256, F * tpf - 1, F * tpf, F * tpf + T - 1, rng.integers(0, F * tpf + T, 10)])
            for _ in segments]
    _run(segments, tpf, 18, H, D, seed=1, rows=rows)


def test_repeatable():
    tpf = 24
    segments = [(2 * tpf, 16, 2 * s) for s in range(3)]
    qb, kb, vb, _ = _inputs(segments, tpf, 2, 128, 2)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    a = nomas.nomas_block_causal_attention(q, k, v, segments, tpf, 3, 2, 128)
    b = nomas.nomas_block_causal_attention(q, k, v, segments, tpf, 3, 2, 128)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
