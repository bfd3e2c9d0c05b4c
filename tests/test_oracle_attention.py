"""Pins of oracle/attention.py: invariants, closed forms, brute force, and the
equality of the cached formulation with full-sequence block-causal attention."""

import math

import numpy as np
import pytest

from oracle import attention, formats, quant, rope
from oracle.ring import RingModel
from segment_autoregressive_dit_amd import synth


def _rand(shape, seed):
    return formats.to_bf16(np.random.default_rng(seed).standard_normal(shape))


def test_probability_rows_sum_to_one():               # A1
    q, k, v = _rand((40, 2, 64), 0), _rand((70, 2, 64), 1), _rand((70, 2, 64), 2)
    _, _, probs = attention.segment_attention(q, k, v, scale=0.3, return_probs=True)
    for p in probs:
        assert np.max(np.abs(p.sum(1) - 1.0)) < 1e-12
        assert np.all(p >= 0)


def test_ones_values_give_ones():                     # A1 through the values
    q, k = _rand((33, 2, 64), 3), _rand((50, 2, 64), 4)
    kp = _rand((24, 2, 64), 5)
    out, _ = attention.segment_attention(q, k, np.ones_like(k), kp, np.ones_like(kp), 0.125)
    assert np.max(np.abs(out - 1.0)) < 1e-13


def test_constant_keys_give_mean_and_frame_histogram():   # A2
    H, D, tpf = 2, 64, 24
    cap = 3
    ring = RingModel(cap)
    # six frames appended; value of a key = one-hot of (frame mod D)
    for f in range(6):
        v = np.zeros((tpf, H, D))
        v[:, :, f % D] = 1.0
        ring.append([v])
    past = ring.retained()
    v_past = np.concatenate([p for _, p in past], 0)
    k_past = np.full_like(v_past, 0.5)
    n_cur = 30
    v_cur = np.zeros((n_cur, H, D))
    v_cur[:, :, 63] = 1.0
    k_cur = np.full((n_cur, H, D), 0.5)
    q = _rand((n_cur, H, D), 6)
    out, _ = attention.segment_attention(q, k_cur, v_cur, k_past, v_past, 0.1)
    n_k = len(v_past) + n_cur
    want = np.zeros(D)
    for f in range(6 - cap, 6):
        want[f] = tpf / n_k
    want[63] = n_cur / n_k
    assert np.max(np.abs(out - want[None, None, :])) < 1e-13


def test_single_key_and_dominant_logit():             # A3
    q, k, v = _rand((5, 1, 64), 7), _rand((1, 1, 64), 8), _rand((1, 1, 64), 9)
    out, lse = attention.segment_attention(q, k, v, scale=0.2)
    assert np.max(np.abs(out - v[0][None])) < 1e-15
    assert np.allclose(lse[0], 0.2 * (q[:, 0] @ k[0, 0]))
    k2 = np.zeros((10, 1, 64))
    k2[3, 0, :] = 50.0
    q2 = np.ones((2, 1, 64))
    v2 = _rand((10, 1, 64), 10)
    out2, _ = attention.segment_attention(q2, k2, v2, scale=1.0)
    assert np.max(np.abs(out2 - v2[3][None])) < 1e-12


def test_key_permutation_invariance():                # A4
    q, k, v = _rand((30, 2, 64), 11), _rand((90, 2, 64), 12), _rand((90, 2, 64), 13)
    perm = np.random.default_rng(0).permutation(90)
    a, la = attention.segment_attention(q, k[:20], v[:20], k[20:], v[20:], 0.125)
    b, lb = attention.segment_attention(q, k[perm][:20], v[perm][:20], k[perm][20:], v[perm][20:], 0.125)
    assert np.max(np.abs(a - b)) < 1e-13 and np.max(np.abs(la - lb)) < 1e-12


def test_brute_force_tiny():                          # A6
    q, k, v = _rand((6, 2, 8), 14), _rand((11, 2, 8), 15), _rand((11, 2, 8), 16)
    a, la = attention.segment_attention(q, k[:5], v[:5], k[5:], v[5:], 0.35)
    kk = np.concatenate([k[5:], k[:5]], 0)
    vv = np.concatenate([v[5:], v[:5]], 0)
    b, lb = attention.brute_force_attention(q.tolist(), kk.tolist(), vv.tolist(), 0.35)
    assert np.max(np.abs(a - b)) < 1e-12 and np.max(np.abs(la - lb)) < 1e-12


def test_brute_force_tiny_workload_rows():            # A6 at the tiny workload's sizes
    wl = synth.WORKLOADS["tiny"]
    q, k, v = (synth.bf16_bits_to_f64(t) for t in synth.current_qkv(wl))
    kp, vp = (synth.bf16_bits_to_f64(t) for t in synth.prefill_kv(wl))
    scale = 1.0 / math.sqrt(wl.head_dim)
    a, la = attention.segment_attention(q, k, v, kp, vp, scale)
    rows = [0, 17, 47, 48, 63]                    # video, frame edge, first/last text
    kk = np.concatenate([kp, k], 0)
    vv = np.concatenate([vp, v], 0)
    b, lb = attention.brute_force_attention(q[rows].tolist(), kk.tolist(), vv.tolist(), scale)
    assert np.max(np.abs(a[rows] - b)) < 1e-12
    assert np.max(np.abs(la[:, rows] - lb)) < 1e-12


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 64])
def test_split_merge_equals_unsplit(n_splits):        # A7
    q, k, v = _rand((40, 2, 64), 17), _rand((200, 2, 64), 18), _rand((200, 2, 64), 19)
    a, la = attention.segment_attention(q, k, v, scale=0.125)
    b, lb = attention.split_attention(q, k, v, n_splits, 0.125)
    assert np.max(np.abs(a - b)) < 1e-13 and np.max(np.abs(la - lb)) < 1e-12


def test_rows_helper_matches_full():
    q, k, v = _rand((20, 2, 64), 20), _rand((45, 2, 64), 21), _rand((45, 2, 64), 22)
    a, la = attention.segment_attention(q, k, v, scale=0.125)
    rows = np.array([0, 5, 19, 7])
    heads = np.array([0, 1, 1, 0])
    o, l = attention.segment_attention_rows(q[rows, heads], heads, k, v, 0.125)
    assert np.max(np.abs(o - a[rows, heads])) < 1e-14
    assert np.max(np.abs(l - la[heads, rows])) < 1e-12


def _session(int8, window, n_segments=4, F=2, gh=4, gw=6, T=16, H=2, D=64):
    """Build a session of segments with RoPE at absolute frames; return both the
    per-segment cached outputs (ring model) and the full block-causal outputs."""
    tpf = gh * gw
    cap = window if window is not None else n_segments * F
    ring = RingModel(cap)
    segs, cached_out = [], []
    for s in range(n_segments):
        rng = np.random.default_rng(100 + s)
        n = F * tpf + T
        q = formats.to_bf16(rng.standard_normal((n, H, D)))
        k = formats.to_bf16(rng.standard_normal((n, H, D)))
        v = formats.to_bf16(rng.standard_normal((n, H, D)))
        t0 = s * F
        nv = F * tpf
        q[:nv] = formats.to_bf16(rope.rope3d_segment(q[:nv], t0, F, gh, gw, 16, 24, 24))
        k[:nv] = formats.to_bf16(rope.rope3d_segment(k[:nv], t0, F, gh, gw, 16, 24, 24))
        if int8:
            qk, sk = quant.quantise(k[:nv])
            qv, sv = quant.quantise(v[:nv])
            kp, vp = quant.dequantise(qk, sk), quant.dequantise(qv, sv)
        else:
            kp, vp = k[:nv], v[:nv]
        past = ring.retained()
        k_past = np.concatenate([p[0] for _, p in past], 0) if past else None
        v_past = np.concatenate([p[1] for _, p in past], 0) if past else None
        out, lse = attention.segment_attention(q, k, v, k_past, v_past, 1 / math.sqrt(D))
        cached_out.append((out, lse))
        ring.append([(kp[f * tpf:(f + 1) * tpf], vp[f * tpf:(f + 1) * tpf]) for f in range(F)])
        segs.append(dict(q=q, k=k, v=v, k_past=kp, v_past=vp, t0=t0, n_frames=F, tpf=tpf))
    full, full_lse = attention.block_causal_full(segs, window_frames=window, return_lse=True)
    return cached_out, (full, full_lse), segs


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("window", [None, 4, 3])
def test_cached_equals_full_block_causal(int8, window):   # A5
    cached, (full, full_lse), _ = _session(int8, window)
    for (a, la), b, lb in zip(cached, full, full_lse):
        assert np.max(np.abs(a - b)) < 1e-12
        assert np.max(np.abs(la - lb)) < 1e-12


def test_block_causal_row_subset():
    # computing selected query rows only gives those rows of the full result (to
    # BLAS blocking order)
    _, (full, full_lse), segs = _session(False, 3)
    rows = [np.array([0, 7, 63]), None, np.array([5]), np.array([63, 1, 48])]
    sub, sub_lse = attention.block_causal_full(segs, window_frames=3, rows=rows, return_lse=True)
    for r, a, la, b, lb in zip(rows, full, full_lse, sub, sub_lse):
        r = np.arange(a.shape[0]) if r is None else r
        assert np.max(np.abs(a[r] - b)) < 1e-14 and np.max(np.abs(la[:, r] - lb)) < 1e-13


def test_window_changes_result():
    # guard against a mask that ignores the window: W=3 must differ from W=None
    a, _, _ = _session(False, None)
    b, _, _ = _session(False, 3)
    assert np.max(np.abs(a[-1][0] - b[-1][0])) > 1e-3
