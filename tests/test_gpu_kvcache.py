"""GPU parity of nomas_kvcache_append: bit-exact against the oracle's ring model
(oracle/ring.py) and quantiser (oracle/quant.py)."""

import numpy as np
import pytest
import torch

from oracle import quant
from oracle.ring import RingModel
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import cache_slots, dev_bf16, say

pytestmark = pytest.mark.gpu


def _check_cache(cache, ring, tpf, int8):
    k, v, ks, vs = cache_slots(cache)
    assert cache.frames_written == ring.frames_written
    assert cache.valid_frames == ring.valid_frames()
    for slot, (f, (kf, vf)) in ring.expected_slots().items():
        sl = slice(slot * tpf, (slot + 1) * tpf)
        if int8:
            qk, sk = quant.quantise(synth.bf16_bits_to_f64(kf))
            qv, sv = quant.quantise(synth.bf16_bits_to_f64(vf))
            assert np.array_equal(k[sl], qk), f"K codes differ in slot {slot} (frame {f})"
            assert np.array_equal(v[sl], qv), f"V codes differ in slot {slot} (frame {f})"
            assert np.array_equal(ks[sl].view(np.uint32), sk.view(np.uint32)), f"K scales differ in slot {slot}"
            assert np.array_equal(vs[sl].view(np.uint32), sv.view(np.uint32)), f"V scales differ in slot {slot}"
        else:
            assert np.array_equal(k[sl], kf) and np.array_equal(v[sl], vf), f"slot {slot} (frame {f})"


CASES = [
    # (grid_h, grid_w, capacity, heads, head_dim, append sizes, outliers)
    (4, 6, 4, 2, 64, [2, 2, 1, 3, 5, 9, 4], 0),          # tiny shape; wraps; n > capacity
    (2, 3, 3, 2, 128, [1, 2, 4, 1, 2], 0),               # tpf = 6: not a multiple of 4
    (3, 5, 5, 3, 64, [2, 7, 1, 3], 0),                   # odd tpf = 15
    (24, 40, 18, 16, 128, [8, 8, 8, 2, 8], 4),           # the layer shape, outlier K channels
]


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}cap{c[2]}h{c[3]}d{c[4]}")
def test_append_bit_exact_against_ring_model(case, int8):
    gh, gw, cap, H, D, sizes, n_out = case
    tpf = gh * gw
    say(f"append: grid {gh}x{gw} cap {cap} H {H} D {D} int8 {int8}")
    cache = nomas.KVCache(H, D, tpf, cap, int8)
    ring = RingModel(cap)
    wl_out = synth.Workload("t", 7, H, D, gh, gw, cap, 0, 1, 0, int8, (D // 4, 3 * D // 8, 3 * D // 8),
                            k_outliers=n_out)
    outl = synth.outlier_channels(wl_out)
    for step, n in enumerate(sizes):
        kb = synth.normal_bf16((n * tpf, H, D), 7, step, 0, 3, outliers=outl)
        vb = synth.normal_bf16((n * tpf, H, D), 7, step, 0, 4)
        cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), n)
        ring.append([(kb[f * tpf:(f + 1) * tpf], vb[f * tpf:(f + 1) * tpf]) for f in range(n)])
        _check_cache(cache, ring, tpf, int8)


def _crafted_frame(tpf, H, D, seed):
    """Vectors that stress the quantiser: zeros, x = m/2 ties, ties next to even
    codes (absmax 127: the scale is 1 and 2.5 -> 2, 62.5 -> 62), subnormal
    scales, huge values, a single non-zero, negative maxima."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tpf, H, D)).astype(np.float32)
    from_bits = synth.bf16_bits_to_f64
    for h in range(H):
        x[0, h] = 0.0
        # (0x3A8F: the float32 scale lies above m/127, so m/2 codes to 63, not 64)
        for t, mb in ((1, 0x3F96), (2, 0x3FB4), (3, 0x0081), (4, 0x7E80), (5, 0x3F80), (9, 0x3A8F)):
            m = np.float32(from_bits(np.array([mb], np.uint16))[0])
            x[t, h] = x[t, h] * (m / 8)
            x[t, h, 0] = m
            x[t, h, 1] = m / 2
            x[t, h, 2] = -m / 2
            x[t, h, 3] = m * np.float32(0.75)
        x[6, h] = 0.0
        x[6, h, 5] = -3.0
        x[7, h] = -np.abs(x[7, h])
        x[8, h] = 0.0
        x[8, h, :10] = [127.0, 0.5, 1.5, 2.5, 3.5, 62.5, 63.5, -0.5, -2.5, -62.5]
    return synth._round_bf16_bits(x)


@pytest.mark.parametrize("int8", [False, True])
def test_append_edge_vectors_bit_exact(int8):
    tpf, H, D, cap = 24, 2, 128, 2
    say(f"append edge vectors int8 {int8}")
    cache = nomas.KVCache(H, D, tpf, cap, int8)
    ring = RingModel(cap)
    for step in range(3):
        kb = _crafted_frame(tpf, H, D, 10 + step)
        vb = _crafted_frame(tpf, H, D, 20 + step)
        cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), 1)
        ring.append([(kb, vb)])
        _check_cache(cache, ring, tpf, int8)


def test_append_strided_input_and_untouched_padding():
    tpf, H, D, cap = 24, 2, 64, 4
    say("append strided input")
    cache = nomas.KVCache(H, D, tpf, cap, True)
    cache.k.fill_(0x55)
    ks_before = cache.k_scale.clone()
    ring = RingModel(cap)
    kb = synth.normal_bf16((2 * tpf, H, D), 8, 0, 0, 3)
    vb = synth.normal_bf16((2 * tpf, H, D), 8, 0, 0, 4)
    fused = torch.zeros((2 * tpf, 2 * H * D + 16), dtype=torch.bfloat16, device="cuda")
    fused[:, :H * D] = dev_bf16(kb).reshape(2 * tpf, H * D)
    fused[:, H * D + 8:2 * H * D + 8] = dev_bf16(vb).reshape(2 * tpf, H * D)
    cache.nomas_kvcache_append(fused[:, :H * D], fused[:, H * D + 8:2 * H * D + 8], 2)
    ring.append([(kb[f * tpf:(f + 1) * tpf], vb[f * tpf:(f + 1) * tpf]) for f in range(2)])
    _check_cache(cache, ring, tpf, True)
    # rows beyond the written slots keep their old bytes
    k, _, ks, _ = cache_slots(cache)
    assert np.all(k[2 * tpf:].view(np.uint8) == 0x55)
    before = ks_before.cpu().numpy().reshape(H, -1).T[2 * tpf:]
    assert np.array_equal(ks[2 * tpf:].view(np.uint32), before.view(np.uint32))
