"""GPU checks of the evicted-frame archive (copy-engine D2H / H2D of ring
slots): archived records are byte-identical to the frames the ring model says
left the window, quantised by the oracle (O3/O4); restored records rebuild a
cache byte-for-byte."""

import numpy as np
import pytest
import torch

from oracle import quant
from oracle.ring import RingModel
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import cache_slots, dev_bf16, say

pytestmark = pytest.mark.gpu


def _record(k_bits, v_bits, int8):
    """Expected record of one frame from its bf16 K/V rows [tpf, H, D]: K
    [H][tpf][D], V^T [H][D][tpf], then (INT8) key and value scales [H][tpf]."""
    if int8:
        qk, sk = quant.quantise(synth.bf16_bits_to_f64(k_bits))
        qv, sv = quant.quantise(synth.bf16_bits_to_f64(v_bits))
        parts = [qk.transpose(1, 0, 2), qv.transpose(1, 2, 0), sk.T.astype(np.float32), sv.T.astype(np.float32)]
    else:
        parts = [k_bits.transpose(1, 0, 2), v_bits.transpose(1, 2, 0)]
    return b"".join(np.ascontiguousarray(p).tobytes() for p in parts)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("int8", [False, True])
def test_archive_matches_evicted_frames(int8, D):
    H, tpf, cap, F = 2, 24, 3, 2
    cache = nomas.KVCache(H, D, tpf, cap, int8)
    ring = RingModel(cap)
    rec = cache.nomas_kvcache_record_bytes()
    assert rec == (H * tpf * D * 2 * (1 if int8 else 2)) + (2 * H * tpf * 4 if int8 else 0)
    say(f"archive: int8={int8} D={D}")
    archived = []
    for s in range(5):
        kb = synth.normal_bf16((F * tpf, H, D), 90, s, 0, 1)
        vb = synth.normal_bf16((F * tpf, H, D), 90, s, 0, 2)
        host = cache.host_records(F)
        n_before = len(ring.evicted)
        n_ev = cache.nomas_kvcache_append_archive(dev_bf16(kb), dev_bf16(vb), F, host)
        ring.append([(kb[f * tpf:(f + 1) * tpf], vb[f * tpf:(f + 1) * tpf]) for f in range(F)])
        assert n_ev == len(ring.evicted) - n_before
        torch.cuda.synchronize()
        raw = host.numpy().tobytes()
        archived += [raw[i * rec:(i + 1) * rec] for i in range(n_ev)]
    assert cache.frames_written == ring.frames_written
    assert len(archived) == len(ring.evicted) == 10 - cap
    for got, (f, (kb, vb)) in zip(archived, ring.evicted):
        assert got == _record(kb, vb, int8), f"archived frame {f}"
    # the retained frames export the same way
    host = cache.host_records(cap)
    cache.nomas_kvcache_export_frames(ring.frames_written - cap, cap, host)
    torch.cuda.synchronize()
    raw = host.numpy().tobytes()
    for i, (f, (kb, vb)) in enumerate(ring.retained()):
        assert raw[i * rec:(i + 1) * rec] == _record(kb, vb, int8), f"exported frame {f}"


@pytest.mark.parametrize("int8", [False, True])
def test_restore_rebuilds_the_cache(int8):
    """Records of 5 frames restored into a fresh 4-frame cache equal, slot by
    slot, a cache that appended the same frames directly."""
    H, D, tpf = 2, 128, 40
    kb = synth.normal_bf16((5 * tpf, H, D), 91, 0, 0, 1)
    vb = synth.normal_bf16((5 * tpf, H, D), 91, 0, 0, 2)
    src = nomas.KVCache(H, D, tpf, 5, int8)
    src.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), 5)
    host = src.host_records(5)
    src.nomas_kvcache_export_frames(0, 5, host)
    torch.cuda.synchronize()
    say(f"restore: int8={int8}")
    a = nomas.KVCache(H, D, tpf, 4, int8)
    rec = a.nomas_kvcache_record_bytes()
    a.nomas_kvcache_restore_frames(host[:3 * rec], 3)
    a.nomas_kvcache_restore_frames(host[3 * rec:], 2)
    b = nomas.KVCache(H, D, tpf, 4, int8)
    b.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), 5)
    torch.cuda.synchronize()
    assert a.frames_written == b.frames_written == 5
    n = a.valid_frames * tpf
    for x, y in zip(cache_slots(a), cache_slots(b)):
        if x is not None:
            assert np.array_equal(x[:n], y[:n])


def _session_step(cache, s, H, D, gh, gw, F, T):
    """Segment s of a seeded session: RoPE of its Q/K video rows, attention
    against the cache, then the append of its K/V; returns the attention output."""
    tpf = gh * gw
    nv, n = F * tpf, F * tpf + T
    q, k, v = (dev_bf16(synth.normal_bf16((n, H, D), 92, s, 0, t)) for t in range(3))
    nomas.nomas_rope3d(q, k, F * s, F, gh, gw, (D // 4, 3 * D // 8, 3 * D // 8), H, D)
    out = nomas.nomas_segment_attention(q, k, v, nv, T, cache)
    cache.nomas_kvcache_append(k[:nv], v[:nv], F)
    return out


@pytest.mark.parametrize("int8", [False, True])
def test_resume_from_archive_is_bitwise_the_uninterrupted_session(int8):
    """Checkpoint / resume: after segment 2 of a 6-segment session the retained
    frames go to pinned host memory as records and the cache is dropped; a fresh
    cache whose frames_written is set to the snapshot's count minus the retained
    frames takes the records back (each lands in its original slot) and the
    session continues. Every later attention output and the final cache bytes
    equal the uninterrupted session's bit for bit."""
    H, D, gh, gw, F, T, W = 2, 128, 4, 10, 2, 24, 5
    tpf = gh * gw
    ref = nomas.KVCache(H, D, tpf, W, int8)
    outs_ref = [_session_step(ref, s, H, D, gh, gw, F, T) for s in range(6)]
    torch.cuda.synchronize()
    say(f"resume: int8={int8}")
    a = nomas.KVCache(H, D, tpf, W, int8)
    for s in range(3):
        _session_step(a, s, H, D, gh, gw, F, T)
    fw, valid = a.frames_written, a.valid_frames
    host = a.host_records(valid)
    a.nomas_kvcache_export_frames(fw - valid, valid, host)
    torch.cuda.synchronize()
    del a
    b = nomas.KVCache(H, D, tpf, W, int8)
    b.desc.frames_written = fw - valid
    b.nomas_kvcache_restore_frames(host, valid)
    assert b.frames_written == fw
    outs = [_session_step(b, s, H, D, gh, gw, F, T) for s in range(3, 6)]
    torch.cuda.synchronize()
    for s, o in zip(range(3, 6), outs):
        assert torch.equal(o, outs_ref[s]), f"segment {s} after the resume differs"
    assert b.frames_written == ref.frames_written
    n = b.valid_frames * tpf
    for x, y in zip(cache_slots(b), cache_slots(ref)):
        if x is not None:
            assert np.array_equal(x[:n], y[:n])
