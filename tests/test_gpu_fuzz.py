"""Seeded random small shapes through the cached, block-causal and sparse
attention calls, against the fp64 oracle: 1-3 heads, head dims 64 and 128,
tokens per frame from 1 to 60 (odd ones included), empty to wrapped caches built
by several appends, text-only and video-only segments, bf16 and INT8 caches,
split counts 0-5. Full rows, the same tolerance as the other attention tests
(max|diff| <= 1e-2 max|ref|, mean|diff| <= 1e-3). Every case is named before its
GPU step."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, quant, sparse
from oracle.ring import RingModel
from segment_autoregressive_dit_amd import nomas, synth

import test_gpu_block_causal as BC
from _gpu_util import dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _check(got, ref, what):
    diff = np.abs(got - ref)
    mx, mean, lim = diff.max(), diff.mean(), 1e-2 * np.abs(ref).max()
    assert mx <= lim and mean <= 1e-3, f"{what}: max|diff| {mx:.3e} (limit {lim:.3e}), mean {mean:.3e}"


def _cached_case(i):
    r = np.random.default_rng([2026, i])
    H = int(r.choice([1, 2, 3]))
    D = int(r.choice([64, 128]))
    gh, gw = int(r.integers(1, 13)), int(r.integers(1, 21))
    cap = int(r.integers(1, 6))
    appends = [int(r.integers(1, cap + 3)) for _ in range(int(r.integers(0, 4)))]
    F = int(r.integers(0, 4))
    T = int(r.integers(0, 301))
    if F == 0 and T == 0:
        T = 1
    return dict(H=H, D=D, gh=gh, gw=gw, cap=cap, appends=appends, F=F, T=T, int8=bool(r.integers(0, 2)),
                splits=int(r.choice([0, 1, 2, 3, 5])))


@pytest.mark.parametrize("i", range(24))
def test_cached_attention_random_shapes(i):
    c = _cached_case(i)
    H, D, tpf = c["H"], c["D"], c["gh"] * c["gw"]
    say(f"fuzz cached {i}: {c}")
    cache = nomas.KVCache(H, D, tpf, c["cap"], c["int8"])
    ring = RingModel(c["cap"])
    for a, n in enumerate(c["appends"]):
        kb = synth.normal_bf16((n * tpf, H, D), 90 + i, a, 0, 3)
        vb = synth.normal_bf16((n * tpf, H, D), 90 + i, a, 0, 4)
        cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), n)
        ring.append([(kb[f * tpf:(f + 1) * tpf], vb[f * tpf:(f + 1) * tpf]) for f in range(n)])
    nv, nt = c["F"] * tpf, c["T"]
    q, k, v = (synth.normal_bf16((nv + nt, H, D), 90 + i, 9, 0, t) for t in range(3))
    lse = torch.empty(H * (nv + nt), dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), nv, nt, cache, lse=lse,
                                        n_splits=c["splits"])
    torch.cuda.synchronize()
    frames = ring.retained()
    kp = vp = None
    if frames:
        kp = np.concatenate([synth.bf16_bits_to_f64(p[0]) for _, p in frames], 0)
        vp = np.concatenate([synth.bf16_bits_to_f64(p[1]) for _, p in frames], 0)
        if c["int8"]:
            kp, vp = quant.dequantise(*quant.quantise(kp)), quant.dequantise(*quant.quantise(vp))
    x = [synth.bf16_bits_to_f64(t) for t in (q, k, v)]
    ref, ref_lse = attention.segment_attention(x[0], x[1], x[2], kp, vp, 1.0 / math.sqrt(D))
    _check(host_f64(out), ref, f"case {i}")
    assert np.max(np.abs(lse.cpu().numpy().reshape(H, -1) - ref_lse)) <= 2.0 ** -8


@pytest.mark.parametrize("i", range(12))
def test_block_causal_random_sessions(i):
    r = np.random.default_rng([2027, i])
    H, D = int(r.choice([1, 2, 3])), int(r.choice([64, 128]))
    tpf = int(r.integers(1, 41))
    segs, t = [], 0
    for _ in range(int(r.integers(1, 5))):
        F, T = int(r.integers(0, 4)), int(r.integers(0, 30))
        if F == 0 and T == 0:
            T = 1
        segs.append((F * tpf, T, t))
        t += F
    window = [None, 0, 1, 2, 3][int(r.integers(0, 5))]
    BC._run(segs, tpf, window, H, D, seed=200 + i)


@pytest.mark.parametrize("i", range(12))
def test_sparse_attention_random_lists(i):
    r = np.random.default_rng([2028, i])
    H, D = int(r.choice([1, 2])), int(r.choice([64, 128]))
    tpf = int(r.integers(20, 61))
    frames = int(r.integers(1, 9))
    int8 = bool(r.integers(0, 2))
    nv, nt = int(r.integers(0, 3)) * tpf, int(r.integers(1, 300))
    n_cached, n_q = frames * tpf, nv + nt
    nc = sparse.n_candidates(n_cached)
    nqb = (n_q + sparse.QUERY_BLOCK - 1) // sparse.QUERY_BLOCK
    n_sel = int(r.integers(0, nc + 1))
    lists = np.stack([np.stack([np.sort(r.choice(nc, n_sel, replace=False)) for _ in range(nqb)])
                      for _ in range(H)]).astype(np.int32).reshape(H, nqb, n_sel)
    say(f"fuzz sparse {i}: H={H} D={D} tpf={tpf} frames={frames} int8={int8} nv={nv} nt={nt} n_sel={n_sel}")
    kp_b = synth.normal_bf16((n_cached, H, D), 300 + i, 0, 0, 3)
    vp_b = synth.normal_bf16((n_cached, H, D), 300 + i, 0, 0, 4)
    cache = nomas.KVCache(H, D, tpf, frames, int8)
    cache.nomas_kvcache_append(dev_bf16(kp_b), dev_bf16(vp_b), frames)
    q, k, v = (synth.normal_bf16((n_q, H, D), 300 + i, 1, 0, t) for t in range(3))
    out = nomas.nomas_segment_attention_sparse(dev_bf16(q), dev_bf16(k), dev_bf16(v), nv, nt, cache,
                                               torch.from_numpy(lists).cuda(), n_splits=int(r.choice([0, 1, 3])))
    torch.cuda.synchronize()
    kp, vp = synth.bf16_bits_to_f64(kp_b), synth.bf16_bits_to_f64(vp_b)
    if int8:
        kp, vp = quant.dequantise(*quant.quantise(kp)), quant.dequantise(*quant.quantise(vp))
    x = [synth.bf16_bits_to_f64(t) for t in (q, k, v)]
    ref, _ = sparse.sparse_segment_attention(x[0], x[1], x[2], kp, vp, lists, 1.0 / math.sqrt(D))
    _check(host_f64(out), ref, f"sparse case {i}")


@pytest.mark.parametrize("i", range(8))
def test_qkv_projection_random_shapes(i):
    import test_gpu_qkv as QK
    r = np.random.default_rng([2029, i])
    H, D = int(r.integers(1, 7)), int(r.choice([64, 128]))
    hidden = int(r.choice([64, 128, 192, 320, 1024]))
    F, gh, gw = int(r.integers(0, 3)), int(r.integers(1, 9)), int(r.integers(1, 13))
    T = int(r.integers(0, 200))
    if F * gh * gw + T == 0:
        T = 1
    band = (D // 4, 3 * D // 8, 3 * D // 8)
    QK._run(H, D, hidden, F, gh, gw, T, int(r.integers(0, 40)), band, seed=400 + i)


@pytest.mark.parametrize("i", range(10))
def test_append_random_sequences_bit_exact(i):
    import test_gpu_kvcache as KV
    r = np.random.default_rng([2030, i])
    H, D = int(r.integers(1, 5)), int(r.choice([64, 128]))
    tpf = int(r.integers(1, 301))
    cap = int(r.integers(1, 13))
    int8 = bool(r.integers(0, 2))
    sizes = [int(r.integers(1, 2 * cap + 2)) for _ in range(int(r.integers(1, 6)))]
    say(f"fuzz append {i}: H={H} D={D} tpf={tpf} cap={cap} int8={int8} sizes={sizes}")
    cache = nomas.KVCache(H, D, tpf, cap, int8)
    ring = RingModel(cap)
    for a, n in enumerate(sizes):
        kb = synth.normal_bf16((n * tpf, H, D), 500 + i, a, 0, 3)
        vb = synth.normal_bf16((n * tpf, H, D), 500 + i, a, 0, 4)
        cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), n)
        ring.append([(kb[f * tpf:(f + 1) * tpf], vb[f * tpf:(f + 1) * tpf]) for f in range(n)])
        KV._check_cache(cache, ring, tpf, int8)


@pytest.mark.parametrize("i", range(6))
def test_cached_attention_medium_shapes_sampled_rows(i):
    # thousands of cached keys, many tiles per block, several query tiles: the
    # ping-pong loop and the split bounds at sizes between the unit tests and
    # the full layer
    r = np.random.default_rng([2031, i])
    H, D = int(r.integers(1, 5)), int(r.choice([64, 128]))
    gh, gw = int(r.integers(4, 25)), int(r.integers(4, 41))
    tpf = gh * gw
    cap = int(r.integers(2, 9))
    F, T = int(r.integers(1, 4)), int(r.integers(0, 257))
    int8 = bool(r.integers(0, 2))
    splits = int(r.choice([0, 1, 2, 4, 7]))
    say(f"fuzz medium {i}: H={H} D={D} tpf={tpf} cap={cap} F={F} T={T} int8={int8} splits={splits}")
    cache = nomas.KVCache(H, D, tpf, cap, int8)
    kb = synth.normal_bf16((cap * tpf, H, D), 600 + i, 0, 0, 3)
    vb = synth.normal_bf16((cap * tpf, H, D), 600 + i, 0, 0, 4)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), cap)
    nv, nt = F * tpf, T
    q, k, v = (synth.normal_bf16((nv + nt, H, D), 600 + i, 1, 0, t) for t in range(3))
    out = nomas.nomas_segment_attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), nv, nt, cache, n_splits=splits)
    torch.cuda.synchronize()
    kp, vp = synth.bf16_bits_to_f64(kb), synth.bf16_bits_to_f64(vb)
    if int8:
        kp, vp = quant.dequantise(*quant.quantise(kp)), quant.dequantise(*quant.quantise(vp))
    rows = np.unique(np.r_[0, nv + nt - 1, max(0, nv - 1), min(nv, nv + nt - 1), r.integers(0, nv + nt, 40)])
    x = [synth.bf16_bits_to_f64(t) for t in (q, k, v)]
    ref, _ = attention.segment_attention(x[0][rows], x[1], x[2], kp, vp, 1.0 / math.sqrt(D))
    _check(host_f64(out)[rows], ref, f"medium case {i}")


@pytest.mark.parametrize("i", range(16))
def test_frame_range_random(i):
    """nomas_segment_attention_frames over a random range of the retained frames
    of a cache built by random appends (wrapping or not), values row-major or as
    V^T with NaN past n_q, against the oracle over the ring model's frames."""
    r = np.random.default_rng([2032, i])
    H, D = int(r.choice([1, 2, 3])), int(r.choice([64, 128]))
    gh, gw = int(r.integers(1, 9)), int(r.integers(1, 11))
    tpf, cap = gh * gw, int(r.integers(1, 8))
    int8 = bool(r.integers(0, 2))
    appends = [int(r.integers(1, cap + 2)) for _ in range(int(r.integers(1, 5)))]
    cache = nomas.KVCache(H, D, tpf, cap, int8)
    ring = RingModel(cap)
    for a, n in enumerate(appends):
        kb = synth.normal_bf16((n * tpf, H, D), 700 + i, a, 0, 3)
        vb = synth.normal_bf16((n * tpf, H, D), 700 + i, a, 0, 4)
        cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), n)
        ring.append([(kb[f * tpf:(f + 1) * tpf], vb[f * tpf:(f + 1) * tpf]) for f in range(n)])
    fw, valid = ring.frames_written, ring.valid_frames()
    n_frames = int(r.integers(0, valid + 1))
    first = int(r.integers(fw - valid, fw - n_frames + 1))
    nv, nt = int(r.integers(0, 3)) * tpf, int(r.integers(0, 150))
    if nv + nt == 0:
        nt = 1
    n_q = nv + nt
    splits = int(r.choice([0, 1, 2, 3, 5]))
    use_vt = bool(r.integers(0, 2))
    say(f"fuzz frames {i}: H={H} D={D} tpf={tpf} cap={cap} appends={appends} int8={int8} range=[{first}, "
        f"{first + n_frames}) nv={nv} nt={nt} splits={splits} vt={use_vt}")
    q, k, v = (synth.normal_bf16((n_q, H, D), 700 + i, 9, 0, t) for t in range(3))
    vd = dev_bf16(v)
    vt = None
    if use_vt:
        vt = torch.full((H * D, (n_q + 127) // 128 * 128 + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
        vt[:, :n_q] = vd.reshape(n_q, H * D).t()
    lse = torch.empty(H * n_q, dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention_frames(dev_bf16(q), dev_bf16(k), None if use_vt else vd, nv, nt, cache,
                                               first, n_frames, v_t=vt, lse=lse, n_splits=splits)
    torch.cuda.synchronize()
    win = [p for f, p in ring.retained() if first <= f < first + n_frames]
    kp = vp = None
    if win:
        kp = np.concatenate([synth.bf16_bits_to_f64(p[0]) for p in win], 0)
        vp = np.concatenate([synth.bf16_bits_to_f64(p[1]) for p in win], 0)
        if int8:
            kp, vp = quant.dequantise(*quant.quantise(kp)), quant.dequantise(*quant.quantise(vp))
    x = [synth.bf16_bits_to_f64(t) for t in (q, k, v)]
    ref, ref_lse = attention.segment_attention(x[0], x[1], x[2], kp, vp, 1.0 / math.sqrt(D))
    _check(host_f64(out), ref, f"frames case {i}")
    assert np.max(np.abs(lse.cpu().numpy().reshape(H, -1) - ref_lse)) <= 2.0 ** -8


@pytest.mark.parametrize("i", range(8))
def test_fused_projection_random(i):
    """The final-step projection (with V^T) on random shapes and cache states:
    qkv bitwise the plain projection's, the cache byte for byte the plain
    projection + nomas_kvcache_append, V^T the value channels transposed."""
    import test_gpu_qkv as QK
    r = np.random.default_rng([2033, i])
    H, D = int(r.integers(1, 5)), int(r.choice([64, 128]))
    hidden = int(r.choice([64, 128, 256]))
    gh, gw = int(r.integers(1, 7)), int(r.integers(1, 9))
    F, T = int(r.integers(1, 4)), int(r.integers(0, 120))
    cap = int(r.integers(1, 6))
    prior = int(r.integers(0, 2 * cap + 1))
    int8 = bool(r.integers(0, 2))
    say(f"fuzz fused projection {i}: H={H} D={D} hidden={hidden} grid={gh}x{gw} F={F} T={T} cap={cap} "
        f"prior={prior} int8={int8}")
    y_fused, y_plain, caches, ring, tpf, vt = QK._fused_case(H, D, hidden, gh, gw, F, T, cap, int8, prior,
                                                             seed=800 + i, with_vt=True)
    assert torch.equal(y_fused, y_plain)
    for name in ("k", "v", "k_scale", "v_scale"):
        a, b = getattr(caches[0], name), getattr(caches[1], name)
        if a is not None:
            assert torch.equal(a, b), f"cache {name} differs"
    assert caches[0].frames_written == caches[1].frames_written == ring.frames_written
    n = F * tpf + T
    assert torch.equal(vt[:, :n], y_plain[:, 2 * H * D:].t())
