"""GPU parity of nomas_segment_attention against the fp64 oracle
(oracle/attention.py), with the cache contents modelled by oracle/ring.py and
oracle/quant.py. Tolerance for bf16 and INT8 paths vs fp64:
max|diff| <= 1e-2 * max|ref| and mean|diff| <= 1e-3. For INT8 the reference
attends to the *dequantised* cache, so the kernel is not charged for the
quantisation error."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, quant
from oracle.ring import RingModel
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import Guarded, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu

# The kernel's softmax denominator sums the probabilities as rounded to bf16 (the
# values the value MFMA multiplies), each within a relative 2^-9 of exact, so the
# sum is within a relative 2^-9 and its log within log(1 + 2^-9) < 2^-9; fp32
# exp2/log2 add ~1e-6. Bound: 2^-8.
LSE_TOL = 2.0 ** -8


def _prefill(wl, cache, ring, chunk=None, layer=0, ones_v=False):
    """Append the workload's pre-fill frames (GPU cache and oracle ring model)."""
    if wl.cached_frames == 0:
        return
    kb, vb = synth.prefill_kv(wl, layer)
    if ones_v:
        vb = np.full_like(vb, 0x3F80)
    tpf = wl.tpf
    chunk = chunk or wl.seg_frames
    f = 0
    while f < wl.cached_frames:
        n = min(chunk, wl.cached_frames - f)
        sl = slice(f * tpf, (f + n) * tpf)
        cache.nomas_kvcache_append(dev_bf16(kb[sl]), dev_bf16(vb[sl]), n)
        ring.append([(kb[(f + i) * tpf:(f + i + 1) * tpf], vb[(f + i) * tpf:(f + i + 1) * tpf]) for i in range(n)])
        f += n


def _past_from_ring(ring, int8):
    frames = ring.retained()
    if not frames:
        return None, None
    k = np.concatenate([synth.bf16_bits_to_f64(p[0]) for _, p in frames], 0)
    v = np.concatenate([synth.bf16_bits_to_f64(p[1]) for _, p in frames], 0)
    if int8:
        qk, sk = quant.quantise(k)
        qv, sv = quant.quantise(v)
        k, v = quant.dequantise(qk, sk), quant.dequantise(qv, sv)
    return k, v


def _check(got, ref, what):
    diff = np.abs(got - ref)
    mx, mean, lim = diff.max(), diff.mean(), 1e-2 * np.abs(ref).max()
    assert mx <= lim and mean <= 1e-3, f"{what}: max|diff| {mx:.3e} (limit {lim:.3e}), mean {mean:.3e}"
    return mx, mean


def _sample_rows(n_q, n_video, rng, extra=24):
    rows = {0, 1, 15, 16, 127, 128, 255, 256, 511, 512, n_q - 1, max(0, n_video - 1), min(n_q - 1, n_video)}
    rows |= set(rng.integers(0, n_q, extra).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n_q))


# full-row oracle references of the full-shape workloads, computed once per
# workload and reused by the tests that run it with different split counts
_FULL_REF = {}


def _run(wl, n_splits=0, full=False, with_lse=True, n_video=None, n_text=None, cached_frames=None,
         ones_v=False, repeat=1):
    """Run one attention call of workload ``wl`` on the GPU and check it
    (``full``: every query row of every head; otherwise sampled rows)."""
    if cached_frames is not None:
        wl = synth.Workload(**{**wl.__dict__, "cached_frames": cached_frames})
    H, D = wl.n_heads, wl.head_dim
    say(f"attention: {wl.name} splits={n_splits} cached={wl.cached_frames} nv={n_video} nt={n_text}")
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, wl.kv_int8)
    ring = RingModel(wl.capacity_frames)
    _prefill(wl, cache, ring, ones_v=ones_v)
    q_bits, k_bits, v_bits = synth.current_qkv(wl)
    nv = wl.n_video if n_video is None else n_video
    nt = wl.n_text if n_text is None else n_text
    rows_all = np.r_[0:nv, wl.n_video:wl.n_video + nt]
    q_bits, k_bits, v_bits = q_bits[rows_all], k_bits[rows_all], v_bits[rows_all]
    if ones_v:
        v_bits = np.full_like(v_bits, 0x3F80)
    q, k, v = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits)
    n_q = nv + nt
    # out, lse and the workspace sit between sentinel bands, checked after every call
    g_lse = Guarded(4 * H * n_q) if with_lse else None
    lse = g_lse.view(torch.float32, (H * n_q,)) if with_lse else None
    g_ws = Guarded(max(256, nomas.nomas_segment_attention_workspace_bytes(
        nv, nt, cache.n_cached, H, D, int(wl.kv_int8), n_splits)))
    ws = g_ws.view(torch.uint8, (g_ws.nbytes,))
    outs = []
    for _ in range(repeat):
        g_out = Guarded(2 * n_q * H * D)
        outs.append(nomas.nomas_segment_attention(q, k, v, nv, nt, cache, out=g_out.view(torch.bfloat16, (n_q, H, D)),
                                                  lse=lse, n_splits=n_splits, workspace=ws))
        g_out.check("attention out")
    g_ws.check("attention workspace")
    if g_lse:
        g_lse.check("attention lse")
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "results differ between identical calls"
    got = host_f64(outs[0])
    scale = 1.0 / math.sqrt(D)
    if full:
        rows = np.arange(n_q)
    else:
        rows = _sample_rows(n_q, nv, np.random.default_rng(n_q))
    key = (wl, nv, nt, ones_v, full)
    if key not in _FULL_REF:
        _FULL_REF.clear()          # keep one reference (they reach 130 MB)
        kp, vp = _past_from_ring(ring, wl.kv_int8)
        x = [synth.bf16_bits_to_f64(t) for t in (q_bits, k_bits, v_bits)]
        say(f"attention: oracle on {len(rows)} rows x {H} heads")
        _FULL_REF[key] = attention.segment_attention(x[0][rows], x[1], x[2], kp, vp, scale)
    ref, ref_lse = _FULL_REF[key]
    res = _check(got[rows], ref, wl.name)
    if with_lse:
        g_lse = lse.cpu().numpy().reshape(H, n_q)[:, rows]
        assert np.max(np.abs(g_lse - ref_lse)) <= LSE_TOL, np.max(np.abs(g_lse - ref_lse))
    return got, res


@pytest.mark.parametrize("int8", [False, True])
def test_tiny_all_rows(int8):
    wl = synth.Workload(**{**synth.WORKLOADS["tiny"].__dict__, "kv_int8": int8})
    _run(wl, full=True, repeat=2)


@pytest.mark.parametrize("splits", [1, 2, 3, 5])
def test_tiny_splits(splits):
    _run(synth.WORKLOADS["tiny"], n_splits=splits, full=True)


@pytest.mark.parametrize("case", ["empty_cache", "text_only", "video_only", "one_query", "one_frame_cache"])
def test_tiny_edge_cases(case):
    wl = synth.WORKLOADS["tiny"]
    kw = dict(empty_cache=dict(cached_frames=0), text_only=dict(n_video=0), video_only=dict(n_text=0),
              one_query=dict(n_video=0, n_text=1), one_frame_cache=dict(cached_frames=1))[case]
    _run(wl, full=True, **kw)


@pytest.mark.parametrize("int8", [False, True])
def test_ones_values_give_ones(int8):
    wl = synth.Workload(**{**synth.WORKLOADS["layer_bf16"].__dict__, "kv_int8": int8})
    got, _ = _run(wl, ones_v=True, with_lse=False)
    # bf16: exactly representable 1; int8: each cached v is 127 * fp32(1/127)
    assert np.max(np.abs(got - 1.0)) <= 2.0 ** -7


def test_layer_bf16():
    # every query row of every head (7,936 x 16) against the oracle
    _run(synth.WORKLOADS["layer_bf16"], full=True, repeat=2)


def test_layer_int8_outliers():
    _run(synth.WORKLOADS["layer_int8"], full=True, repeat=2)


def test_layer_880_ragged():
    # 22x40 = 880 tokens per frame: ragged cache tail, ragged query tail
    _run(synth.WORKLOADS["layer_880"], full=True)


@pytest.mark.parametrize("splits", [1, 2, 4, 8, 0])
def test_long_history_splits(splits):
    # 84,480 cached + 7,936 current keys, all rows; the oracle runs once for the
    # five split counts
    _run(synth.WORKLOADS["long_bf16"], n_splits=splits, full=True)


@pytest.mark.parametrize("splits", [1, 0])
@pytest.mark.parametrize("int8", [False, True])
def test_head_share_of_eight_gpus(int8, splits):
    # one GPU's share when the 16 heads are spread over 8 GPUs: 2 heads at the
    # full sequence lengths (7,936 queries x 25,216 keys), every row; with
    # n_splits = 0 the plan splits the keys to fill the chip
    base = synth.WORKLOADS["layer_int8" if int8 else "layer_bf16"]
    _run(synth.Workload(**{**base.__dict__, "n_heads": 2}), n_splits=splits, full=True)


@pytest.mark.parametrize("int8", [False, True])
def test_one_query_long_history_many_splits(int8):
    # one text query of one head against 84,480 cached keys: the automatic plan
    # cuts the keys into 38 (bf16) or 75 (INT8) splits of one block each, and
    # the merge combines them
    base = synth.WORKLOADS["long_bf16"]
    wl = synth.Workload(**{**base.__dict__, "n_heads": 1, "kv_int8": int8})
    assert nomas.nomas_segment_attention_splits(0, 1, wl.n_cached, 1, wl.head_dim, int(int8), 0) == (75 if int8 else 38)
    _run(wl, n_video=0, n_text=1, full=True)


def test_split_results_agree():
    # every split count gives the same answer to within fp32 merge rounding
    wl = synth.WORKLOADS["long_bf16"]
    cache = nomas.KVCache(wl.n_heads, wl.head_dim, wl.tpf, wl.capacity_frames, False)
    _prefill(wl, cache, RingModel(wl.capacity_frames))
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    say("attention: split agreement")
    res = [host_f64(nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, n_splits=s))
           for s in (1, 3, 8)]
    for r in res[1:]:
        assert np.max(np.abs(r - res[0])) <= 2.0 ** -6 * np.abs(res[0]).max()


def test_session_rope_append_attention():
    """Four segments through the whole path (RoPE -> attention -> append) with an
    INT8 window of 3 frames that evicts inside a segment, against the oracle run
    of the same session (oracle RoPE, quantiser and ring)."""
    from oracle import formats, rope
    H, D, gh, gw, F, T, W = 2, 64, 4, 6, 2, 16, 3
    tpf = gh * gw
    cache = nomas.KVCache(H, D, tpf, W, True)
    ring = RingModel(W)
    for s in range(4):
        say(f"session segment {s}")
        n = F * tpf + T
        qb = synth.normal_bf16((n, H, D), 11, 0, s, 0)
        kb = synth.normal_bf16((n, H, D), 11, 0, s, 1)
        vb = synth.normal_bf16((n, H, D), 11, 0, s, 2)
        q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
        nomas.nomas_rope3d(q, k, s * F, F, gh, gw, (16, 24, 24), H, D)
        out = nomas.nomas_segment_attention(q, k, v, F * tpf, T, cache)
        cache.nomas_kvcache_append(k, v, F)
        # oracle
        xq, xk, xv = (synth.bf16_bits_to_f64(t) for t in (qb, kb, vb))
        nv = F * tpf
        xq[:nv] = formats.to_bf16(rope.rope3d_segment(xq[:nv], s * F, F, gh, gw, 16, 24, 24))
        xk[:nv] = formats.to_bf16(rope.rope3d_segment(xk[:nv], s * F, F, gh, gw, 16, 24, 24))
        frames = ring.retained()
        kp = vp = None
        if frames:
            kp = np.concatenate([quant.dequantise(*p[0]) for _, p in frames], 0)
            vp = np.concatenate([quant.dequantise(*p[1]) for _, p in frames], 0)
        ref, _ = attention.segment_attention(xq, xk, xv, kp, vp, 1 / math.sqrt(D))
        _check(host_f64(out), ref, f"session segment {s}")
        ring.append([(quant.quantise(xk[f * tpf:(f + 1) * tpf]), quant.quantise(xv[f * tpf:(f + 1) * tpf]))
                     for f in range(F)])


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_rising_logits_raise_reference(D, int8, splits):
    """Every 64-key run holds one key whose logit tops all earlier ones by about
    140 (log2 units), at a position that moves from run to run: each tile must
    raise the running softmax reference, and a raise missed for any key position
    overflows the probabilities (inf/NaN output)."""
    H, tpf, frames, nv, nt = 2, 64, 12, 128, 16
    n_cached = frames * tpf
    q_b, kc_b, vc_b, kn_b, vn_b = synth.rising_logit_inputs(H, D, n_cached, nv + nt, seed=D + 2 * int8)
    say(f"attention: rising logits D={D} int8={int8} splits={splits}")
    cache = nomas.KVCache(H, D, tpf, frames, int8)
    cache.nomas_kvcache_append(dev_bf16(kc_b), dev_bf16(vc_b), frames)
    lse = torch.empty(H * (nv + nt), dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention(dev_bf16(q_b), dev_bf16(kn_b), dev_bf16(vn_b), nv, nt, cache, lse=lse,
                                        n_splits=splits)
    torch.cuda.synchronize()
    got = host_f64(out)
    assert np.all(np.isfinite(got)), "non-finite output: a tile did not raise the softmax reference"
    kp, vp = synth.bf16_bits_to_f64(kc_b), synth.bf16_bits_to_f64(vc_b)
    if int8:
        kp, vp = quant.dequantise(*quant.quantise(kp)), quant.dequantise(*quant.quantise(vp))
    x = [synth.bf16_bits_to_f64(t) for t in (q_b, kn_b, vn_b)]
    ref, ref_lse = attention.segment_attention(x[0], x[1], x[2], kp, vp, 1.0 / math.sqrt(D))
    _check(got, ref, f"rising logits D={D} int8={int8}")
    g_lse = lse.cpu().numpy().reshape(H, nv + nt)
    # logits reach ~1.5e3 (natural units): fp32 rounding of the logit itself adds
    # a few ulp of that size on top of the probability-sum bound
    assert np.max(np.abs(g_lse - ref_lse)) <= LSE_TOL + 1e-3, np.max(np.abs(g_lse - ref_lse))


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_rising_and_falling_logits_in_one_wave(D, int8):
    """Even query rows climb as above while odd rows peak in the first tile and
    fall about 140 (log2 units) below that peak afterwards: every later tile
    raises the reference for the even rows of a wave but must leave the odd
    rows' reference where it is (a raise that lowered it would rescale their
    output by about 2^140 and overflow)."""
    H, tpf, frames, nv, nt = 2, 64, 12, 128, 16
    n_cached = frames * tpf
    q_b, kc_b, vc_b, kn_b, vn_b = synth.rising_logit_inputs(H, D, n_cached, nv + nt, seed=5 + D + 2 * int8,
                                                            mixed=True)
    say(f"attention: rising and falling logits D={D} int8={int8}")
    cache = nomas.KVCache(H, D, tpf, frames, int8)
    cache.nomas_kvcache_append(dev_bf16(kc_b), dev_bf16(vc_b), frames)
    lse = torch.empty(H * (nv + nt), dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention(dev_bf16(q_b), dev_bf16(kn_b), dev_bf16(vn_b), nv, nt, cache, lse=lse,
                                        n_splits=1)
    torch.cuda.synchronize()
    got = host_f64(out)
    assert np.all(np.isfinite(got)), "non-finite output: a raise moved some query's reference down"
    kp, vp = synth.bf16_bits_to_f64(kc_b), synth.bf16_bits_to_f64(vc_b)
    if int8:
        kp, vp = quant.dequantise(*quant.quantise(kp)), quant.dequantise(*quant.quantise(vp))
    x = [synth.bf16_bits_to_f64(t) for t in (q_b, kn_b, vn_b)]
    ref, ref_lse = attention.segment_attention(x[0], x[1], x[2], kp, vp, 1.0 / math.sqrt(D))
    _check(got, ref, f"rising and falling logits D={D} int8={int8}")
    g_lse = lse.cpu().numpy().reshape(H, nv + nt)
    assert np.max(np.abs(g_lse - ref_lse)) <= LSE_TOL + 1e-3, np.max(np.abs(g_lse - ref_lse))


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_values_of_one_key_range(D, int8):
    """Values nonzero in one key range at a time (a full cache tile, the partial
    last cache tile, a full current tile, the partial last current tile), with
    all other values zero: the output is then that range's share alone, so a
    tile whose values are lost, misplaced or zeroed in LDS shows as a large
    error, not one hidden under the tolerance. 6 frames of 240 cached rows =
    1,440 (a partial last tile for both key-tile sizes), 480 + 40 current rows
    (a partial last current tile)."""
    H, tpf, frames, nv, nt = 2, 240, 6, 480, 40
    n_cached, n_q = frames * tpf, nv + nt
    kp = synth.normal_bf16((n_cached, H, D), 71, 0, 0, 3)
    vp_all = synth.normal_bf16((n_cached, H, D), 71, 0, 0, 4)
    q = synth.normal_bf16((n_q, H, D), 71, 0, 0, 0)
    kc = synth.normal_bf16((n_q, H, D), 71, 0, 0, 1)
    vc_all = synth.normal_bf16((n_q, H, D), 71, 0, 0, 2)
    kpf = synth.bf16_bits_to_f64(kp)
    if int8:
        kpf = quant.dequantise(*quant.quantise(kpf))
    x = [synth.bf16_bits_to_f64(t) for t in (q, kc)]
    for part, lo, hi in (("cache", 128, 256), ("cache", 1408, 1440), ("current", 128, 256), ("current", 512, 520)):
        vp = np.zeros_like(vp_all)
        vc = np.zeros_like(vc_all)
        (vp if part == "cache" else vc)[lo:hi] = (vp_all if part == "cache" else vc_all)[lo:hi]
        say(f"attention: values of {part} rows [{lo}, {hi}) only, D={D} int8={int8}")
        cache = nomas.KVCache(H, D, tpf, frames, int8)
        cache.nomas_kvcache_append(dev_bf16(kp), dev_bf16(vp), frames)
        out = nomas.nomas_segment_attention(dev_bf16(q), dev_bf16(kc), dev_bf16(vc), nv, nt, cache, n_splits=1)
        torch.cuda.synchronize()
        vpf = synth.bf16_bits_to_f64(vp)
        if int8:
            vpf = quant.dequantise(*quant.quantise(vpf))
        ref, _ = attention.segment_attention(x[0], x[1], synth.bf16_bits_to_f64(vc), kpf, vpf, 1.0 / math.sqrt(D))
        _check(host_f64(out), ref, f"values of {part} rows [{lo}, {hi}) only")


@pytest.mark.parametrize("int8", [False, True])
def test_strided_out_leaves_the_gaps(int8):
    """Full layer shape with out as a strided view (row stride H*D + 64): the
    64 columns between rows keep their sentinel bytes, and the values equal the
    contiguous call's bit for bit."""
    wl = synth.Workload(**{**synth.WORKLOADS["layer_bf16"].__dict__, "kv_int8": int8})
    H, D, n_q = wl.n_heads, wl.head_dim, wl.n_q
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, int8)
    _prefill(wl, cache, RingModel(wl.capacity_frames))
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    say(f"attention: strided out, int8={int8}")
    wide = torch.full((n_q, H * D + 64), -7.0, dtype=torch.bfloat16, device="cuda")
    ref = nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache)
    got = nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=wide[:, :H * D])
    torch.cuda.synchronize()
    assert bool((wide[:, H * D:] == -7.0).all()), "bytes between output rows changed"
    assert torch.equal(got.reshape(n_q, H, D), ref)
