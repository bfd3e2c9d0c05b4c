"""GPU parity of block-sparse segment attention and of the candidate-block
selection against the fp64 oracle (oracle/sparse.py).

Attention is checked given explicit lists (so it does not depend on how the
selection rounds); the selection is checked for validity against fp64 scores
(a near-tie may go either way in float32) and exactly where the scores are well
separated. Tolerances as for the dense call."""

import math

import numpy as np
import pytest
import torch

from oracle import quant, sparse
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import Guarded, dev_bf16, guarded_like, host_f64, say

pytestmark = pytest.mark.gpu

LSE_TOL = 2.0 ** -8


def _check(got, ref, what):
    diff = np.abs(got - ref)
    mx, mean, lim = diff.max(), diff.mean(), 1e-2 * np.abs(ref).max()
    assert mx <= lim and mean <= 1e-3, f"{what}: max|diff| {mx:.3e} (limit {lim:.3e}), mean {mean:.3e}"


def _setup(H, D, tpf, frames, nv, nt, int8, seed, planted=False):
    """Cache of ``frames`` frames + current rows; returns device tensors, the
    cache and the oracle's view of the cached keys/values."""
    n_cached, n_q = frames * tpf, nv + nt
    kp = synth.normal_bf16((n_cached, H, D), 60 + seed, 0, 0, 3)
    vp = synth.normal_bf16((n_cached, H, D), 60 + seed, 0, 0, 4)
    q = synth.normal_bf16((n_q, H, D), 60 + seed, 0, 0, 0)
    if planted:
        # every 128-row cache block leans towards its own direction; query
        # blocks lean towards a few of them, so the top scores are far apart
        rng = np.random.default_rng(seed)
        nc = sparse.n_candidates(n_cached)
        dirs = rng.standard_normal((nc, H, D)).astype(np.float32)
        kf = synth.bf16_bits_to_f64(kp).astype(np.float32) * 0.1
        for c in range(nc):
            kf[c * 128:(c + 1) * 128] += dirs[c]
        qf = synth.bf16_bits_to_f64(q).astype(np.float32) * 0.1
        for b in range((n_q + 255) // 256):
            qf[b * 256:(b + 1) * 256] += dirs[(3 * b) % nc] + 0.7 * dirs[(3 * b + 5) % nc]
        kp = synth._round_bf16_bits(kf)
        q = synth._round_bf16_bits(qf)
    kc = synth.normal_bf16((n_q, H, D), 60 + seed, 0, 0, 1)
    vc = synth.normal_bf16((n_q, H, D), 60 + seed, 0, 0, 2)
    cache = nomas.KVCache(H, D, tpf, frames, int8)
    cache.nomas_kvcache_append(dev_bf16(kp), dev_bf16(vp), frames)
    kpf, vpf = synth.bf16_bits_to_f64(kp), synth.bf16_bits_to_f64(vp)
    if int8:
        kpf, vpf = quant.dequantise(*quant.quantise(kpf)), quant.dequantise(*quant.quantise(vpf))
    x = [synth.bf16_bits_to_f64(t) for t in (q, kc, vc)]
    return (dev_bf16(q), dev_bf16(kc), dev_bf16(vc)), cache, x, kpf, vpf


def _random_lists(H, nqb, nc, n_sel, seed):
    rng = np.random.default_rng(seed)
    lists = np.stack([np.stack([np.sort(rng.choice(nc, n_sel, replace=False)) for _ in range(nqb)])
                      for _ in range(H)]).astype(np.int32)
    lists[0, 0, -1] = nc - 1 if nc - 1 not in lists[0, 0, :-1] else lists[0, 0, -1]   # the short last block
    lists[0, 0] = np.sort(lists[0, 0])
    return lists


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("int8", [False, True])
def test_sparse_attention_given_lists(int8, splits, D):
    # 12x20 grid, 6 cached frames = 1,440 rows = 12 candidate blocks (the last of
    # 32 rows); 2-frame segment + 40 text = 520 queries = 3 query blocks
    H, tpf, nv, nt = 2, 240, 480, 40
    (q, k, v), cache, x, kp, vp = _setup(H, D, tpf, 6, nv, nt, int8, seed=int8)
    nc = sparse.n_candidates(kp.shape[0])
    assert nc == 12
    lists = _random_lists(H, 3, nc, 3, seed=10 + splits)
    say(f"sparse attention: int8={int8} splits={splits} D={D}")
    lse = torch.empty(H * (nv + nt), dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention_sparse(q, k, v, nv, nt, cache, torch.from_numpy(lists).cuda(), lse=lse,
                                               n_splits=splits)
    torch.cuda.synchronize()
    ref, ref_lse = sparse.sparse_segment_attention(x[0], x[1], x[2], kp, vp, lists, 1 / math.sqrt(D))
    _check(host_f64(out), ref, "sparse attention")
    assert np.max(np.abs(lse.cpu().numpy().reshape(H, -1) - ref_lse)) <= LSE_TOL


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("int8", [False, True])
def test_sparse_automatic_many_splits(int8, D):
    # one head, 3 query blocks against lists of 100 of 113 candidate blocks (the
    # short last one included): the automatic plan cuts the listed rows several
    # ways (one block per split), so splits that get no key tile and the merge
    # of many partials are both exercised
    H, tpf, nv, nt = 1, 240, 480, 40
    (q, k, v), cache, x, kp, vp = _setup(H, D, tpf, 60, nv, nt, int8, seed=20 + int8)
    nc = sparse.n_candidates(kp.shape[0])
    assert nc == 113
    lists = _random_lists(H, 3, nc, 100, seed=30 + D)
    splits = nomas.nomas_segment_attention_splits(nv, nt, 100 * 128, H, D, int(int8), 0)
    assert splits >= 6, splits
    say(f"sparse attention, automatic {splits} splits: int8={int8} D={D}")
    lse = torch.empty(H * (nv + nt), dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention_sparse(q, k, v, nv, nt, cache, torch.from_numpy(lists).cuda(), lse=lse,
                                               n_splits=0)
    torch.cuda.synchronize()
    ref, ref_lse = sparse.sparse_segment_attention(x[0], x[1], x[2], kp, vp, lists, 1 / math.sqrt(D))
    _check(host_f64(out), ref, "sparse attention, automatic splits")
    assert np.max(np.abs(lse.cpu().numpy().reshape(H, -1) - ref_lse)) <= LSE_TOL


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("int8", [False, True])
def test_all_blocks_equals_dense(int8, D):
    H, tpf, nv, nt = 2, 240, 480, 40
    (q, k, v), cache, _, kp, _ = _setup(H, D, tpf, 6, nv, nt, int8, seed=2)
    nc = sparse.n_candidates(kp.shape[0])
    lists = torch.arange(nc, dtype=torch.int32).repeat(H, 3, 1).cuda()
    say(f"sparse all blocks vs dense: int8={int8} D={D}")
    a = nomas.nomas_segment_attention_sparse(q, k, v, nv, nt, cache, lists, n_splits=1)
    b = nomas.nomas_segment_attention(q, k, v, nv, nt, cache, n_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_no_blocks_is_segment_only():
    H, D, tpf, nv, nt = 2, 64, 24, 48, 16
    (q, k, v), cache, x, kp, vp = _setup(H, D, tpf, 4, nv, nt, False, seed=3)
    lists = torch.empty((H, 1, 0), dtype=torch.int32, device="cuda")
    out = nomas.nomas_segment_attention_sparse(q, k, v, nv, nt, cache, lists)
    torch.cuda.synchronize()
    ref, _ = sparse.sparse_segment_attention(x[0], x[1], x[2], kp, vp, np.zeros((H, 1, 0), np.int32), 0.125)
    _check(host_f64(out), ref, "no blocks")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("int8", [False, True])
def test_selection_is_valid(int8, D):
    H, tpf, nv, nt = 2, 240, 480, 40
    (q, _, _), cache, x, kp, _ = _setup(H, D, tpf, 6, nv, nt, int8, seed=4)
    nc = sparse.n_candidates(kp.shape[0])
    say(f"sparse select: int8={int8} D={D}")
    for n_sel in (1, 3, nc):
        got = nomas.nomas_sparse_select(q, nv + nt, cache, n_sel).cpu().numpy()
        scores = sparse.block_scores(x[0], kp)
        for h in range(H):
            for b in range(got.shape[1]):
                g = got[h, b]
                assert np.all(np.diff(g) > 0) and g[0] >= 0 and g[-1] < nc
                s = scores[h, b]
                rest = np.setdiff1d(np.arange(nc), g)
                tol = 1e-4 * (np.abs(s).max() + 1.0)
                if len(rest):
                    assert s[g].min() >= s[rest].max() - tol


def test_selection_matches_oracle_when_separated():
    H, D, tpf, nv, nt = 2, 128, 240, 480, 40
    for int8 in (False, True):
        (q, _, _), cache, x, kp, _ = _setup(H, D, tpf, 6, nv, nt, int8, seed=5, planted=True)
        got = nomas.nomas_sparse_select(q, nv + nt, cache, 2).cpu().numpy()
        ref = sparse.select_blocks(x[0], kp, 2)
        assert np.array_equal(got, ref), (got, ref)


def test_layer_select_then_attend_sampled_rows():
    """Full head shape (16x128, 17,280 cached rows = 135 candidates, 7,936
    queries): GPU selection of 34 blocks (25 %), then sparse attention; sampled
    rows against the oracle given the GPU's lists."""
    wl = synth.WORKLOADS["layer_bf16"]
    H, D = wl.n_heads, wl.head_dim
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, False)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    qb, kcb, vcb = synth.current_qkv(wl)
    q, k, v = dev_bf16(qb), dev_bf16(kcb), dev_bf16(vcb)
    nc = nomas.nomas_sparse_candidates(cache.n_cached)
    assert nc == 135
    say("sparse layer: select + attend")
    # the block lists, the selection's workspace, out, lse and the attention
    # workspace sit between sentinel bands; the lists must also come back unchanged
    nqb = (wl.n_q + 255) // 256
    g_l = Guarded(4 * H * nqb * 34)
    g_sw = Guarded(max(256, nomas.lib().nomas_sparse_select_workspace_bytes(wl.n_q, cache.n_cached, H, D)))
    lists = nomas.nomas_sparse_select(q, wl.n_q, cache, 34, block_list=g_l.view(torch.int32, (H, nqb, 34)),
                                      workspace=g_sw.view(torch.uint8, (g_sw.nbytes,)))
    g_l.check("selection block_list")
    g_sw.check("selection workspace")
    g_lists, lists_in = guarded_like(lists)
    g_out = Guarded(2 * wl.n_q * H * D)
    g_lse = Guarded(4 * H * wl.n_q)
    g_ws = Guarded(max(256, nomas.nomas_segment_attention_workspace_bytes(wl.n_video, wl.n_text, 34 * 128, H, D, 0)))
    out = nomas.nomas_segment_attention_sparse(q, k, v, wl.n_video, wl.n_text, cache, lists_in,
                                               out=g_out.view(torch.bfloat16, (wl.n_q, H, D)),
                                               lse=g_lse.view(torch.float32, (H * wl.n_q,)),
                                               workspace=g_ws.view(torch.uint8, (g_ws.nbytes,)))
    for g, what in ((g_lists, "sparse block_list"), (g_out, "sparse out"), (g_lse, "sparse lse"),
                    (g_ws, "sparse workspace")):
        g.check(what)
    assert torch.equal(lists_in, lists), "the attention call changed its block lists"
    torch.cuda.synchronize()
    got, L = host_f64(out), lists.cpu().numpy()
    xq, xk, xv = (synth.bf16_bits_to_f64(t) for t in (qb, kcb, vcb))
    kp, vp = synth.bf16_bits_to_f64(kb), synth.bf16_bits_to_f64(vb)
    rows = [0, 255, 256, 4000, wl.n_video - 1, wl.n_video, wl.n_q - 1]
    for r in rows:
        ref, _ = sparse.sparse_segment_attention(xq[r:r + 1], xk, xv, kp, vp, L[:, r // 256:r // 256 + 1], 1 / math.sqrt(D))
        _check(got[r:r + 1], ref, f"row {r}")


@pytest.mark.parametrize("splits", [2, 3])
@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_split_without_key_tiles(D, int8, splits):
    """A list whose only block is the short last candidate (one 20-row frame):
    the split count is planned for 128 listed rows, so with 64-key tiles (INT8,
    or head dim 64) a block has fewer key tiles than splits and one split gets
    none. That split must count for nothing in the merge (it once wrote NaN)."""
    H, tpf, nv, nt = 2, 20, 0, 16
    (q, k, v), cache, x, kp, vp = _setup(H, D, tpf, 1, nv, nt, int8, seed=7)
    lists = np.zeros((H, 1, 1), np.int32)
    say(f"sparse split without tiles: D={D} int8={int8} splits={splits}")
    lse = torch.empty(H * (nv + nt), dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention_sparse(q, k, v, nv, nt, cache, torch.from_numpy(lists).cuda(), lse=lse,
                                               n_splits=splits)
    torch.cuda.synchronize()
    got = host_f64(out)
    assert np.all(np.isfinite(got)), "non-finite output from an empty split"
    ref, ref_lse = sparse.sparse_segment_attention(x[0], x[1], x[2], kp, vp, lists, 1 / math.sqrt(D))
    _check(got, ref, "split without key tiles")
    assert np.max(np.abs(lse.cpu().numpy().reshape(H, -1) - ref_lse)) <= LSE_TOL
