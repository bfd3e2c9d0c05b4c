"""GPU check of nomas_segment_attention_noalloc, the variant of
nomas_segment_attention that allocates nothing (its workspace is the library's
own scratch array): called through the C ABI, its output and log-sum-exp equal
the workspace entry point's, bit for bit (same kernels, same plan), on two calls
in a row, the second smaller than the first (the array keeps the first call's
contents); sizes beyond the array are refused before anything is enqueued."""

import numpy as np
import pytest
import torch

from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


def _setup(wl, int8):
    cache = nomas.KVCache(wl.n_heads, wl.head_dim, wl.tpf, wl.capacity_frames, int8)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    return cache, q, k, v


def _both(wl, cache, q, k, v, n_splits):
    H, n_q = wl.n_heads, wl.n_q
    out_a, out_b = torch.empty_like(q), torch.full_like(q, float("nan"))
    lse_a = torch.empty(H * n_q, dtype=torch.float32, device="cuda")
    lse_b = torch.full_like(lse_a, float("nan"))
    nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out_a, lse=lse_a, n_splits=n_splits)
    nomas.nomas_segment_attention_noalloc(q, k, v, wl.n_video, wl.n_text, cache, out_b, lse=lse_b,
                                          n_splits=n_splits)
    torch.cuda.synchronize()
    return (out_a, lse_a), (out_b, lse_b)


@pytest.mark.parametrize("int8", [False, True])
def test_noalloc_equals_workspace_call_large_then_small(int8):
    big = synth.WORKLOADS["layer_int8" if int8 else "layer_bf16"]
    small = synth.Workload(**{**synth.WORKLOADS["tiny"].__dict__, "kv_int8": int8})
    for wl, splits in ((big, 0), (small, 3)):
        need = nomas.nomas_segment_attention_workspace_bytes(wl.n_video, wl.n_text, wl.n_cached, wl.n_heads,
                                                             wl.head_dim, int(int8), splits)
        assert need <= nomas.nomas_segment_attention_noalloc_max_bytes()
        say(f"noalloc: {wl.name} int8={int8} splits={splits} ({need} bytes of scratch)")
        cache, q, k, v = _setup(wl, int8)
        (oa, la), (ob, lb) = _both(wl, cache, q, k, v, splits)
        assert torch.equal(oa, ob), f"{wl.name}: outputs differ"
        assert torch.equal(la, lb), f"{wl.name}: log-sum-exps differ"
        assert torch.isfinite(ob.float()).all()


def test_noalloc_refuses_sizes_beyond_the_array():
    wl = synth.WORKLOADS["layer_bf16"]
    cache, q, k, v = _setup(wl, False)
    out = torch.zeros_like(q)
    # 8 splits at the layer shape need 32.5 MB + 8 x 65 MB of partials
    need = nomas.nomas_segment_attention_workspace_bytes(wl.n_video, wl.n_text, wl.n_cached, wl.n_heads,
                                                         wl.head_dim, 0, 8)
    assert need > nomas.nomas_segment_attention_noalloc_max_bytes()
    with pytest.raises(nomas.NomasError) as e:
        nomas.nomas_segment_attention_noalloc(q, k, v, wl.n_video, wl.n_text, cache, out, n_splits=8)
    assert e.value.code == nomas.NOMAS_E_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not out.any(), "a refused call wrote its output"
