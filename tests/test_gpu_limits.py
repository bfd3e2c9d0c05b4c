"""GPU checks at the library's size limits: one head's cache slice just under
2 GiB (the kernels address a head's K or V slice, and the buffer ranges of its
loads, with 32-bit byte offsets), filled by the append kernel and read back by
attention at its first, middle and very last tokens.

Almost every key and value is zero; four marker keys k_m = b e_m (channel m)
sit at chosen cache tokens with values v_m, and the queries are a e_m or zero.
The exact result then follows from the definition of attention in closed form
(softmax weights exp(logit) over all N keys, zero keys having logit 0):
  query m:   O = (e^L v_m + sum_{m' != m} v_m') / (e^L + N - 1),  lse = ln(e^L + N - 1)
  zero query: O = sum_m v_m / N,                                   lse = ln N
with L = a b / sqrt(D) (INT8: b and v_m as the cache holds them, dequantised by
oracle.quant). Tolerance as for every attention test: max|diff| <= 1e-2 max|ref|,
mean|diff| <= 1e-3; lse within 2^-8."""

import math

import numpy as np
import pytest
import torch

from oracle import quant
from segment_autoregressive_dit_amd import nomas

from _gpu_util import host_f64, say

pytestmark = pytest.mark.gpu

H, D, TPF = 1, 128, 1024
N_TEXT = 16
A = 16.0          # query scale (bf16-exact)
B = 21.25         # marker key scale (bf16-exact): L = 16 * 21.25 / sqrt(128) ~ 30.05


def _marker_values(m):
    """v_m: distinct bf16-exact values per marker."""
    return np.array([(m + 1) * 0.5 + (d % 7) * 0.125 for d in range(D)])


@pytest.mark.parametrize("int8", [False, True])
def test_head_slice_just_under_2gib(int8):
    # the largest capacity whose per-head slice stays below 2 GiB
    cap = 16383 if int8 else 8191
    pitch = nomas.lib().nomas_kvcache_token_pitch(TPF, cap)
    assert pitch * D * (1 if int8 else 2) < 2 ** 31
    assert (pitch + TPF) * D * (1 if int8 else 2) >= 2 ** 31 - 2 ** 20   # within a frame of the limit
    n_cached = cap * TPF
    say(f"limits: int8={int8} capacity={cap} frames, {n_cached} cached tokens, slice {pitch * D * (1 if int8 else 2)} B")
    cache = nomas.KVCache(H, D, TPF, cap, int8)
    markers = [0, n_cached // 3 + 5, 2 * n_cached // 3 + 77, n_cached - 1]
    chunk_frames = 512
    kz = torch.zeros((chunk_frames * TPF, H * D), dtype=torch.bfloat16, device="cuda")
    vz = torch.zeros_like(kz)
    f = 0
    while f < cap:
        n = min(chunk_frames, cap - f)
        r0, r1 = f * TPF, (f + n) * TPF
        hit = [(m, t) for m, t in enumerate(markers) if r0 <= t < r1]
        for m, t in hit:
            kz[t - r0, m] = B
            vz[t - r0] = torch.tensor(_marker_values(m), dtype=torch.bfloat16, device="cuda")
        cache.nomas_kvcache_append(kz[:n * TPF], vz[:n * TPF], n)
        for m, t in hit:
            kz[t - r0].zero_()
            vz[t - r0].zero_()
        f += n
    assert cache.frames_written == cap

    q = torch.zeros((N_TEXT, H * D), dtype=torch.bfloat16, device="cuda")
    for m in range(4):
        q[m, m] = A
    kc = torch.zeros_like(q)
    vc = torch.zeros_like(q)
    lse = torch.empty(H * N_TEXT, dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention(q, kc, vc, 0, N_TEXT, cache, lse=lse)
    torch.cuda.synchronize()
    got, g_lse = host_f64(out).reshape(N_TEXT, D), lse.cpu().numpy().astype(np.float64)

    # the keys and values as the cache holds them
    kb = np.zeros((4, D))
    vb = np.stack([_marker_values(m) for m in range(4)])
    for m in range(4):
        kb[m, m] = B
    if int8:
        kb = quant.dequantise(*quant.quantise(kb))
        vb = quant.dequantise(*quant.quantise(vb))
    n_keys = n_cached + N_TEXT
    ref = np.zeros((N_TEXT, D))
    ref_lse = np.full(N_TEXT, math.log(n_keys))
    for m in range(4):
        logit = A * kb[m, m] / math.sqrt(D)
        w = math.exp(logit)
        ref[m] = (w * vb[m] + vb.sum(0) - vb[m]) / (w + n_keys - 1)
        ref_lse[m] = math.log(w + n_keys - 1)
    ref[4:] = vb.sum(0) / n_keys
    diff = np.abs(got - ref)
    assert diff.max() <= 1e-2 * np.abs(ref).max() and diff.mean() <= 1e-3, (diff.max(), diff.mean())
    assert np.max(np.abs(g_lse - ref_lse)) <= 2.0 ** -8, np.abs(g_lse - ref_lse)


def test_current_rows_just_under_2gib():
    """The current segment's rows read through a row stride that puts their last
    row's bytes just under 2 GiB from the first (16 rows x 67,108,856 elements x
    2 B = 2^31 - 256 B): the strided loads of q, k_cur and v_cur reach the end
    of their 32-bit range. Small cache (the tiny workload); oracle reference."""
    from oracle import attention
    from segment_autoregressive_dit_amd import synth
    from _gpu_util import dev_bf16

    wl = synth.WORKLOADS["tiny"]
    Hh, Dd, nt = wl.n_heads, wl.head_dim, 16
    ld = (2 ** 31 - 1) // (nt * 2) // 8 * 8
    assert nt * ld * 2 < 2 ** 31 and nt * (ld + 8) * 2 >= 2 ** 31
    say(f"limits: {nt} current rows at row stride {ld} ({nt * ld * 2} B)")
    cache = nomas.KVCache(Hh, Dd, wl.tpf, wl.capacity_frames, False)
    kp, vp = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kp), dev_bf16(vp), wl.cached_frames)
    bits = [synth.normal_bf16((nt, Hh, Dd), 77, 0, 0, tid) for tid in range(3)]
    views = []
    for b in bits:
        full = torch.empty((nt, ld), dtype=torch.bfloat16, device="cuda")
        full[:, :Hh * Dd] = dev_bf16(b).reshape(nt, Hh * Dd)
        views.append(full[:, :Hh * Dd])
    lse = torch.empty(Hh * nt, dtype=torch.float32, device="cuda")
    out = nomas.nomas_segment_attention(views[0], views[1], views[2], 0, nt, cache, lse=lse)
    torch.cuda.synchronize()
    got = host_f64(out).reshape(nt, Hh, Dd)
    x = [synth.bf16_bits_to_f64(b) for b in bits]
    ref, ref_lse = attention.segment_attention(x[0], x[1], x[2], synth.bf16_bits_to_f64(kp),
                                               synth.bf16_bits_to_f64(vp), 1.0 / math.sqrt(Dd))
    diff = np.abs(got - ref)
    assert diff.max() <= 1e-2 * np.abs(ref).max() and diff.mean() <= 1e-3, (diff.max(), diff.mean())
    g_lse = lse.cpu().numpy().reshape(Hh, nt)
    assert np.max(np.abs(g_lse - ref_lse)) <= 2.0 ** -8
