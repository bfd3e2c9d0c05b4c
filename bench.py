#!/usr/bin/env python3
"""Benchmark of the segment-attention hot path on one MI355X.

A step is one pass of the whole path over one layer's segment at the full head
shape (16 x 128 heads, 24x40 latent grid, 18-frame bf16 window = 17,280 cached
tokens, 8-frame segment = 7,680 video tokens + 256 text tokens):
    nomas_rope3d(Q, K) -> nomas_segment_attention -> nomas_kvcache_append (8 frames,
    evicting the 8 oldest, so every step sees the same 18-frame window).
``value`` = attention FLOP (4 * n_q * n_k * D * H) per step / step time.

Also reported (outside the timed steps):
  * the attention launch alone (HIP events on the launch stream) against the
    bf16 MFMA peak -> ``roofline``;
  * one multi-segment block-causal call at a training shape (4 segments x 7,936
    rows, 18-frame window) -> ``block_causal_tflops``;
  * the evicted-frame archive: 8 INT8 frame records of one layer window to
    pinned host memory and back by the copy engines -> ``archive_d2h_gbps``,
    ``archive_h2d_gbps``;
  * the fused QKV projection + RoPE of the layer (7,936 x 2,048 -> 6,144)
    -> ``qkv_tflops``;
  * one layer's projection + attention (+ append) at the INT8 layer shape,
    unfused and through the fused calls (projection writing V^T and, at the
    final step, the cache; attention reading V^T and the frames before the
    segment) -> ``chain_turn_ms_per_layer_unfused`` / ``_fused``;
  * the layer shape under the sparse policy: selection of 34 of the 135
    candidate blocks + sparse attention -> ``sparse_select_us``,
    ``sparse_attention_ms``;
  * the full denoise sweep: 54 layers x 8 steps x 3 turns of RoPE + attention
    against per-layer INT8 18-frame windows, with the 54 appends after step 8
    of each turn -> ``denoise_ms_per_step`` (median over the 24 steps); and the
    same turns under the sparse policy (steps 1-2 dense, then candidate-block
    selection + attention to 25 % of the blocks) -> ``denoise_sparse_ms_per_step``
    (mean over the 8 steps of a turn, averaged over turns);
  * the attention launch with the caches flushed between reps (512 MB written)
    -> ``attention_cold_ms``; p10/p90 of the timed steps' attention launches;
  * turn 12 of a full-history session (84,480 cached tokens), split-KV with
    n_splits 1, 2, 4, 8 and auto -> ``long_history_ms``, ``long_history_tflops``
    (auto);
  * the fp64 oracle on a bounded sample of query rows -> ``cpu_baseline`` (all the
    BLAS threads), and on one thread over a sample cut by the thread count
    -> ``cpu_baseline.one_thread``.
``--headline-only`` times the single-layer step and nothing else (no clock
sampling either), so a kernel trace of that run holds only the headline's
launches. ``--config 1|3|4|5`` prints one line for that workload alone (tiny,
single-layer INT8, full history, the denoise sweep); 2 is the default line.
Inputs are seeded synthetic N(0,1) bf16 tensors already resident in HBM.
"""

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
H_HIDDEN = 2048                 # DiT hidden size
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attention_layer_bf16_hbm_traffic.json")
ATTN_SRC = os.path.join(ROOT, "segment_autoregressive_dit_amd", "csrc", "attention.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-denoise", action="store_true", help="skip the 54-layer denoise sweep")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--headline-only", action="store_true",
                   help="time the single-layer step only (no extra measurements): a kernel trace of this run "
                        "holds the headline attention launches alone")
    p.add_argument("--cpu-rows", type=int, default=7936, help="query rows per head in the CPU sample")
    p.add_argument("--config", type=int, choices=[1, 2, 3, 4, 5], default=2,
                   help="the workload of the line: 1 tiny (correctness shape), 2 single layer bf16 (default, with "
                        "every extra measurement), 3 single layer INT8 (+ quantise-append), 4 full history "
                        "(split-KV sweep), 5 the 54-layer INT8 denoise sweep")
    return p.parse_args()


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def layer_step_bench(args):
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["layer_bf16"]
    H, D, tpf, F = wl.n_heads, wl.head_dim, wl.tpf, wl.seg_frames
    log(f"[bench] layer step: {wl.n_q} queries x {wl.n_k} keys, {H}x{D} heads, bf16 window {wl.capacity_frames} frames")
    cache = nomas.KVCache(H, D, tpf, wl.capacity_frames, False)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    qb, kb, vb = synth.current_qkv(wl)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    out = torch.empty_like(q)
    ws = nomas.workspace_for(cache, wl.n_video, wl.n_text)
    torch.cuda.synchronize()
    flop = wl.attention_flop()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record()
        nomas.nomas_rope3d(q, k, wl.t0, F, wl.grid_h, wl.grid_w, wl.rope_split, H, D)
        if e: e[1].record()
        nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, workspace=ws)
        if e: e[2].record()
        cache.nomas_kvcache_append(k, v, F)
        if e: e[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the graphics clock under this load: the same attention launches repeated
    # for a few seconds while amd-smi is sampled (the timed steps above last
    # well under the sampling period); not in --headline-only runs, whose kernel
    # trace is to hold the timed steps' launches alone
    clk = ClockSampler()
    if not args.headline_only:
        with clk:
            t_end = time.perf_counter() + 3.0
            while time.perf_counter() < t_end:
                for _ in range(20):
                    nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, workspace=ws)
                torch.cuda.synchronize()
    rope_ms = [e[0].elapsed_time(e[1]) for e in ev]
    attn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    app_ms = [e[2].elapsed_time(e[3]) for e in ev]
    res = dict(
        ms_per_step=wall * 1e3 / args.steps,
        flop=flop,
        attn_ms_mean=statistics.mean(attn_ms),
        attn_ms_median=statistics.median(attn_ms),
        attn_ms_p10=statistics.quantiles(attn_ms, n=10)[0],
        attn_ms_p90=statistics.quantiles(attn_ms, n=10)[-1],
        rope_ms_mean=statistics.mean(rope_ms),
        append_ms_mean=statistics.mean(app_ms),
        sclk_mhz=clk.mhz(),
        sclk_samples=len(clk.samples),
        sclk_raw=None if clk.samples else clk.raw,
        rope_bytes=2 * 2 * wl.n_video * H * D * 2,             # read + write Q and K video rows
        append_bytes=2 * wl.n_video * H * D * 2 * 2,           # bf16 window: read K,V + write K,V
    )
    log(f"[bench] layer step: {res['ms_per_step']:.3f} ms/step, attention {res['attn_ms_mean']:.3f} ms "
        f"({flop / res['attn_ms_mean'] / 1e9:.1f} TFLOP/s)")
    return wl, res


class ClockSampler:
    """Samples the GPU's graphics clock with amd-smi in a background thread
    while a timed region runs (a child process per sample; the GPU work is
    not touched). ``mhz()`` is the median of the samples, or None when the
    tool gives no reading."""

    def __init__(self, period_s=0.2):
        import threading
        self.period_s = period_s
        self.samples = []
        self.raw = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)

    def _read(self):
        import re
        import subprocess
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True, text=True,
                               timeout=10)
        except Exception as e:
            self.raw = self.raw or f"amd-smi failed: {e}"
            return None
        if self.raw is None:
            self.raw = r.stdout[:4000]
        # the graphics clock's current value: the first "gfx" entry's clk value
        m = re.search(r'"gfx_0"\s*:\s*\{[^{}]*?"clk"\s*:\s*\{\s*"value"\s*:\s*(\d+)', r.stdout)
        if not m:
            m = re.search(r'"gfx[^"]*"\s*:\s*\{[^{}]*?"clk"\s*:\s*(\d+)', r.stdout)
        return int(m.group(1)) if m else None

    def _loop(self):
        while not self._stop.is_set():
            v = self._read()
            if v:
                self.samples.append(v)
            self._stop.wait(self.period_s)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)

    def mhz(self):
        return statistics.median(self.samples) if self.samples else None


_SLEEP_CYCLES_PER_MS = None


def time_launches(fn, reps):
    """Mean GPU time (ms) of ``reps`` back-to-back launches of ``fn``. A spin
    kernel holds the GPU for a few ms first, so the host has enqueued the whole
    batch before it starts: the events then bracket GPU work only, not the
    host's launch overhead (which exceeds a short kernel's run time)."""
    import torch
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * (5 + 0.1 * reps)))
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_calls(fn, reps):
    """Median GPU time (ms) of one call of ``fn`` over ``reps`` back-to-back
    calls, HIP events recorded between them on the current stream, for calls
    far longer than the host's launch cost (the timed step's own method)."""
    import torch
    for _ in range(3):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return statistics.median(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))


def layer_int8_bench(reps=20):
    """The single-layer shape with an INT8 window (16x128 heads, 18 frames of
    24x40, 4 outlier key channels per head at 20x): the attention call (median
    of back-to-back calls, HIP events between them) and the quantise-append of
    the 8-frame segment (batches behind a spin kernel), each on its own."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["layer_int8"]
    H, D, F = wl.n_heads, wl.head_dim, wl.seg_frames
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, True)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    out = torch.empty_like(q)
    ws = nomas.workspace_for(cache, wl.n_video, wl.n_text)
    attn = lambda: nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, workspace=ws)
    app = lambda: cache.nomas_kvcache_append(k, v, F)
    # attention as in the timed step (a call lasts ~1.5 ms, far beyond the
    # host's launch cost); the short append in batches behind a spin kernel
    res = {"attention": time_calls(attn, reps), "append": time_launches(app, 5 * reps)}
    flop = wl.attention_flop()
    # read K, V bf16 + write K, V codes + one fp32 scale per (token, head) each
    app_bytes = 2 * wl.n_video * H * D * 2 + 2 * wl.n_video * H * D + 2 * wl.n_video * H * 4
    log(f"[bench] INT8 layer: attention {res['attention']:.3f} ms ({flop / res['attention'] / 1e9:.1f} TFLOP/s), "
        f"quantise-append {res['append'] * 1e3:.1f} us ({app_bytes / res['append'] / 1e6:.0f} GB/s)")
    return dict(int8_attention_ms=round(res["attention"], 4),
                int8_attention_tflops=round(flop / res["attention"] / 1e9, 1),
                int8_attention_pct_mfma_peak=round(100 * flop / res["attention"] / 1e9 / PEAK_BF16_TFLOPS, 2),
                int8_append_us=round(res["append"] * 1e3, 2),
                int8_append_gbps=round(app_bytes / res["append"] / 1e6, 1),
                int8_append_bytes=app_bytes)


def attention_cold_bench(reps=20):
    """The layer-shape attention launch with the caches flushed before each rep:
    512 MB (twice the MALL) written between reps, so K/V come from HBM."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["layer_bf16"]
    H, D = wl.n_heads, wl.head_dim
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, False)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    out = torch.empty_like(q)
    ws = nomas.workspace_for(cache, wl.n_video, wl.n_text)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, workspace=ws)
    ms = []
    for i in range(reps):
        flush.fill_(i & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = statistics.median(ms)
    log(f"[bench] attention, caches flushed: {med:.3f} ms ({wl.attention_flop() / med / 1e9:.1f} TFLOP/s)")
    return dict(attention_cold_ms=round(med, 4), attention_cold_tflops=round(wl.attention_flop() / med / 1e9, 1))


def long_history_bench(reps=10):
    """Turn 12 of a session with full history: 84,480 cached tokens (88 frames) +
    7,936 current rows, 16x128 heads, bf16; split-KV with n_splits in
    {1, 2, 4, 8, auto}."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["long_bf16"]
    H, D = wl.n_heads, wl.head_dim
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, False)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    del kb, vb
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    out = torch.empty_like(q)
    flop = wl.attention_flop()
    res = {}
    for splits in (1, 2, 4, 8, 0):
        ws = nomas.workspace_for(cache, wl.n_video, wl.n_text, splits)
        for _ in range(2):
            nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, n_splits=splits, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, n_splits=splits, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[splits] = ms
        del ws
    best = min(res, key=res.get)
    log("[bench] long history: " + ", ".join(f"splits {s or 'auto'} {m:.3f} ms" for s, m in res.items()))
    return dict(long_history_ms={str(s or "auto"): round(m, 4) for s, m in res.items()},
                long_history_tflops=round(flop / res[0] / 1e9, 1),
                long_history_best_tflops=round(flop / res[best] / 1e9, 1))


def head_share_bench(reps=20):
    """One GPU's share of the layer shape when the 16 heads are spread over 8
    GPUs: 2 heads at the full sequence lengths (7,936 queries x 25,216 keys,
    bf16 window). The 2 x 31 query-tile blocks alone fill a quarter of the
    chip, so the automatic plan splits the keys; both are timed."""
    import dataclasses
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = dataclasses.replace(synth.WORKLOADS["layer_bf16"], n_heads=2)
    H, D = wl.n_heads, wl.head_dim
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, False)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    out = torch.empty_like(q)
    flop = wl.attention_flop()
    res = {}
    for splits in (1, 0):
        ws = nomas.workspace_for(cache, wl.n_video, wl.n_text, splits)
        res[splits] = time_calls(lambda: nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out,
                                                                       n_splits=splits, workspace=ws), reps)
    auto = nomas.nomas_segment_attention_splits(wl.n_video, wl.n_text, cache.n_cached, H, D, 0, 0)
    log(f"[bench] 2-head share: splits 1 {res[1]:.3f} ms, auto ({auto}) {res[0]:.3f} ms "
        f"({flop / res[0] / 1e9:.1f} TFLOP/s)")
    return dict(head_share_2_ms={"1": round(res[1], 4), "auto": round(res[0], 4)}, head_share_2_auto_splits=auto,
                head_share_2_tflops=round(flop / res[0] / 1e9, 1),
                head_share_2_pct_mfma_peak=round(100 * flop / res[0] / 1e9 / PEAK_BF16_TFLOPS, 2))


def denoise_bench(n_turns=3):
    """54 layers x 8 Euler steps x n_turns against INT8 18-frame windows."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["denoise_int8"]
    H, D, tpf, F = wl.n_heads, wl.head_dim, wl.tpf, wl.seg_frames
    L, S = wl.n_layers, wl.n_steps
    log(f"[bench] denoise sweep: {L} layers x {S} steps x {n_turns} turns, INT8 window {wl.capacity_frames} frames")
    g = torch.Generator(device="cuda")

    def randn(shape, seed):
        g.manual_seed(seed)
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    caches, ws = [], None
    for layer in range(L):
        c = nomas.KVCache(H, D, tpf, wl.capacity_frames, True)
        n = wl.cached_frames * tpf
        c.nomas_kvcache_append(randn((n, H, D), 1000 * layer + 3), randn((n, H, D), 1000 * layer + 4),
                               wl.cached_frames)
        caches.append(c)
    ws = nomas.workspace_for(caches[0], wl.n_video, wl.n_text)
    out = torch.empty((wl.n_q, H, D), dtype=torch.bfloat16, device="cuda")
    # sparse policy: dense for steps 1-2, then 25 % of the candidate blocks
    n_sel = (nomas.nomas_sparse_candidates(caches[0].n_cached) + 3) // 4
    nqb = (wl.n_q + nomas.NOMAS_SPARSE_QUERY_BLOCK - 1) // nomas.NOMAS_SPARSE_QUERY_BLOCK
    lists = torch.empty((H, nqb, n_sel), dtype=torch.int32, device="cuda")
    ws_sel = torch.empty(nomas.lib().nomas_sparse_select_workspace_bytes(wl.n_q, caches[0].n_cached, H, D),
                         dtype=torch.uint8, device="cuda")
    step_ms, append_ms, sparse_ms = [], [], []
    for turn in range(n_turns):
        qkv = [tuple(randn((wl.n_q, H, D), 1000 * layer + 100 * (turn + 1) + t) for t in range(3))
               for layer in range(L)]
        t0 = wl.cached_frames + F * turn
        torch.cuda.synchronize()
        for s in range(S):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for layer in range(L):
                q, k, v = qkv[layer]
                nomas.nomas_rope3d(q, k, t0, F, wl.grid_h, wl.grid_w, wl.rope_split, H, D)
                nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, caches[layer], out=out, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            step_ms.append(e0.elapsed_time(e1))
        # the same turn under the sparse policy (RoPE is in place, so the sparse
        # pass sees Q/K rotated once more than the dense one: same cost)
        for s in range(S):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for layer in range(L):
                q, k, v = qkv[layer]
                nomas.nomas_rope3d(q, k, t0, F, wl.grid_h, wl.grid_w, wl.rope_split, H, D)
                if s < 2:
                    nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, caches[layer], out=out,
                                                  workspace=ws)
                else:
                    nomas.nomas_sparse_select(q, wl.n_q, caches[layer], n_sel, block_list=lists, workspace=ws_sel)
                    nomas.nomas_segment_attention_sparse(q, k, v, wl.n_video, wl.n_text, caches[layer], lists,
                                                         out=out, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            sparse_ms.append(e0.elapsed_time(e1))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for layer in range(L):
            caches[layer].nomas_kvcache_append(qkv[layer][1], qkv[layer][2], F)
        e1.record()
        torch.cuda.synchronize()
        append_ms.append(e0.elapsed_time(e1))
        log(f"[bench] denoise turn {turn + 1}: median step {statistics.median(step_ms[-S:]):.2f} ms, sparse policy "
            f"{statistics.mean(sparse_ms[-S:]):.2f} ms/step on average, appends {append_ms[-1]:.2f} ms")
        del qkv
    flop_step = L * wl.attention_flop()
    med = statistics.median(step_ms)
    return dict(denoise_ms_per_step=med, denoise_tflops=flop_step / med / 1e9,
                denoise_sparse_ms_per_step=statistics.mean(sparse_ms), denoise_sparse_n_select=n_sel,
                denoise_append_ms_per_turn=statistics.mean(append_ms),
                denoise_int8_append_bytes_per_layer=2 * wl.n_video * H * D * 2 + 2 * wl.n_video * H * D
                + 2 * wl.n_video * H * 4)


def sparse_layer_bench(reps=20):
    """The single-layer bf16 shape under the sparse policy: candidate-block
    selection (34 of the 135 blocks of 128 cached rows, 25 %) + sparse attention."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["layer_bf16"]
    H, D = wl.n_heads, wl.head_dim
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, False)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
    out = torch.empty_like(q)
    nc = nomas.nomas_sparse_candidates(cache.n_cached)
    n_sel = (nc + 3) // 4
    nqb = (wl.n_q + nomas.NOMAS_SPARSE_QUERY_BLOCK - 1) // nomas.NOMAS_SPARSE_QUERY_BLOCK
    lists = torch.empty((H, nqb, n_sel), dtype=torch.int32, device="cuda")
    ws_sel = torch.empty(nomas.lib().nomas_sparse_select_workspace_bytes(wl.n_q, cache.n_cached, H, D),
                         dtype=torch.uint8, device="cuda")
    ws = torch.empty(nomas.nomas_segment_attention_workspace_bytes(wl.n_video, wl.n_text, n_sel * 128, H, D, 0),
                     dtype=torch.uint8, device="cuda")
    sel = lambda: nomas.nomas_sparse_select(q, wl.n_q, cache, n_sel, block_list=lists, workspace=ws_sel)
    att = lambda: nomas.nomas_segment_attention_sparse(q, k, v, wl.n_video, wl.n_text, cache, lists, out=out,
                                                       workspace=ws)
    times = {"select": time_launches(sel, reps), "attention": time_calls(att, reps)}
    flop = 4 * wl.n_q * (n_sel * 128 + wl.n_q) * D * H
    log(f"[bench] sparse layer: select {times['select'] * 1e3:.1f} us, attention {times['attention']:.3f} ms "
        f"({flop / times['attention'] / 1e9:.1f} TFLOP/s on the kept keys)")
    return dict(sparse_select_us=round(times["select"] * 1e3, 2), sparse_attention_ms=round(times["attention"], 4),
                sparse_attention_tflops=round(flop / times["attention"] / 1e9, 1), sparse_n_select=n_sel)


def qkv_bench(reps=20):
    """The QKV projection of one layer at the single-layer shape with the RoPE
    epilogue: 7,936 rows x hidden 2,048 -> 3 x 16 x 128 channels."""
    import numpy as np
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["layer_bf16"]
    H, D, hidden = wl.n_heads, wl.head_dim, H_HIDDEN
    x = dev_bf16(synth.normal_bf16((wl.n_q, 1, hidden), 79, 0, 0, 0)[:, 0])
    w = torch.randn((3 * H * D, hidden), device="cuda", dtype=torch.float32).div_(math.sqrt(hidden)).to(torch.bfloat16)
    y = torch.empty((wl.n_q, 3 * H * D), dtype=torch.bfloat16, device="cuda")
    table = nomas.nomas_rope3d_table(D, wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split)
    fn = lambda: nomas.nomas_qkv_projection(x, w, H, D, n_video=wl.n_video, rope_table=table, qkv=y)
    # the first batch of a ~0.2 ms kernel in a process runs ~10 % slow while the
    # clock ramps up: 30 untimed calls first
    for _ in range(30):
        fn()
    ms = time_calls(fn, reps)
    flop = 2 * wl.n_q * hidden * 3 * H * D
    log(f"[bench] qkv projection + RoPE: {ms * 1e3:.1f} us, {flop / ms / 1e9:.1f} TFLOP/s")
    return dict(qkv_us=round(ms * 1e3, 2), qkv_tflops=round(flop / ms / 1e9, 1))


def fused_chain_bench(reps=10):
    """One layer's QKV projection + attention (+ the segment's append at the
    final step) at the INT8 layer shape (16x128 heads, 18-frame window of 24x40,
    8-frame segment + 256 text, hidden 2,048), unfused and fused. Unfused: the
    projection, attention on its views (values transposed inside the call), and
    at the final step the quantise-append. Fused: the projection also writes
    V^T (nomas_qkv_projection_vt; at the final step nomas_qkv_projection_append,
    which also writes the segment into a cache of 18 + 8 frames) and attention
    reads V^T and the 18 frames before the segment
    (nomas_segment_attention_frames). A turn is 7 steps + the final one."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["layer_int8"]
    H, D, F, W, hidden = wl.n_heads, wl.head_dim, wl.seg_frames, wl.capacity_frames, H_HIDDEN
    nv, nt, n = wl.n_video, wl.n_text, wl.n_q
    kb, vb = synth.prefill_kv(wl)
    plain = nomas.KVCache(H, D, wl.tpf, W, True)
    plain.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    roomy = nomas.KVCache(H, D, wl.tpf, W + F, True)
    roomy.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
    x = dev_bf16(synth.normal_bf16((n, 1, hidden), 79, 1, 0, 0)[:, 0])
    w = torch.randn((3 * H * D, hidden), device="cuda", dtype=torch.float32).div_(math.sqrt(hidden)).to(torch.bfloat16)
    table = nomas.nomas_rope3d_table(D, wl.t0, F, wl.grid_h, wl.grid_w, wl.rope_split)
    y = torch.empty((n, 3 * H * D), dtype=torch.bfloat16, device="cuda")
    vt = nomas.new_vt(n, H, D)
    out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    q, k, v = (y[:, i * H * D:(i + 1) * H * D] for i in range(3))
    ws = nomas.workspace_for(plain, nv, nt)

    def unfused(final):
        nomas.nomas_qkv_projection(x, w, H, D, n_video=nv, rope_table=table, qkv=y)
        nomas.nomas_segment_attention(q, k, v, nv, nt, plain, out=out, workspace=ws)
        if final:
            plain.nomas_kvcache_append(k, v, F)

    def fused(final):
        if final:
            nomas.nomas_qkv_projection_append(x, w, H, D, nv, table, roomy, qkv=y, v_t=vt)
            first = roomy.frames_written - F - W
        else:
            nomas.nomas_qkv_projection_vt(x, w, H, D, nv, table, vt, qkv=y)
            first = roomy.frames_written - W
        nomas.nomas_segment_attention_frames(q, k, None, nv, nt, roomy, first, W, v_t=vt, out=out, workspace=ws)

    t = {}
    for name, fn in (("unfused_step", lambda: unfused(False)), ("unfused_final", lambda: unfused(True)),
                     ("fused_step", lambda: fused(False)), ("fused_final", lambda: fused(True))):
        t[name] = time_calls(fn, reps)
    t["qkv_vt"] = time_calls(lambda: nomas.nomas_qkv_projection_vt(x, w, H, D, nv, table, vt, qkv=y), reps)
    turn_u = 7 * t["unfused_step"] + t["unfused_final"]
    turn_f = 7 * t["fused_step"] + t["fused_final"]
    log(f"[bench] fused chain (INT8 layer): step {t['unfused_step']:.3f} -> {t['fused_step']:.3f} ms, final step "
        f"{t['unfused_final']:.3f} -> {t['fused_final']:.3f} ms, turn per layer {turn_u:.3f} -> {turn_f:.3f} ms; "
        f"projection with V^T {t['qkv_vt'] * 1e3:.1f} us")
    return dict(chain_step_ms_unfused=round(t["unfused_step"], 4), chain_step_ms_fused=round(t["fused_step"], 4),
                chain_final_ms_unfused=round(t["unfused_final"], 4), chain_final_ms_fused=round(t["fused_final"], 4),
                chain_turn_ms_per_layer_unfused=round(turn_u, 4), chain_turn_ms_per_layer_fused=round(turn_f, 4),
                qkv_vt_us=round(t["qkv_vt"] * 1e3, 2))


def archive_bench(reps=10):
    """Host archive of evicted frames: one INT8 layer window (18 frames of the
    24x40 grid, 16x128 heads); the 8 frames a segment evicts are exported to
    pinned host memory, and restored back, by the copy engines."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    wl = synth.WORKLOADS["denoise_int8"]
    H, D, tpf, F = wl.n_heads, wl.head_dim, wl.tpf, wl.seg_frames
    cache = nomas.KVCache(H, D, tpf, wl.capacity_frames, True)
    n = wl.cached_frames * tpf
    cache.nomas_kvcache_append(dev_bf16(synth.normal_bf16((n, H, D), 78, 0, 0, 3)),
                               dev_bf16(synth.normal_bf16((n, H, D), 78, 0, 0, 4)), wl.cached_frames)
    host = cache.host_records(F)
    rec = cache.nomas_kvcache_record_bytes()
    first = cache.frames_written - cache.valid_frames
    res = {}
    for name, fn in (("d2h", lambda: cache.nomas_kvcache_export_frames(first, F, host)),
                     ("h2d", lambda: cache.nomas_kvcache_restore_frames(host, F))):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / reps
        res[name] = F * rec / dt / 1e9
    log(f"[bench] archive: {F} frames x {rec / 1e6:.2f} MB records, D2H {res['d2h']:.1f} GB/s, "
        f"H2D {res['h2d']:.1f} GB/s")
    return dict(archive_record_mb=round(rec / 1e6, 3), archive_d2h_gbps=round(res["d2h"], 1),
                archive_h2d_gbps=round(res["h2d"], 1))


def block_causal_bench(reps=20):
    """Multi-segment call at a training shape: 4 segments of 8 frames on the
    24x40 grid + 256 text rows each (31,744 rows), 16x128 heads, 18-frame window."""
    import torch
    from segment_autoregressive_dit_amd import nomas, synth

    H, D, tpf, F, T, W = 16, 128, 960, 8, 256, 18
    segments = [(F * tpf, T, F * s) for s in range(4)]
    n = sum(nv + nt for nv, nt, _ in segments)
    q, k, v = (dev_bf16(synth.normal_bf16((n, H, D), 77, 0, 0, t)) for t in range(3))
    out = torch.empty_like(q)
    nb = nomas.nomas_block_causal_attention_workspace_bytes(segments, tpf, H, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    # visible keys per query segment: its own rows + earlier video frames >= t0 - W
    flop = 0
    for i, (nv, nt, t0) in enumerate(segments):
        keys = nv + nt + sum(tpf * sum(1 for f in range(t0p, t0p + nvp // tpf) if f >= t0 - W)
                             for nvp, _, t0p in segments[:i])
        flop += 4 * (nv + nt) * keys * D * H
    call = lambda: nomas.nomas_block_causal_attention(q, k, v, segments, tpf, W, H, D, out=out, workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    log(f"[bench] block-causal 4-segment call: {ms:.3f} ms, {flop / ms / 1e9:.1f} TFLOP/s")
    return dict(block_causal_ms=round(ms, 4), block_causal_tflops=round(flop / ms / 1e9, 1),
                block_causal_flop=flop)


def cpu_baseline(rows_per_head):
    """The fp64 oracle (as it stands) on a bounded sample of the layer workload."""
    import numpy as np
    from oracle import attention
    from segment_autoregressive_dit_amd import synth
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = cores
    wl = synth.WORKLOADS["layer_bf16"]
    q, k, v = (synth.bf16_bits_to_f64(t) for t in synth.current_qkv(wl))
    kp, vp = (synth.bf16_bits_to_f64(t) for t in synth.prefill_kv(wl))
    rows = np.linspace(0, wl.n_q - 1, rows_per_head).astype(int)
    t0 = time.perf_counter()
    attention.segment_attention(q[rows], k, v, kp, vp, 1.0 / math.sqrt(wl.head_dim))
    dt = time.perf_counter() - t0
    flop = 4 * len(rows) * wl.n_k * wl.head_dim * wl.n_heads
    log(f"[bench] cpu oracle: {len(rows)} rows x {wl.n_heads} heads in {dt:.2f} s")
    full_call_s = dt * wl.n_q / len(rows)
    dn = synth.WORKLOADS["denoise_int8"]
    calls = dn.n_layers * dn.n_steps * dn.n_turns
    out = dict(value=flop / dt / 1e12, unit="TFLOP/s", cores=cores, blas_threads=threads, kind="oracle",
               sample=f"{len(rows)} of {wl.n_q} query rows per head, all {wl.n_heads} heads, all {wl.n_k} keys "
                      f"({flop / 1e9:.1f} GFLOP in {dt:.1f} s, float64 numpy)",
               # the denoise sweep's attention calls have the layer call's shape
               # (its INT8 window enters the oracle as float64 values)
               denoise_sweep_s=round(full_call_s * calls, 1),
               denoise_sweep_kind=f"extrapolation: one layer call ({full_call_s:.2f} s) x {calls} calls "
                                  f"({dn.n_layers} layers x {dn.n_steps} steps x {dn.n_turns} turns), not a run")
    # the same oracle on one thread, on a sample cut by the thread count
    try:
        from threadpoolctl import threadpool_limits
        rows1 = rows[::max(1, threads)]
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            attention.segment_attention(q[rows1], k, v, kp, vp, 1.0 / math.sqrt(wl.head_dim))
            dt1 = time.perf_counter() - t0
        flop1 = 4 * len(rows1) * wl.n_k * wl.head_dim * wl.n_heads
        log(f"[bench] cpu oracle, 1 thread: {len(rows1)} rows x {wl.n_heads} heads in {dt1:.2f} s")
        out["one_thread"] = dict(value=flop1 / dt1 / 1e12, unit="TFLOP/s", cores=1,
                                 sample=f"{len(rows1)} query rows per head ({flop1 / 1e9:.1f} GFLOP in {dt1:.1f} s)")
    except Exception as e:   # threadpoolctl missing: report the all-core figure only
        log(f"[bench] cpu oracle, 1 thread: not measured ({e})")
    return out


def traffic_per_launch():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    or None when the summary is missing or the kernel source changed since."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
        from segment_autoregressive_dit_amd.profile_workload import source_digest
        if s.get("source_digest") != source_digest(ATTN_SRC):
            return None
        return s["hbm_bytes_per_launch"]
    except Exception:
        return None


def single_config(args):
    """One JSON line for workload 1, 3, 4 or 5 alone (no roofline or CPU
    baseline objects: those belong to the default line)."""
    from segment_autoregressive_dit_amd import nomas, synth
    import torch
    line = {"metric": "segment-attention TFLOP/s + % MFMA peak; ms per denoise step (54 blocks)", "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if args.config == 1:
        wl = synth.WORKLOADS["tiny"]
        cache = nomas.KVCache(wl.n_heads, wl.head_dim, wl.tpf, wl.capacity_frames, False)
        kb, vb = synth.prefill_kv(wl)
        cache.nomas_kvcache_append(dev_bf16(kb), dev_bf16(vb), wl.cached_frames)
        q, k, v = (dev_bf16(t) for t in synth.current_qkv(wl))
        out = torch.empty_like(q)
        ms = time_launches(lambda: nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out),
                           args.steps)
        value, ms_step = wl.attention_flop() / ms / 1e9, ms
        line["config"] = {"workload": "tiny: 2x64 heads, 4x6 grid, 4 cached frames, 2-frame segment + 16 text "
                                      "(a correctness shape; its time is launch-bound)"}
        extra = {"attention_ms": round(ms, 5)}
    elif args.config == 3:
        extra = layer_int8_bench(reps=args.steps)
        value, ms_step = extra["int8_attention_tflops"], extra["int8_attention_ms"]
        line["config"] = {"workload": "single layer, INT8 window: 16x128 heads, 24x40 grid, 18 frames, 8-frame "
                                      "segment + 256 text; 4 outlier key channels per head at 20x"}
    elif args.config == 4:
        extra = long_history_bench(reps=args.steps)
        value, ms_step = extra["long_history_tflops"], extra["long_history_ms"]["auto"]
        line["config"] = {"workload": "full history, bf16: 84,480 cached tokens (88 frames) + 7,936 queries, "
                                      "16x128 heads, automatic split-KV"}
    else:
        d = denoise_bench()
        value, ms_step = d["denoise_tflops"], d["denoise_ms_per_step"]
        extra = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}
        line["config"] = {"workload": "denoise sweep: 54 layers x 8 steps x 3 turns of RoPE + attention against "
                                      "INT8 18-frame windows, 54 appends per turn; ms_per_step = median step"}
    line.update(value=round(value, 2), ms_per_step=round(ms_step, 4), extra=extra)
    line["config"]["parallelism"] = "single GPU"
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path runs on a single "
              f"MI355X and has no multi-GPU sharding.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from segment_autoregressive_dit_amd import nomas
    nomas.lib()
    if args.config != 2:
        single_config(args)
        return

    wl, r = layer_step_bench(args)
    value = r["flop"] / (r["ms_per_step"] * 1e-3) / 1e12
    # roofline: the median attention launch of the timed steps
    attn_tflops = r["flop"] / (r["attn_ms_median"] * 1e-3) / 1e12
    extra = dict(
        attention_ms=round(r["attn_ms_median"], 4),
        attention_ms_mean=round(r["attn_ms_mean"], 4),
        attention_tflops=round(attn_tflops, 1),
        attention_pct_mfma_peak=round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        sclk_mhz_under_attention=r["sclk_mhz"],
        sclk_samples=r["sclk_samples"],
        rope_us=round(r["rope_ms_mean"] * 1e3, 2),
        rope_gbps=round(r["rope_bytes"] / (r["rope_ms_mean"] * 1e-3) / 1e9, 1),
        append_us=round(r["append_ms_mean"] * 1e3, 2),
        append_gbps=round(r["append_bytes"] / (r["append_ms_mean"] * 1e-3) / 1e9, 1),
        attention_ms_p10=round(r["attn_ms_p10"], 4),
        attention_ms_p90=round(r["attn_ms_p90"], 4),
    )
    if r["sclk_raw"] is not None:
        extra["sclk_raw"] = r["sclk_raw"][:400]
    if not args.headline_only:
        extra.update(layer_int8_bench())
        extra.update(attention_cold_bench())
        extra.update(long_history_bench())
        extra.update(head_share_bench())
    if not args.no_denoise and not args.headline_only:
        d = denoise_bench()
        extra.update(denoise_sparse_ms_per_step=round(d["denoise_sparse_ms_per_step"], 3),
                     denoise_sparse_n_select=d["denoise_sparse_n_select"])
        extra.update(denoise_ms_per_step=round(d["denoise_ms_per_step"], 3),
                     denoise_attention_tflops=round(d["denoise_tflops"], 1),
                     denoise_append_ms_per_turn=round(d["denoise_append_ms_per_turn"], 3))
    if not args.headline_only:
        extra.update(block_causal_bench())
        extra.update(sparse_layer_bench())
        extra.update(archive_bench())
        extra.update(qkv_bench())
        extra.update(fused_chain_bench())
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_rows)
    line = {
        "metric": "segment-attention TFLOP/s + % MFMA peak; ms per denoise step (54 blocks)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "single layer, full head shape, bf16 window: 16x128 heads, 24x40 latent grid, "
                               "18-frame window (17,280 cached tokens), 8-frame segment (7,680 video) + 256 text; "
                               "step = rope3d + segment attention + cache append",
                   "n_q": wl.n_q, "n_k": wl.n_k, "heads": wl.n_heads, "head_dim": wl.head_dim,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_per_launch()},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
