"""Seeded synthetic inputs and workload shapes.

This module holds no arithmetic of the method: it only draws random numbers and
states shapes. Both the product tests and the CPU oracle take their inputs from
here, so both sides see bit-identical bfloat16 values.

Every tensor is drawn as float32 N(0, 1) from
``numpy.random.default_rng(SeedSequence([workload_id, layer, turn, tensor_id]))``
and rounded to bfloat16 (round to nearest even). tensor_id: 0/1/2 = current
Q/K/V, 3/4 = pre-fill cache K/V, 5 = choice of outlier channels.

Shapes follow the pages' model: 16 heads x 128 (hidden 2048), 54 double-stream
blocks, 8 denoising steps ("Hy-Nomas auf einer RTX 4090", inferencekey.com,
section "Modell und Dateien"), a window of 18 latent frames ("Das
Single-GPU-Preset"), 8-frame output chunks (blog.authon.dev config excerpt
``output_chunk_frames: 8``).
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed namespace of the workload
    n_heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    capacity_frames: int     # ring capacity (the window)
    cached_frames: int       # frames resident before the measured call
    seg_frames: int          # latent frames in the current segment
    n_text: int
    kv_int8: bool
    rope_split: tuple        # (d_t, d_h, d_w)
    n_layers: int = 1
    n_steps: int = 1
    n_turns: int = 1
    k_outliers: int = 0      # outlier channels per head in K (x20)
    n_splits: int = 1
    theta: float = 10000.0

    @property
    def tpf(self):
        return self.grid_h * self.grid_w

    @property
    def n_video(self):
        return self.seg_frames * self.tpf

    @property
    def n_q(self):
        return self.n_video + self.n_text

    @property
    def n_cached(self):
        return min(self.cached_frames, self.capacity_frames) * self.tpf

    @property
    def n_k(self):
        return self.n_cached + self.n_q

    @property
    def t0(self):
        """First latent frame of the measured segment."""
        return self.cached_frames

    def attention_flop(self):
        """4 * n_q * n_k * D * H: two contractions of 2 flop per multiply-add."""
        return 4 * self.n_q * self.n_k * self.head_dim * self.n_heads


WORKLOADS = {
    # 2 x 64 heads, 4x6 grid, 2 cached segments of 2 frames, 2-frame segment, 16 text
    "tiny": Workload("tiny", 1, 2, 64, 4, 6, 4, 4, 2, 16, False, (16, 24, 24)),
    # one layer, full head shape, bf16 cache of 18 frames, 8-frame segment, 256 text
    "layer_bf16": Workload("layer_bf16", 2, 16, 128, 24, 40, 18, 18, 8, 256, False, (32, 48, 48)),
    # as above with an INT8 cache and 4 outlier K channels per head at 20x
    "layer_int8": Workload("layer_int8", 3, 16, 128, 24, 40, 18, 18, 8, 256, True, (32, 48, 48),
                           k_outliers=4),
    # turn 12 of a session with full history (11 x 8 cached frames), split-KV
    "long_bf16": Workload("long_bf16", 4, 16, 128, 24, 40, 96, 88, 8, 256, False, (32, 48, 48),
                          n_splits=4),
    # 54 layers x 8 steps x 3 turns against an INT8 18-frame window
    "denoise_int8": Workload("denoise_int8", 5, 16, 128, 24, 40, 18, 18, 8, 256, True, (32, 48, 48),
                             n_layers=54, n_steps=8, n_turns=3),
    # tail-handling shape: 22x40 = 880 tokens per frame (1280x704 at 32x), uncounted
    "layer_880": Workload("layer_880", 6, 16, 128, 22, 40, 18, 18, 8, 256, True, (32, 48, 48)),
}


def rng_for(wid, layer, turn, tid):
    return np.random.default_rng(np.random.SeedSequence([int(wid), int(layer), int(turn), int(tid)]))


def _round_bf16_bits(x32):
    """float32 array -> uint16 bfloat16 patterns, round to nearest even (torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def device_normal_bf16(shape, wid, layer, turn, tid, device="cuda"):
    """bf16 CUDA tensor of N(0, 1) float32 draws rounded to nearest even, from
    torch's device generator seeded by (wid, layer, turn, tid).

    For workloads too large to draw on the host in a test's time (the 54-layer
    sweep draws about 12 billion values); the oracle reads the same values back
    from the tensor. Same role as ``normal_bf16``: numbers only, no arithmetic of
    the method."""
    import torch
    seed = int(np.random.SeedSequence([int(wid), int(layer), int(turn), int(tid)]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed >> 1)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def outlier_channels(wl, layer=0):
    """[n_heads, k_outliers] channel indices scaled by 20 in every K row."""
    rng = rng_for(wl.wid, layer, 0, 5)
    return np.stack([rng.choice(wl.head_dim, wl.k_outliers, replace=False)
                     for _ in range(wl.n_heads)]) if wl.k_outliers else None


def normal_bf16(shape, wid, layer, turn, tid, outliers=None, out_scale=20.0, std=1.0):
    """uint16 bf16 patterns of N(0, std^2) draws of ``shape`` = [rows, H, D]."""
    x = rng_for(wid, layer, turn, tid).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outliers is not None:
        for h in range(shape[1]):
            x[:, h, outliers[h]] *= np.float32(out_scale)
    return _round_bf16_bits(x)


def current_qkv(wl, layer=0, turn=0):
    """Current segment's Q, K, V rows [n_q, H, D] (video rows first, then text)."""
    shape = (wl.n_q, wl.n_heads, wl.head_dim)
    outl = outlier_channels(wl, layer)
    q = normal_bf16(shape, wl.wid, layer, turn, 0)
    k = normal_bf16(shape, wl.wid, layer, turn, 1, outliers=outl)
    v = normal_bf16(shape, wl.wid, layer, turn, 2)
    return q, k, v


def prefill_kv(wl, layer=0):
    """Pre-fill video K, V for the cached frames [cached_frames*tpf, H, D]."""
    shape = (wl.cached_frames * wl.tpf, wl.n_heads, wl.head_dim)
    outl = outlier_channels(wl, layer)
    k = normal_bf16(shape, wl.wid, layer, 0, 3, outliers=outl)
    v = normal_bf16(shape, wl.wid, layer, 0, 4)
    return k, v


def bf16_bits_to_f64(u):
    """Values of bf16 patterns (widening only: no rounding happens)."""
    u = np.asarray(u).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def rising_logit_inputs(n_heads, head_dim, n_cached, n_cur, seed, growth_log2=140.0, block=64, mixed=False):
    """Inputs whose attention logits climb steeply along the key order.

    Every query is a per-head sign pattern u (entries +-1) plus N(0, 0.05^2)
    noise. In each run of ``block`` consecutive keys (cache keys first, then the
    current segment's) one key is a_b * u and the others are N(0, 0.05^2) noise,
    with a_b chosen so that this key's logit (scale 1/sqrt(head_dim), log2 units)
    grows by about ``growth_log2`` from one run to the next; the key's place in
    run b is (7b + 3) mod block, so it visits every position class. A running
    softmax maximum that is not raised on some run overflows exp2 at once.
    Values are N(0, 1). With ``mixed``, odd query rows are negated (their
    logits fall along the key order) and run 0 holds one more key, -a_0 * u at
    place 5, so that those rows' largest logit sits in the first run, about
    ``growth_log2`` above everything after it, while the even rows still climb.
    Returns bf16 patterns (q [n_cur,H,D], k_cache, v_cache [n_cached,H,D],
    k_cur, v_cur [n_cur,H,D])."""
    rng = np.random.default_rng(np.random.SeedSequence([9001, seed]))
    H, D = n_heads, head_dim
    u = rng.choice(np.array([-1.0, 1.0], np.float32), size=(H, D))
    q = u[None] + np.float32(0.05) * rng.standard_normal((n_cur, H, D), dtype=np.float32)
    n_k = n_cached + n_cur
    k = np.float32(0.05) * rng.standard_normal((n_k, H, D), dtype=np.float32)
    per_unit = np.sqrt(D) * 1.4426950408889634   # logit of a*u against u, per unit a
    for b in range((n_k + block - 1) // block):
        j = b * block + (7 * b + 3) % block
        if j < n_k:
            k[j] = np.float32(growth_log2 * (b + 1) / per_unit) * u
    if mixed:
        q[1::2] *= np.float32(-1.0)
        if 5 < min(block, n_k):
            k[5] = np.float32(-growth_log2 / per_unit) * u
    v = rng.standard_normal((n_k, H, D), dtype=np.float32)
    kb, vb = _round_bf16_bits(k), _round_bf16_bits(v)
    return _round_bf16_bits(q), kb[:n_cached], vb[:n_cached], kb[n_cached:], vb[n_cached:]
