"""Parity of the full denoise sweep at its real shape: 54 layers, each with its
own INT8 ring window of 18 latent frames of 24x40 tokens, 16x128 heads, 8 Euler
steps per turn, 3 turns. The windows start pre-filled with 18 frames (their keys
rotated at frames 0..17), so every turn attends 17,280 cached tokens and every
append evicts 8 frames. A step runs, for each layer, the 3D RoPE of the
segment's queries and keys, then the segment attention; after step 8 the
segment's 8 frames (7,680 rows) are appended to every layer's window.

Pages: 54 double-stream blocks, 8 denoising steps, hidden 2,048 = 16 x 128, 3D
RoPE ("Hy-Nomas auf einer RTX 4090", section "Modell und Dateien"); INT8 KV and
an 18-latent-frame window (same page, section "Das Single-GPU-Preset").

Each stage is checked on the inputs it actually received:
* every one of the 162 appends (54 layers x 3 turns): the 8 written frames'
  codes and scales bit-exact against oracle/quant.py of the bf16 K (as the RoPE
  kernel rotated it) and V that the append read, at the slots oracle/ring.py
  assigns them; every other slot unchanged; frames_written as the ring model's;
* layers 0, 26 and 53 at steps 1 and 8 of every turn: the attention output of
  every query row of every head, and its log-sum-exp, against
  oracle/attention.py (max|diff| <= 1e-2 max|ref|, mean|diff| <= 1e-3), the
  cache entering as the ring model's dequantised frames; steps 1 and 8 see the
  same inputs, so their outputs must also be bitwise equal;
* the same layers' RoPE output against oracle/rope.py (the bound of
  test_gpu_rope.py).
Inputs are per-layer seeded N(0, 1) draws (synth.device_normal_bf16)."""

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import attention, formats, quant, rope
from oracle.ring import RingModel
from segment_autoregressive_dit_amd import nomas, synth

from _gpu_util import host_f64, say
from test_gpu_rope import _bound as rope_bound

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["denoise_int8"]
CHECK_LAYERS = (0, 26, 53)
CHECK_STEPS = (1, 8)
LSE_TOL = 2.0 ** -8


def _codes(t):
    """uint8 device tensor of INT8 codes -> int8 numpy array."""
    return t.cpu().numpy().view(np.int8)


def _frames_of(qs, tpf, n):
    """Split per-row quantiser output (qk, sk, qv, sv) into n frame payloads."""
    return [tuple(a[f * tpf:(f + 1) * tpf] for a in qs) for f in range(n)]


class Sweep:
    def __init__(self):
        self.H, self.D, self.tpf = WL.n_heads, WL.head_dim, WL.tpf
        self.cap, self.F = WL.capacity_frames, WL.seg_frames
        self.nv, self.nt, self.nq = WL.n_video, WL.n_text, WL.n_q
        self.pool = ThreadPoolExecutor(8)
        self.caches, self.rings = [], []
        self.turns_done = 0
        H, D, tpf = self.H, self.D, self.tpf
        for layer in range(WL.n_layers):
            say(f"denoise: pre-fill layer {layer}")
            c = nomas.KVCache(H, D, tpf, self.cap, True)
            n = WL.cached_frames * tpf
            k = synth.device_normal_bf16((n, H, D), WL.wid, layer, 0, 3)
            v = synth.device_normal_bf16((n, H, D), WL.wid, layer, 0, 4)
            nomas.nomas_rope3d(k, None, 0, WL.cached_frames, WL.grid_h, WL.grid_w, WL.rope_split, H, D)
            c.nomas_kvcache_append(k, v, WL.cached_frames)
            ring = RingModel(self.cap)
            if layer in CHECK_LAYERS:
                qs = self._quantise(k, v)
                ring.append(_frames_of(qs, tpf, WL.cached_frames))
                self._check_slots(c, ring, range(WL.cached_frames), f"pre-fill layer {layer}")
            else:
                ring.append([None] * WL.cached_frames)
            self.caches.append(c)
            self.rings.append(ring)
        torch.cuda.synchronize()

    def _quantise(self, k, v):
        xk, xv = host_f64(k), host_f64(v)
        (qk, sk), (qv, sv) = self.pool.map(quant.quantise, (xk, xv))
        return qk, sk, qv, sv

    def _check_slots(self, cache, ring, frames, what):
        """The given absolute frames hold the ring model's payloads, bit for bit."""
        H, D, P, tpf = self.H, self.D, cache.token_pitch, self.tpf
        slots = ring.expected_slots()
        for slot, (f, p) in sorted(slots.items()):
            if f not in frames:
                continue
            sl = slice(slot * tpf, (slot + 1) * tpf)
            kc = _codes(cache.k.view(H, P, D)[:, sl]).transpose(1, 0, 2)
            vc = _codes(cache.v.view(H, D, P)[:, :, sl]).transpose(2, 0, 1)
            ks = cache.k_scale.view(H, P)[:, sl].cpu().numpy().T
            vs = cache.v_scale.view(H, P)[:, sl].cpu().numpy().T
            qk, sk, qv, sv = p
            assert np.array_equal(kc, qk), f"{what}: K codes differ in slot {slot} (frame {f})"
            assert np.array_equal(vc, qv), f"{what}: V codes differ in slot {slot} (frame {f})"
            assert np.array_equal(ks.view(np.uint32), sk.view(np.uint32)), f"{what}: K scales differ in slot {slot}"
            assert np.array_equal(vs.view(np.uint32), sv.view(np.uint32)), f"{what}: V scales differ in slot {slot}"

    def run_turn(self, u):
        """Turn u (1-based): 8 steps over the 54 layers, then the appends."""
        while self.turns_done < u - 1:
            self.run_turn(self.turns_done + 1)
        if self.turns_done >= u:
            return
        H, D, F, nv, nt, nq, tpf = self.H, self.D, self.F, self.nv, self.nt, self.nq, self.tpf
        t0 = WL.cached_frames + F * (u - 1)
        scale = 1.0 / math.sqrt(D)
        say(f"denoise turn {u}: inputs, t0 = {t0}")
        pristine = [tuple(synth.device_normal_bf16((nq, H, D), WL.wid, layer, u, tid) for tid in range(3))
                    for layer in range(WL.n_layers)]
        q = torch.empty((nq, H, D), dtype=torch.bfloat16, device="cuda")
        k = torch.empty_like(q)
        out = torch.empty_like(q)
        lse = torch.empty(H * nq, dtype=torch.float32, device="cuda")
        ws = nomas.workspace_for(self.caches[0], nv, nt)
        saved, rotated, k_final = {}, {}, []
        for s in range(1, WL.n_steps + 1):
            say(f"denoise turn {u} step {s}: 54 x (rope3d + segment attention)")
            for layer in range(WL.n_layers):
                q0, k0, v0 = pristine[layer]
                q.copy_(q0)
                k.copy_(k0)
                nomas.nomas_rope3d(q, k, t0, F, WL.grid_h, WL.grid_w, WL.rope_split, H, D)
                nomas.nomas_segment_attention(q, k, v0, nv, nt, self.caches[layer], out=out, lse=lse, workspace=ws)
                if layer in CHECK_LAYERS and s in CHECK_STEPS:
                    saved[(layer, s)] = (out.clone(), lse.clone())
                if layer in CHECK_LAYERS and s == 1:
                    rotated[layer] = (q.clone(), k.clone())
                if s == WL.n_steps:
                    k_final.append(k.clone())
            torch.cuda.synchronize()

        # attention of the checked layers, against the windows as they stood
        for layer in CHECK_LAYERS:
            o1, l1 = saved[(layer, 1)]
            o8, l8 = saved[(layer, 8)]
            assert torch.equal(o1, o8) and torch.equal(l1, l8), f"layer {layer}: steps 1 and 8 differ"
            gq, gk = rotated[layer]
            x0 = [host_f64(t) for t in pristine[layer]]
            for name, x, got in (("q", x0[0], host_f64(gq)), ("k", x0[1], host_f64(gk))):
                assert np.array_equal(got[nv:], x[nv:]), f"layer {layer}: text rows of {name} changed"
                ref = rope.rope3d_segment(x[:nv], t0, F, WL.grid_h, WL.grid_w, *WL.rope_split)
                err = np.abs(got[:nv] - formats.to_bf16(ref))
                bound = rope_bound(x[:nv], ref, got[:nv], t0 + F + max(WL.grid_h, WL.grid_w))
                assert np.all(err <= bound), f"layer {layer} turn {u}: RoPE of {name} off by {err.max():.3e}"
            frames = self.rings[layer].retained()
            kp = np.concatenate([quant.dequantise(p[0], p[1]) for _, p in frames], 0)
            vp = np.concatenate([quant.dequantise(p[2], p[3]) for _, p in frames], 0)
            say(f"denoise turn {u}: oracle attention of layer {layer} ({len(frames)} cached frames, all rows)")
            ref, ref_lse = attention.segment_attention(host_f64(gq), host_f64(gk), x0[2], kp, vp, scale)
            got = host_f64(o1)
            diff = np.abs(got - ref)
            lim = 1e-2 * np.abs(ref).max()
            assert diff.max() <= lim and diff.mean() <= 1e-3, \
                f"layer {layer} turn {u}: max|diff| {diff.max():.3e} (limit {lim:.3e}), mean {diff.mean():.3e}"
            g_lse = l1.cpu().numpy().reshape(H, nq)
            assert np.max(np.abs(g_lse - ref_lse)) <= LSE_TOL, f"layer {layer} turn {u}: lse"

        # the appends after step 8, each against the oracle quantiser and ring
        for layer in range(WL.n_layers):
            say(f"denoise turn {u}: append of layer {layer}")
            c, ring = self.caches[layer], self.rings[layer]
            before = [t.clone() for t in (c.k, c.v, c.k_scale, c.v_scale)]
            fw0 = ring.frames_written
            c.nomas_kvcache_append(k_final[layer], pristine[layer][2], F)
            qs = self._quantise(k_final[layer][:nv], pristine[layer][2][:nv])
            ring.append(_frames_of(qs, tpf, F))
            assert c.frames_written == ring.frames_written and c.valid_frames == ring.valid_frames()
            new = range(fw0, fw0 + F)
            self._check_slots(c, ring, new, f"turn {u} layer {layer}")
            # every slot the append did not own is unchanged
            P = c.token_pitch
            owned = torch.zeros(P, dtype=torch.bool, device="cuda")
            for slot, (f, _) in ring.expected_slots().items():
                if f in new:
                    owned[slot * tpf:(slot + 1) * tpf] = True
            keep = ~owned
            assert torch.equal(before[0].view(H, P, D)[:, keep], c.k.view(H, P, D)[:, keep])
            assert torch.equal(before[1].view(H, D, P)[:, :, keep], c.v.view(H, D, P)[:, :, keep])
            assert torch.equal(before[2].view(H, P)[:, keep], c.k_scale.view(H, P)[:, keep])
            assert torch.equal(before[3].view(H, P)[:, keep], c.v_scale.view(H, P)[:, keep])
            if layer not in CHECK_LAYERS:
                # payloads are kept only where the attention is checked
                ring.frames = [(f, None) for f, _ in ring.frames]
        torch.cuda.synchronize()
        self.turns_done = u


@pytest.fixture(scope="module")
def sweep():
    s = Sweep()
    yield s
    s.pool.shutdown()


@pytest.mark.parametrize("turn", [1, 2, 3])
def test_denoise_turn(sweep, turn):
    sweep.run_turn(turn)
