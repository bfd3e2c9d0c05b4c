"""Helpers shared by the GPU parity tests: device upload/readback and the
logical view of the library's cache buffers. No arithmetic of the method."""

import sys

import numpy as np
import torch

from segment_autoregressive_dit_amd import nomas


def say(*a):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(bits):
    """uint16 bf16 patterns -> bf16 CUDA tensor of the same shape."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_f64(t):
    """bf16/fp32 CUDA tensor -> float64 numpy (widening only)."""
    return t.float().cpu().numpy().astype(np.float64)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def cache_slots(cache):
    """Read the cache back in logical order of physical slots.

    Returns (k, v, ks, vs) with k, v as [pitch, H, D] arrays (int8 codes or bf16
    bit patterns) and scales [pitch, H] float32 (None for bf16)."""
    d = cache.desc
    H, D, P = d.n_heads, d.head_dim, d.token_pitch
    torch.cuda.synchronize()
    if cache.int8:
        k = cache.k.cpu().numpy().view(np.int8).reshape(H, P, D).transpose(1, 0, 2)
        v = cache.v.cpu().numpy().view(np.int8).reshape(H, D, P).transpose(2, 0, 1)
        ks = cache.k_scale.cpu().numpy().reshape(H, P).T
        vs = cache.v_scale.cpu().numpy().reshape(H, P).T
        return k, v, ks, vs
    k = cache.k.cpu().numpy().view(np.uint16).reshape(H, P, D).transpose(1, 0, 2)
    v = cache.v.cpu().numpy().view(np.uint16).reshape(H, D, P).transpose(2, 0, 1)
    return k, v, None, None


def attention_tolerance(got, ref):
    """max|diff| <= 1e-2 * max|ref| and mean|diff| <= 1e-3 (bf16/int8 paths vs fp64)."""
    diff = np.abs(got - ref)
    return diff.max(), diff.mean(), 1e-2 * np.abs(ref).max()


def new_cache(wl, int8=None, capacity=None):
    return nomas.KVCache(wl.n_heads, wl.head_dim, wl.tpf, capacity or wl.capacity_frames,
                         wl.kv_int8 if int8 is None else int8)


class Guarded:
    """A device buffer of ``nbytes`` between two sentinel bands of BAND bytes
    (256-byte aligned payload). ``check()`` asserts that no byte outside the
    payload changed -- the call under test wrote only where it owns."""
    BAND = 4096
    FILL = 0xA5

    def __init__(self, nbytes):
        self.nbytes = int(nbytes)
        self.raw = torch.full((self.nbytes + 2 * self.BAND,), self.FILL, dtype=torch.uint8, device="cuda")

    def view(self, dtype, shape):
        return self.raw[self.BAND:self.BAND + self.nbytes].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        lo, hi = self.raw[:self.BAND], self.raw[self.BAND + self.nbytes:]
        assert bool((lo == self.FILL).all()) and bool((hi == self.FILL).all()), f"{what}: bytes outside it changed"


def guarded_like(t):
    """A guarded copy of tensor ``t`` (same dtype, shape and contents)."""
    g = Guarded(t.numel() * t.element_size())
    v = g.view(t.dtype, tuple(t.shape))
    v.copy_(t)
    return g, v
