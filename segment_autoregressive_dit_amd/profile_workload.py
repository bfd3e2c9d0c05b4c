"""Profiling driver: run one kernel of the hot path a fixed number of times on a
named synthetic workload, for use under ``rocprofv3`` (kernel trace or counters).

    python -m segment_autoregressive_dit_amd.profile_workload --kernel attention --workload layer_bf16 --reps 5
    python -m segment_autoregressive_dit_amd.profile_workload --kernel copy --bytes 1073741824

``--kernel copy`` runs a plain device-to-device copy of known size (torch's copy
kernel), the calibration for HBM byte counters (FETCH_SIZE / WRITE_SIZE).
"""

import argparse
import os
import sys

import numpy as np
import torch

from segment_autoregressive_dit_amd import nomas, synth


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--kernel", choices=["attention", "rope", "append", "copy"], required=True)
    p.add_argument("--workload", default="layer_bf16", choices=sorted(synth.WORKLOADS))
    p.add_argument("--reps", type=int, default=5)
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--bytes", type=int, default=1 << 30)
    a = p.parse_args(argv)
    if a.kernel == "copy":
        src = torch.empty(a.bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(a.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy: {a.reps} x {a.bytes} bytes", file=sys.stderr)
        return
    wl = synth.WORKLOADS[a.workload]
    H, D = wl.n_heads, wl.head_dim
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, wl.kv_int8)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(_dev(kb), _dev(vb), wl.cached_frames)
    q, k, v = (_dev(t) for t in synth.current_qkv(wl))
    out = torch.empty_like(q)
    ws = nomas.workspace_for(cache, wl.n_video, wl.n_text, a.splits)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        if a.kernel == "attention":
            nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, n_splits=a.splits,
                                          workspace=ws)
        elif a.kernel == "rope":
            nomas.nomas_rope3d(q, k, wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split, H, D)
        else:
            cache.nomas_kvcache_append(k, v, wl.seg_frames)
    torch.cuda.synchronize()
    print(f"{a.kernel} on {a.workload}: {a.reps} launches", file=sys.stderr)


if __name__ == "__main__":
    main()
