"""Write the oracle fixtures of the tiny workload (2 heads x 64, 4x6 grid, 4
cached frames, a 2-frame segment + 16 text tokens) to tiny_oracle.json.

The pages print no worked example values, so these fixtures are not the pages':
they are outputs of oracle/ alone (this script imports nothing else of the
library's arithmetic; the seeded inputs come from the input generator), kept so
that an unintended change of the oracle's arithmetic shows up as a failing test.
A deliberate change must regenerate them and cite, in its commit message, the
passage or the reading that justifies it.

    python tests/golden/make_golden.py
"""

import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from oracle import attention, formats, quant, rope  # noqa: E402
from segment_autoregressive_dit_amd import synth  # noqa: E402

ROWS = [0, 1, 23, 24, 47, 48, 63]           # first/last video rows of each frame, text rows


def compute():
    wl = synth.WORKLOADS["tiny"]
    H, D, F = wl.n_heads, wl.head_dim, wl.seg_frames
    q_b, k_b, v_b = synth.current_qkv(wl)
    kp_b, vp_b = synth.prefill_kv(wl)
    x = [synth.bf16_bits_to_f64(t) for t in (q_b, k_b, v_b)]
    nv = wl.n_video
    rq = formats.to_bf16(rope.rope3d_segment(x[0][:nv], wl.t0, F, wl.grid_h, wl.grid_w, *wl.rope_split))
    rk = formats.to_bf16(rope.rope3d_segment(x[1][:nv], wl.t0, F, wl.grid_h, wl.grid_w, *wl.rope_split))
    kq, ks = quant.quantise(synth.bf16_bits_to_f64(kp_b))
    vq, vs = quant.quantise(synth.bf16_bits_to_f64(vp_b))
    qr = np.concatenate([rq, x[0][nv:]])
    kr = np.concatenate([rk, x[1][nv:]])
    out, lse = attention.segment_attention(qr, kr, x[2], quant.dequantise(kq, ks), quant.dequantise(vq, vs),
                                           1.0 / math.sqrt(D))
    return {
        "workload": "tiny: 2 heads x 64, grid 4x6, 4 cached frames (INT8), 2-frame segment (t0 = 4) + 16 text",
        "rows": ROWS,
        "rope_q_bf16_bits": formats.bf16_bits(rq[[r for r in ROWS if r < nv]]).astype(int).tolist(),
        "rope_k_bf16_bits": formats.bf16_bits(rk[[r for r in ROWS if r < nv]]).astype(int).tolist(),
        "k_codes_first_rows": kq[:3].astype(int).tolist(),
        "k_scales_f32_bits_first_rows": ks[:3].view(np.uint32).astype(int).tolist(),
        "v_codes_first_rows": vq[:3].astype(int).tolist(),
        "v_scales_f32_bits_first_rows": vs[:3].view(np.uint32).astype(int).tolist(),
        "attention_out": [[[float(v) for v in out[r, h]] for h in range(H)] for r in ROWS],
        "attention_lse": [[float(lse[h, r]) for r in ROWS] for h in range(H)],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(compute(), f, separators=(",", ":"))
        f.write("\n")
    print("wrote", os.path.join(HERE, "tiny_oracle.json"))
