"""QKV projection with 3D RoPE (test infrastructure only).

The step before the hot path: the DiT block projects its hidden states (size
2,048) to the 16 x 128 query, key and value heads, and the queries and keys of
video tokens are rotated by 3D RoPE ("Hy-Nomas auf einer RTX 4090",
inferencekey.com, section "Modell und Dateien": hidden size 2,048, 16 heads,
3D RoPE; blog.authon.dev, section "What Hy-Nomas is"). Readings:

* y = x W^T, W of shape [3 * H * D, hidden] (query, key, value channels in that
  order, each head's D channels together); no bias (the pages name none).
* RoPE (oracle/rope.py) is applied to the query and key channels of the video
  rows (the first n_video rows); text rows and value channels are unchanged.
* The result is rounded to bfloat16 once (projection and rotation exact).
"""

import numpy as np

from . import formats
from .rope import rope3d_segment


def qkv_projection(x, w, n_heads, head_dim, n_video=0, rope=None):
    """x [n, hidden], w [3*H*D, hidden] (float64 holding bf16 values).

    rope: None, or dict(t0, n_frames, grid_h, grid_w, d_t, d_h, d_w[, theta])
    describing the n_video = n_frames*grid_h*grid_w video rows.
    Returns bf16-rounded q, k, v, each [n, H, D] (float64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    H, D = n_heads, head_dim
    y = x @ w.T
    q, k, v = (y[:, i * H * D:(i + 1) * H * D].reshape(-1, H, D).copy() for i in range(3))
    if rope is not None and n_video > 0:
        r = dict(rope)
        args = (r["t0"], r["n_frames"], r["grid_h"], r["grid_w"], r["d_t"], r["d_h"], r["d_w"])
        theta = r.get("theta", 10000.0)
        q[:n_video] = rope3d_segment(q[:n_video], *args, theta=theta)
        k[:n_video] = rope3d_segment(k[:n_video], *args, theta=theta)
    return formats.to_bf16(q), formats.to_bf16(k), formats.to_bf16(v)
