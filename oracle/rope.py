"""3D rotary position embedding (test infrastructure only).

The pages name "3D RoPE" in the model card's architecture list ("Hy-Nomas auf
einer RTX 4090", inferencekey.com, section "Modell und Dateien"; orcarouter.ai,
section "Die Schleife": "3D-Rotations-Positions-Embeddings"; blog.authon.dev,
section "What Hy-Nomas is") and give nothing else. Readings taken here, each a
call argument of the library so that no reading is baked in:

* The head dimension D is cut into three bands, [0, d_t), [d_t, d_t+d_h),
  [d_t+d_h, D), rotated by the frame, row and column index respectively.
  (D = 64 uses 16/24/24 as the tiny configuration states; D = 128 uses 32/48/48.)
* Inside a band of width d_a, channels (2j, 2j+1) form a pair rotated by the
  angle pos_a * theta**(-2j/d_a), theta = 10000 (the RoFormer law, per axis).
* Token i of a segment whose first latent frame is t0, on a grid_h x grid_w
  latent grid, sits at t = t0 + i // (grid_h*grid_w), h = (i // grid_w) % grid_h,
  w = i % grid_w. Frame indices count from the start of the session.
* Text tokens are not rotated.

All arithmetic is float64; the caller rounds to bfloat16 where a value is stored.
"""

import numpy as np


def video_positions(t0, n_frames, grid_h, grid_w):
    """(t, h, w) integer positions of the n_frames*grid_h*grid_w video tokens."""
    i = np.arange(n_frames * grid_h * grid_w, dtype=np.int64)
    t = t0 + i // (grid_h * grid_w)
    h = (i // grid_w) % grid_h
    w = i % grid_w
    return t, h, w


def angles(pos, width, theta=10000.0):
    """Angle of every pair of one band: [n_tokens, width//2] float64."""
    j = np.arange(width // 2, dtype=np.float64)
    omega = theta ** (-2.0 * j / width)
    return np.asarray(pos, dtype=np.float64)[:, None] * omega[None, :]


def rope3d(x, t, h, w, d_t, d_h, d_w, theta=10000.0, sign=1.0):
    """Rotate x[n, H, D] (float64) by the 3D positions; returns a new array.

    ``sign = -1`` applies the inverse rotation (the negated angles).
    """
    x = np.asarray(x, dtype=np.float64)
    n, H, D = x.shape
    if d_t + d_h + d_w != D or d_t % 2 or d_h % 2 or d_w % 2:
        raise ValueError("band widths must be even and sum to the head dim")
    out = x.copy()
    offset = 0
    for pos, width in ((t, d_t), (h, d_h), (w, d_w)):
        if width:
            phi = sign * angles(pos, width, theta)           # [n, width/2]
            c = np.cos(phi)[:, None, :]
            s = np.sin(phi)[:, None, :]
            u = x[:, :, offset:offset + width:2]
            v = x[:, :, offset + 1:offset + width:2]
            out[:, :, offset:offset + width:2] = u * c - v * s
            out[:, :, offset + 1:offset + width:2] = u * s + v * c
        offset += width
    return out


def rope3d_segment(x_video, t0, n_frames, grid_h, grid_w, d_t, d_h, d_w,
                   theta=10000.0, sign=1.0):
    """Rotate the video rows of one segment (rows ordered frame, row, col)."""
    t, h, w = video_positions(t0, n_frames, grid_h, grid_w)
    if x_video.shape[0] != t.shape[0]:
        raise ValueError("row count does not match n_frames*grid_h*grid_w")
    return rope3d(x_video, t, h, w, d_t, d_h, d_w, theta, sign)
