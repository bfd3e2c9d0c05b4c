"""Segment-wise causal joint attention (test infrastructure only).

The pages: each DiT block runs "segment-wise causal joint attention" over the
current segment while earlier segments enter through a persistent KV cache
(madebyagents.com model page "Hy-Nomas", component list: "Segment-Autoregressive
DiT" and "Persistent Lifelong KV Cache"; orcarouter.ai, section "Die Schleife").
Readings:

* Queries are the current segment's rows [video; text]. Keys and values are the
  retained cached video frames of earlier segments plus all rows of the current
  segment: bidirectional inside the segment, causal across segments.
* Only video keys/values are cached; text tokens live only in their segment.
* With an INT8 cache the cached keys/values enter as their dequantised values;
  the current segment's keys/values are used as given (bf16).
* softmax(scale * q.k) with scale = 1/sqrt(D) unless given.

Functions:

* ``segment_attention``  -- the cached formulation (one call per segment).
* ``block_causal_full``  -- the whole session as one sequence with an explicit
  boolean visibility mask; used to check the cached formulation.
* ``split_attention``    -- keys cut into contiguous chunks, each normalised on
  its own, then merged through their log-sum-exp.
* ``brute_force_attention`` -- explicit Python loops, for tiny inputs.
"""

import math

import numpy as np

CHUNK = 512


def _softmax_rows(s):
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=-1, keepdims=True)
    return p / l, (m + np.log(l))[..., 0]


def segment_attention(q, k_cur, v_cur, k_past=None, v_past=None, scale=None,
                      return_probs=False):
    """Cached segment attention in float64.

    q, k_cur, v_cur : [n_cur, H, D]   (current segment rows, video then text)
    k_past, v_past  : [n_past, H, D]  (retained cached video rows, any order)
    Returns out [n_cur, H, D] and lse [H, n_cur] (natural log of the softmax
    denominator of the scaled logits); with ``return_probs`` also the list of
    per-head probability matrices.
    """
    q = np.asarray(q, np.float64)
    n_q, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if k_past is None or len(k_past) == 0:
        k = np.asarray(k_cur, np.float64)
        v = np.asarray(v_cur, np.float64)
    else:
        k = np.concatenate([np.asarray(k_past, np.float64), np.asarray(k_cur, np.float64)], 0)
        v = np.concatenate([np.asarray(v_past, np.float64), np.asarray(v_cur, np.float64)], 0)
    out = np.empty((n_q, H, D))
    lse = np.empty((H, n_q))
    probs = []
    for h in range(H):
        kh, vh = k[:, h, :], v[:, h, :]
        ph = []
        for r0 in range(0, n_q, CHUNK):
            r1 = min(n_q, r0 + CHUNK)
            s = scale * (q[r0:r1, h, :] @ kh.T)
            p, l = _softmax_rows(s)
            out[r0:r1, h, :] = p @ vh
            lse[h, r0:r1] = l
            if return_probs:
                ph.append(p)
        if return_probs:
            probs.append(np.concatenate(ph, 0))
    if return_probs:
        return out, lse, probs
    return out, lse


def segment_attention_rows(q_rows, row_heads, k, v, scale):
    """Attention of selected query rows only (for sampled checks at full size).

    q_rows : [m, D] query vectors; row_heads : [m] head of each row;
    k, v   : [n_k, H, D] all keys/values of the call (past then current).
    """
    q_rows = np.asarray(q_rows, np.float64)
    out = np.empty_like(q_rows)
    lse = np.empty(q_rows.shape[0])
    for i, h in enumerate(row_heads):
        s = scale * (np.asarray(k[:, h, :], np.float64) @ q_rows[i])
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        out[i] = (p @ np.asarray(v[:, h, :], np.float64)) / l
        lse[i] = m + math.log(l)
    return out, lse


def split_attention(q, k, v, n_splits, scale):
    """Key range cut into ``n_splits`` contiguous chunks, merged by log-sum-exp.

    q [n_q, H, D]; k, v [n_k, H, D]. Each chunk s yields O_s (normalised inside
    the chunk) and lse_s; then lse = log sum_s exp(lse_s) and
    O = sum_s exp(lse_s - lse) O_s, summed in chunk order.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_k = k.shape[0]
    bounds = np.linspace(0, n_k, n_splits + 1).round().astype(int)
    parts = []
    for s in range(n_splits):
        a, b = bounds[s], bounds[s + 1]
        if b > a:
            parts.append(segment_attention(q, k[a:b], v[a:b], scale=scale))
    lse_all = np.stack([p[1] for p in parts])                 # [S, H, n_q]
    m = lse_all.max(0)
    lse = m + np.log(np.sum(np.exp(lse_all - m), 0))
    out = np.zeros_like(q)
    for o_s, l_s in parts:
        w = np.exp(l_s - lse)                                 # [H, n_q]
        out += o_s * w.T[:, :, None]
    return out, lse


def block_causal_full(segments, window_frames=None, scale=None, rows=None, return_lse=False):
    """Whole session as one sequence under the block-causal visibility mask.

    ``segments`` is a list, in session order, of dicts with
      q, k, v        : [F*tpf + T, H, D]  rows [video; text] of the segment
      k_past, v_past : optional [F*tpf, H, D] -- the values the segment's video
                       keys/values take when *later* segments see them (the
                       dequantised values for an INT8 cache); default k, v
      t0, n_frames, tpf : first latent frame, frames, tokens per frame
    Key j is visible to query i iff seg(j) == seg(i), or seg(j) < seg(i), j is
    a video token and frame(j) >= t0(seg(i)) - window_frames.
    ``rows``: optional per-segment arrays of the query rows to compute (None:
    all). Returns the list of per-segment outputs [rows, H, D], and with
    ``return_lse`` also the list of per-segment log-sum-exps [H, rows].
    """
    key_rows = []       # (segment id, is_video, frame)
    for sid, sg in enumerate(segments):
        nv = sg["n_frames"] * sg["tpf"]
        nt = sg["q"].shape[0] - nv
        for i in range(nv):
            key_rows.append((sid, True, sg["t0"] + i // sg["tpf"]))
        for i in range(nt):
            key_rows.append((sid, False, -1))
    seg_id = np.array([r[0] for r in key_rows])
    is_vid = np.array([r[1] for r in key_rows])
    frame = np.array([r[2] for r in key_rows])
    H, D = segments[0]["q"].shape[1:]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    outs, lses = [], []
    for sid, sg in enumerate(segments):
        sel = np.arange(sg["q"].shape[0]) if rows is None or rows[sid] is None else np.asarray(rows[sid])
        qi = np.asarray(sg["q"], np.float64)[sel]
        # keys as seen by this segment: own rows raw, earlier video rows as cached
        ks, vs = [], []
        for tid, tg in enumerate(segments):
            if tid == sid:
                ks.append(np.asarray(tg["k"], np.float64))
                vs.append(np.asarray(tg["v"], np.float64))
            else:
                nv = tg["n_frames"] * tg["tpf"]
                kp = np.asarray(tg.get("k_past", tg["k"][:nv]), np.float64)
                vp = np.asarray(tg.get("v_past", tg["v"][:nv]), np.float64)
                ks.append(np.concatenate([kp, np.asarray(tg["k"][nv:], np.float64)], 0))
                vs.append(np.concatenate([vp, np.asarray(tg["v"][nv:], np.float64)], 0))
        k = np.concatenate(ks, 0)
        v = np.concatenate(vs, 0)
        lower = -np.inf if window_frames is None else sg["t0"] - window_frames
        visible = (seg_id == sid) | ((seg_id < sid) & is_vid & (frame >= lower))
        out = np.empty((len(sel), H, D))
        lse = np.empty((H, len(sel)))
        for h in range(H):
            s = scale * (qi[:, h, :] @ k[:, h, :].T)
            s = np.where(visible[None, :], s, -np.inf)
            p, lse[h] = _softmax_rows(s)
            out[:, h, :] = p @ v[:, h, :]
        outs.append(out)
        lses.append(lse)
    return (outs, lses) if return_lse else outs


def brute_force_attention(q, k, v, scale):
    """softmax(scale q.k) v with explicit loops over (h, i, j, d). Tiny inputs only."""
    n_q, H, D = len(q), len(q[0]), len(q[0][0])
    n_k = len(k)
    out = [[[0.0] * D for _ in range(H)] for _ in range(n_q)]
    lse = [[0.0] * n_q for _ in range(H)]
    for h in range(H):
        for i in range(n_q):
            logits = []
            for j in range(n_k):
                acc = 0.0
                for d in range(D):
                    acc += float(q[i][h][d]) * float(k[j][h][d])
                logits.append(scale * acc)
            m = max(logits)
            e = [math.exp(x - m) for x in logits]
            tot = math.fsum(e)
            for d in range(D):
                out[i][h][d] = math.fsum(e[j] * float(v[j][h][d]) for j in range(n_k)) / tot
            lse[h][i] = m + math.log(tot)
    return np.array(out), np.array(lse)
