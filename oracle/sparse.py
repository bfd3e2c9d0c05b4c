"""Block-sparse segment attention (test infrastructure only).

The pages: after two dense denoising steps, attention keeps 25 % of the
candidate video blocks ("Hy-Nomas auf einer RTX 4090", inferencekey.com, section
"Das Single-GPU-Preset", citing the tech report's section 6.2). They name no
block size and no selection rule. Readings:

* Candidates are the cached (history) video keys, cut into blocks of
  KEY_BLOCK = 128 consecutive cache rows (the last block may be shorter). The
  current segment's rows stay dense.
* Selection is per head and per block of QUERY_BLOCK = 256 consecutive query
  rows: candidate c scores mean_q . mean_k(c) (means of the block's query rows
  and of the candidate's keys, as the attention sees them), and the n_select
  highest scores are kept (equal scores: the lower block index first). The
  list is stored in ascending block order.
* Given the lists, each query attends to its block's selected candidate rows
  plus the whole current segment, with the usual softmax(scale q.k) v.
"""

import numpy as np

from .attention import segment_attention

KEY_BLOCK = 128
QUERY_BLOCK = 256


def n_candidates(n_cached):
    return (n_cached + KEY_BLOCK - 1) // KEY_BLOCK


def block_means(x, block):
    """Row means of consecutive blocks of ``block`` rows: [n, H, D] -> [nb, H, D]."""
    x = np.asarray(x, np.float64)
    nb = (x.shape[0] + block - 1) // block
    return np.stack([x[b * block:(b + 1) * block].mean(axis=0) for b in range(nb)])


def block_scores(q, k_past):
    """scores[h, qb, c] = mean_q(qb) . mean_k(c)."""
    mq = block_means(q, QUERY_BLOCK)
    mk = block_means(k_past, KEY_BLOCK)
    return np.einsum("bhd,chd->hbc", mq, mk)


def select_blocks(q, k_past, n_select):
    """[H, n_qblocks, n_select] int32 lists: top scores, ties to the lower index,
    each list ascending."""
    s = block_scores(q, k_past)
    H, nqb, nc = s.shape
    out = np.empty((H, nqb, n_select), np.int32)
    for h in range(H):
        for b in range(nqb):
            order = sorted(range(nc), key=lambda c: (-s[h, b, c], c))
            out[h, b] = sorted(order[:n_select])
    return out


def sparse_segment_attention(q, k_cur, v_cur, k_past, v_past, lists, scale):
    """Each query block attends to its selected candidate blocks (per head) plus
    the whole current segment. Returns out [n_q, H, D] and lse [H, n_q]."""
    n_q, H, D = q.shape
    out = np.empty((n_q, H, D))
    lse = np.empty((H, n_q))
    for b in range((n_q + QUERY_BLOCK - 1) // QUERY_BLOCK):
        r = slice(b * QUERY_BLOCK, min(n_q, (b + 1) * QUERY_BLOCK))
        for h in range(H):
            rows = np.concatenate([np.arange(c * KEY_BLOCK, min(k_past.shape[0], (c + 1) * KEY_BLOCK))
                                   for c in lists[h, b]]) if len(lists[h, b]) else np.zeros(0, int)
            kp = k_past[rows, h:h + 1] if len(rows) else None
            vp = v_past[rows, h:h + 1] if len(rows) else None
            o, l = segment_attention(q[r, h:h + 1], k_cur[:, h:h + 1], v_cur[:, h:h + 1], kp, vp, scale)
            out[r, h] = o[:, 0]
            lse[h, r] = l[0]
    return out, lse
