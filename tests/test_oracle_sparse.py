"""Pins of the block-sparse oracle (oracle/sparse.py) against the dense oracle
and closed forms."""

import math

import numpy as np

from oracle import attention, sparse


def _r(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_blocks_selected_is_dense():
    # selecting every candidate block reproduces the dense cached attention
    q, kc, vc = _r((300, 2, 64), 1), _r((70, 2, 64), 2), _r((70, 2, 64), 3)
    kp, vp = _r((500, 2, 64), 4), _r((500, 2, 64), 5)
    nc = sparse.n_candidates(500)
    assert nc == 4
    lists = sparse.select_blocks(q, kp, nc)
    assert np.array_equal(lists, np.broadcast_to(np.arange(nc), lists.shape))
    a, la = attention.segment_attention(q, kc, vc, kp, vp, 0.125)
    b, lb = sparse.sparse_segment_attention(q, kc, vc, kp, vp, lists, 0.125)
    assert np.max(np.abs(a - b)) < 1e-13 and np.max(np.abs(la - lb)) < 1e-12


def test_no_blocks_selected_is_segment_only():
    q, kc, vc = _r((40, 1, 64), 6), _r((40, 1, 64), 7), _r((40, 1, 64), 8)
    kp, vp = _r((256, 1, 64), 9), _r((256, 1, 64), 10)
    a, _ = attention.segment_attention(q, kc, vc, None, None, 0.125)
    b, _ = sparse.sparse_segment_attention(q, kc, vc, kp, vp, np.zeros((1, 1, 0), np.int32), 0.125)
    assert np.max(np.abs(a - b)) < 1e-13


def test_selected_rows_only_matter():
    # changing keys/values of unselected blocks leaves the result unchanged;
    # changing a selected block changes it
    q, kc, vc = _r((256, 1, 64), 11), _r((30, 1, 64), 12), _r((30, 1, 64), 13)
    kp, vp = _r((640, 1, 64), 14), _r((640, 1, 64), 15)
    lists = np.array([[[1, 3]]], np.int32)
    a, _ = sparse.sparse_segment_attention(q, kc, vc, kp, vp, lists, 0.125)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[0:128] += 5.0
    vp2[512:640] -= 3.0
    b, _ = sparse.sparse_segment_attention(q, kc, vc, kp2, vp2, lists, 0.125)
    assert np.max(np.abs(a - b)) < 1e-14
    vp2[128:256] += 1.0
    c, _ = sparse.sparse_segment_attention(q, kc, vc, kp2, vp2, lists, 0.125)
    assert np.max(np.abs(a - c)) > 1e-3


def test_planted_blocks_are_chosen():
    # query blocks aligned with chosen candidate directions: a block whose keys
    # share the query block's mean direction scores highest (closed form: the
    # score of block c is mean_q . mean_k(c))
    D, nc = 64, 10
    rng = np.random.default_rng(16)
    dirs = rng.standard_normal((nc, D))
    kp = 0.01 * rng.standard_normal((nc * 128, 1, D))
    for c in range(nc):
        kp[c * 128:(c + 1) * 128, 0] += dirs[c]
    q = 0.01 * rng.standard_normal((512, 1, D))
    q[:256, 0] += dirs[7]
    q[256:, 0] += dirs[2] + dirs[5]
    s = sparse.block_scores(q, kp)
    # the keys' 0.01 noise moves each block mean by ~0.01/sqrt(128) per channel
    assert np.max(np.abs(s[0, 0] - dirs @ q[:256, 0].mean(0))) < 0.05
    lists = sparse.select_blocks(q, kp, 1)
    assert lists[0, 0, 0] == 7
    assert set(sparse.select_blocks(q, kp, 2)[0, 1]) == {2, 5}


def test_ties_go_to_lower_index_and_lists_ascend():
    kp = np.zeros((6 * 128, 1, 8))
    kp[:, 0, 0] = np.repeat([1.0, 3.0, 3.0, 2.0, 3.0, 0.0], 128)
    q = np.zeros((10, 1, 8))
    q[:, 0, 0] = 1.0
    assert sparse.select_blocks(q, kp, 2)[0, 0].tolist() == [1, 2]
    assert sparse.select_blocks(q, kp, 4)[0, 0].tolist() == [1, 2, 3, 4]


def test_selection_invariances():
    # positive query scaling and key order inside a block leave the lists unchanged
    q, kp = _r((700, 2, 32), 17), _r((1000, 2, 32), 18)
    base = sparse.select_blocks(q, kp, 3)
    assert np.array_equal(base, sparse.select_blocks(3.5 * q, kp, 3))
    perm = np.concatenate([np.random.default_rng(19).permutation(np.arange(b * 128, min(1000, (b + 1) * 128)))
                           for b in range(8)])
    assert np.array_equal(base, sparse.select_blocks(q, kp[perm], 3))


def test_short_last_block_mean_is_over_its_own_rows():
    """A candidate block's score uses the plain mean of the rows it holds: the
    short last block of a cache that is not a whole number of blocks averages
    over its own rows (here 2 of 128), written out by hand."""
    x = np.ones((130, 1, 2))
    x[128] = [2.0, 4.0]
    x[129] = [4.0, 8.0]
    m = sparse.block_means(x, 128)
    assert m.shape == (2, 1, 2)
    assert np.array_equal(m[0], [[1.0, 1.0]])
    assert np.array_equal(m[1], [[3.0, 6.0]])


def test_each_head_uses_its_own_list():
    # two heads with different lists and two query blocks: every (query block,
    # head) output equals the dense cached attention of that head against the
    # rows its own list names (and a query block uses its own list)
    q, kc, vc = _r((300, 2, 64), 31), _r((20, 2, 64), 32), _r((20, 2, 64), 33)
    kp, vp = _r((384, 2, 64), 34), _r((384, 2, 64), 35)
    lists = np.array([[[0], [2]], [[1], [0]]], np.int32)          # [H, query block, n_select]
    out, lse = sparse.sparse_segment_attention(q, kc, vc, kp, vp, lists, 0.125)
    for h in range(2):
        for b, r in enumerate((slice(0, 256), slice(256, 300))):
            c = lists[h, b, 0]
            rows = slice(c * 128, (c + 1) * 128)
            a, la = attention.segment_attention(q[r, h:h + 1], kc[:, h:h + 1], vc[:, h:h + 1],
                                                kp[rows, h:h + 1], vp[rows, h:h + 1], 0.125)
            assert np.max(np.abs(out[r, h] - a[:, 0])) < 1e-13
            assert np.max(np.abs(lse[h, r] - la[0])) < 1e-12
