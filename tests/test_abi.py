"""CPU checks of the C ABI: the library loads, exports every symbol nomas.h
declares, and rejects invalid arguments on the host before anything is enqueued
(no call here reaches a kernel launch, so no GPU is needed)."""

import ctypes
import os
import re

import pytest

from segment_autoregressive_dit_amd import nomas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "nomas.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nomas_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = nomas.lib()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_binding_names_match_the_c_entry_points():
    for n in ["nomas_rope3d", "nomas_segment_attention", "nomas_segment_attention_workspace_bytes",
              "nomas_segment_attention_splits", "nomas_kvcache_bytes", "nomas_version",
              "nomas_block_causal_attention", "nomas_block_causal_attention_workspace_bytes"]:
        assert callable(getattr(nomas, n))
    assert callable(nomas.KVCache.nomas_kvcache_append)


def test_version_and_sizes():
    L = nomas.lib()
    assert L.nomas_version() >= 1
    assert L.nomas_kvcache_token_pitch(960, 18) == 17280            # 135 * 128
    assert L.nomas_kvcache_token_pitch(880, 18) == 15872            # round_up(15840, 128)
    assert L.nomas_kvcache_token_pitch(24, 4) == 128
    assert L.nomas_kvcache_token_pitch(0, 4) == -1
    pitch = L.nomas_kvcache_token_pitch(960, 18)
    assert L.nomas_kvcache_bytes(16, 128, 960, 18, 1, 0) == 16 * pitch * 128
    assert L.nomas_kvcache_bytes(16, 128, 960, 18, 0, 1) == 16 * pitch * 128 * 2
    assert L.nomas_kvcache_bytes(16, 128, 960, 18, 1, 2) == 16 * pitch * 4
    assert L.nomas_kvcache_bytes(16, 128, 960, 18, 0, 2) == 0
    assert L.nomas_kvcache_bytes(16, 96, 960, 18, 0, 0) == 0


def _desc(dtype=1, heads=2, dim=64, tpf=24, cap=4):
    L = nomas.lib()
    d = nomas.KVCacheDesc()
    fake = 1 << 20          # 16-byte aligned placeholder addresses, never dereferenced
    sc = ctypes.c_void_p(fake * 3) if dtype == 1 else None
    sv = ctypes.c_void_p(fake * 4) if dtype == 1 else None
    rc = L.nomas_kvcache_init(ctypes.byref(d), heads, dim, tpf, cap, dtype,
                              ctypes.c_void_p(fake), ctypes.c_void_p(fake * 2), sc, sv)
    return L, d, rc


def test_kvcache_init_validation():
    L, d, rc = _desc()
    assert rc == 0 and d.frames_written == 0 and d.token_pitch == 128
    assert L.nomas_kvcache_valid_frames(ctypes.byref(d)) == 0
    bad = nomas.KVCacheDesc()
    f = ctypes.c_void_p(1 << 20)
    assert L.nomas_kvcache_init(ctypes.byref(bad), 2, 96, 24, 4, 0, f, f, None, None) == nomas.NOMAS_E_UNSUPPORTED
    assert L.nomas_kvcache_init(ctypes.byref(bad), 2, 64, 24, 4, 1, f, f, None, None) == nomas.NOMAS_E_INVALID
    assert b"INT8" in L.nomas_last_error()
    assert L.nomas_kvcache_init(ctypes.byref(bad), 2, 64, 24, 4, 0, ctypes.c_void_p((1 << 20) + 4), f, None,
                                None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_init(ctypes.byref(bad), 2, 64, 0, 4, 0, f, f, None, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_init(None, 2, 64, 24, 4, 0, f, f, None, None) == nomas.NOMAS_E_INVALID


def test_per_head_slice_limit():
    """The kernels address one head's K or V slice with 32-bit byte offsets, so a
    cache whose per-head slice reaches 2 GiB is refused at init and by every call
    that takes the descriptor (rather than wrapping on the GPU)."""
    L = nomas.lib()
    f = ctypes.c_void_p(1 << 20)
    s = ctypes.c_void_p(1 << 21)
    d = nomas.KVCacheDesc()
    # bf16, head dim 128: token_pitch 8,387,584 -> 2,147,221,504 bytes per head (fits)
    assert L.nomas_kvcache_init(ctypes.byref(d), 1, 128, 1024, 8191, 0, f, f, None, None) == 0
    # token_pitch 8,389,632 -> 2,147,745,792 bytes: one past the limit
    assert L.nomas_kvcache_init(ctypes.byref(d), 1, 128, 1024, 8193, 0, f, f, None, None) == nomas.NOMAS_E_INVALID
    assert b"2 GiB" in L.nomas_last_error()
    # INT8 codes are one byte: twice the tokens fit
    assert L.nomas_kvcache_init(ctypes.byref(d), 1, 128, 1024, 16383, 1, f, f, s, s) == 0
    assert L.nomas_kvcache_init(ctypes.byref(d), 1, 128, 1024, 16385, 1, f, f, s, s) == nomas.NOMAS_E_INVALID
    # a descriptor edited past the limit is refused by the calls that read it
    L2, d2, rc = _desc(dtype=0)
    assert rc == 0
    d2.tokens_per_frame, d2.capacity_frames = 1024, 16385
    d2.token_pitch = L.nomas_kvcache_token_pitch(1024, 16385)
    p = ctypes.c_void_p(1 << 24)
    assert L.nomas_kvcache_append(ctypes.byref(d2), p, p, 128, 1, None) == nomas.NOMAS_E_INVALID
    assert b"2 GiB" in L.nomas_last_error()
    assert d2.frames_written == 0


def test_append_rejects_before_launch_and_keeps_descriptor():
    L, d, _ = _desc()
    p = ctypes.c_void_p(1 << 24)
    for args in [(None, p, 128, 2), (p, p, 64, 2), (p, p, 130, 2), (p, p, 128, 0),
                 (ctypes.c_void_p((1 << 24) + 2), p, 128, 2)]:
        rc = L.nomas_kvcache_append(ctypes.byref(d), args[0], args[1], args[2], args[3], None)
        assert rc == nomas.NOMAS_E_INVALID, args
        assert d.frames_written == 0
    assert L.nomas_kvcache_append(None, p, p, 128, 1, None) == nomas.NOMAS_E_INVALID
    d.token_pitch = 64      # corrupted descriptor
    assert L.nomas_kvcache_append(ctypes.byref(d), p, p, 128, 1, None) == nomas.NOMAS_E_INVALID


def test_rope_rejects_before_launch():
    L = nomas.lib()
    p = ctypes.c_void_p(1 << 24)
    ok = dict(q=p, k=p, ld=128, H=2, D=64, t0=0, F=2, gh=4, gw=6, dt=16, dh=24, dw=24, theta=1e4, inv=0)
    cases = [dict(q=None), dict(D=96), dict(dt=18, dh=24), dict(dt=15, dh=25), dict(dt=16, dh=24, dw=26),
             dict(F=0), dict(gh=0), dict(t0=-1), dict(theta=0.0), dict(ld=100), dict(ld=127),
             dict(q=ctypes.c_void_p((1 << 24) + 8))]
    for c in cases:
        a = dict(ok, **c)
        rc = L.nomas_rope3d(a["q"], a["k"], a["ld"], a["H"], a["D"], a["t0"], a["F"], a["gh"], a["gw"], a["dt"],
                            a["dh"], a["dw"], a["theta"], a["inv"], None)
        assert rc in (nomas.NOMAS_E_INVALID, nomas.NOMAS_E_UNSUPPORTED), c
        assert L.nomas_last_error()


def test_attention_rejects_before_launch():
    L, d, _ = _desc()
    p = ctypes.c_void_p(1 << 24)
    ws = ctypes.c_void_p(1 << 26)
    need = L.nomas_segment_attention_workspace_bytes(48, 16, 0, 2, 64, d.kv_dtype, 0)
    assert need > 0

    def call(**kw):
        a = dict(q=p, k=p, v=p, ld=128, nv=48, nt=16, out=p, ldo=128, lse=None, scale=0.125, splits=0,
                 ws=ws, wsb=need)
        a.update(kw)
        return L.nomas_segment_attention(a["q"], a["k"], a["v"], a["ld"], a["nv"], a["nt"], ctypes.byref(d),
                                         a["out"], a["ldo"], a["lse"], a["scale"], a["splits"], a["ws"], a["wsb"],
                                         None)
    assert call(q=None) == nomas.NOMAS_E_INVALID
    assert call(ld=64) == nomas.NOMAS_E_INVALID
    assert call(ldo=120) == nomas.NOMAS_E_INVALID
    assert call(nv=0, nt=0) == nomas.NOMAS_E_INVALID
    assert call(nv=-1) == nomas.NOMAS_E_INVALID
    assert call(scale=0.0) == nomas.NOMAS_E_INVALID
    assert call(scale=float("inf")) == nomas.NOMAS_E_INVALID
    assert call(splits=-2) == nomas.NOMAS_E_INVALID
    assert call(ws=None) == nomas.NOMAS_E_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 26) + 16)) == nomas.NOMAS_E_WORKSPACE
    assert call(wsb=need - 1) == nomas.NOMAS_E_WORKSPACE
    assert b"workspace" in L.nomas_last_error()
    # 64 rows at a row stride of 2**24 elements: 2 GiB of current-segment bytes,
    # past the kernels' 32-bit byte ranges
    assert call(ld=1 << 24, ldo=1 << 24) == nomas.NOMAS_E_INVALID
    assert b"2 GiB" in L.nomas_last_error()


def test_workspace_and_split_planning():
    L = nomas.lib()
    BF16, INT8 = nomas.NOMAS_KV_BF16, nomas.NOMAS_KV_INT8
    # the measured single-layer shape: 7,680 video + 256 text queries, 17,280 cached
    for dt in (BF16, INT8):
        s = L.nomas_segment_attention_splits(7680, 256, 17280, 16, 128, dt, 0)
        assert s >= 1
        for req in (1, 2, 4, 8):
            assert L.nomas_segment_attention_splits(7680, 256, 84480, 16, 128, dt, req) == req
            b1 = L.nomas_segment_attention_workspace_bytes(7680, 256, 84480, 16, 128, dt, req)
            assert b1 >= 16 * 128 * 7936 * 2 + (req > 1) * req * 16 * 7936 * 128 * 4
    # more splits than key tiles is clamped (10 current keys: one tile)
    assert L.nomas_segment_attention_splits(10, 0, 0, 1, 64, BF16, 50) == 1
    # 1,000 cached + 24 current keys at head dim 128: 8 + 1 tiles of 128 keys
    # (bf16) or 16 + 1 tiles of 64 keys (INT8)
    assert L.nomas_segment_attention_splits(16, 8, 1000, 1, 128, BF16, 50) == 9
    assert L.nomas_segment_attention_splits(16, 8, 1000, 1, 128, INT8, 50) == 17
    assert L.nomas_segment_attention_workspace_bytes(0, 0, 0, 16, 128, BF16, 0) == 0
    assert L.nomas_segment_attention_splits(10, 0, 0, 1, 96, BF16, 0) == -1
    assert L.nomas_segment_attention_splits(10, 0, 0, 1, 64, 7, 0) == -1


def test_automatic_split_count_minimises_rounds():
    """n_splits = 0 at the layer lengths (7,936 queries in 31 blocks per head,
    197 bf16 / 394 INT8 key tiles): with s splits the call runs
    ceil(31*H*s / 256) rounds of blocks that each take 1/s of the keys; the plan
    takes the smallest s within 10 % of the shortest such makespan (s <= 256,
    >= 16 key tiles per split), and 1 once the blocks fill the 256 CUs."""
    import math
    L = nomas.lib()

    def expected(H, tiles=197):
        blocks = 31 * H
        if blocks >= 256:
            return 1
        span = {s: math.ceil(blocks * s / 256) / s for s in range(1, min(256, tiles // 16) + 1)}
        best = min(span.values())
        return min(s for s in span if span[s] <= best * 1.10)

    for H in range(1, 17):
        for dt, tiles in ((nomas.NOMAS_KV_BF16, 197), (nomas.NOMAS_KV_INT8, 394)):
            assert L.nomas_segment_attention_splits(7680, 256, 17280, H, 128, dt, 0) == expected(H, tiles), H
    # one GPU's share of 8-way head sharding (2 heads): 62 blocks x 4 = one round
    assert expected(2) == 4 and expected(1) == 8 and expected(16) == 1
    # one query against a long history (721 key tiles, so at most 45 splits of
    # 16 tiles): one block per split, and 41 is the smallest count within 10 %
    # of the 45-split makespan
    assert L.nomas_segment_attention_splits(0, 1, 92160, 1, 128, nomas.NOMAS_KV_BF16, 0) == 41


def test_sparse_split_plan_can_leave_a_split_without_tiles():
    """The sparse call plans its splits for n_select * 128 listed rows, while a
    block whose list ends in the short last candidate block has fewer key tiles.
    A block's split s covers tiles [s*T/S, (s+1)*T/S) of its T tiles; with
    64-key tiles (INT8 at head dim 128, or head dim 64) and one listed 20-row
    block, the library plans S = 3 but the block has T = 2 tiles (1 cache + 1
    current), so split 0 is empty. The kernel writes such a split as O = 0,
    lse = -inf, which the merge weighs by 0 (GPU regression:
    test_gpu_sparse.py::test_split_without_key_tiles)."""
    L = nomas.lib()
    for D, dt, key_tile in ((128, nomas.NOMAS_KV_INT8, 64), (64, nomas.NOMAS_KV_BF16, 64),
                            (64, nomas.NOMAS_KV_INT8, 64)):
        S = L.nomas_segment_attention_splits(0, 16, 128, 2, D, dt, 3)
        assert S == 3
        T = -(-20 // key_tile) + -(-16 // key_tile)
        ranges = [(s * T // S, (s + 1) * T // S) for s in range(S)]
        assert ranges[0] == (0, 0) and sum(b - a for a, b in ranges) == T
    # bf16 at head dim 128 (128-key tiles) plans exactly the block's 2 tiles
    assert L.nomas_segment_attention_splits(0, 16, 128, 2, 128, nomas.NOMAS_KV_BF16, 3) == 2


def test_block_causal_rejects_before_launch():
    L = nomas.lib()
    segs = nomas._segments([(48, 16, 0), (48, 16, 2)])
    need = L.nomas_block_causal_attention_workspace_bytes(segs, 2, 24, 2, 64)
    # V^T of 128 rows: a 128-row pitch plus one 128-column block of padding (a
    # segment's partial tail tile reads a whole tile of columns)
    assert need == 2 * 64 * 256 * 2
    p = ctypes.c_void_p(1 << 24)
    ws = ctypes.c_void_p(1 << 26)

    def call(**kw):
        a = dict(q=p, k=p, v=p, ld=128, segs=segs, n=2, tpf=24, win=-1, H=2, D=64, out=p, ldo=128, lse=None,
                 scale=0.125, ws=ws, wsb=need)
        a.update(kw)
        return L.nomas_block_causal_attention(a["q"], a["k"], a["v"], a["ld"], a["segs"], a["n"], a["tpf"], a["win"],
                                              a["H"], a["D"], a["out"], a["ldo"], a["lse"], a["scale"], a["ws"],
                                              a["wsb"], None)
    assert call(n=0) == nomas.NOMAS_E_INVALID
    assert call(n=65) == nomas.NOMAS_E_INVALID
    assert call(tpf=25) == nomas.NOMAS_E_INVALID              # 48 video rows not a multiple
    assert call(segs=nomas._segments([(0, 0, 0), (48, 16, 2)])) == nomas.NOMAS_E_INVALID
    assert call(segs=nomas._segments([(48, 16, -1), (48, 16, 2)])) == nomas.NOMAS_E_INVALID
    assert call(D=96) == nomas.NOMAS_E_UNSUPPORTED
    assert call(q=None) == nomas.NOMAS_E_INVALID
    assert call(ld=64) == nomas.NOMAS_E_INVALID
    assert call(scale=0.0) == nomas.NOMAS_E_INVALID
    assert call(wsb=need - 1) == nomas.NOMAS_E_WORKSPACE
    assert call(ws=None) == nomas.NOMAS_E_WORKSPACE
    assert b"workspace" in L.nomas_last_error()
    assert call(ld=1 << 24, ldo=1 << 24) == nomas.NOMAS_E_INVALID     # 128 rows x 2**24 x 2 bytes
    assert b"2 GiB" in L.nomas_last_error()


def test_sparse_rejects_before_launch():
    L, d, _ = _desc(dtype=0, heads=2, dim=64, tpf=24, cap=4)
    d.frames_written = 4                        # 96 cached rows: 1 candidate block
    assert L.nomas_sparse_candidates(96) == 1 and L.nomas_sparse_candidates(129) == 2
    assert L.nomas_sparse_candidates(-1) == -1
    p = ctypes.c_void_p(1 << 24)
    ws = ctypes.c_void_p(1 << 26)
    need = L.nomas_sparse_select_workspace_bytes(64, 96, 2, 64)
    assert need > 0
    assert L.nomas_sparse_select(p, 128, 64, ctypes.byref(d), 2, p, ws, need, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_sparse_select(p, 128, 64, ctypes.byref(d), -1, p, ws, need, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_sparse_select(p, 128, 64, ctypes.byref(d), 1, None, ws, need, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_sparse_select(p, 128, 64, ctypes.byref(d), 1, p, ws, need - 1, None) == nomas.NOMAS_E_WORKSPACE
    assert L.nomas_sparse_select(p, 128, 64, ctypes.byref(d), 0, None, None, 0, None) == nomas.NOMAS_OK
    wsb = L.nomas_segment_attention_workspace_bytes(48, 16, 128, 2, 64, 0, 0)

    def att(**kw):
        a = dict(lst=p, n=1, ws=ws, wsb=wsb)
        a.update(kw)
        return L.nomas_segment_attention_sparse(p, p, p, 128, 48, 16, ctypes.byref(d), a["lst"], a["n"], p, 128, None,
                                                0.125, 0, a["ws"], a["wsb"], None)
    assert att(n=2) == nomas.NOMAS_E_INVALID
    assert att(n=-1) == nomas.NOMAS_E_INVALID
    assert att(lst=None) == nomas.NOMAS_E_INVALID
    assert att(lst=ctypes.c_void_p((1 << 24) + 2)) == nomas.NOMAS_E_INVALID
    assert att(wsb=0) == nomas.NOMAS_E_WORKSPACE


def test_archive_rejects_before_launch():
    L, d, _ = _desc(dtype=1, heads=2, dim=64, tpf=24, cap=4)
    rec = L.nomas_kvcache_record_bytes(ctypes.byref(d))
    assert rec == 2 * 24 * 64 * 2 + 2 * 2 * 24 * 4
    d.frames_written = 6                                   # retained frames 2..5
    host = ctypes.create_string_buffer(rec * 4)
    assert L.nomas_kvcache_export_frames(ctypes.byref(d), 1, 1, host, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_export_frames(ctypes.byref(d), 5, 2, host, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_export_frames(ctypes.byref(d), 2, 1, None, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_export_frames(ctypes.byref(d), 3, 0, None, None) == nomas.NOMAS_OK
    n = ctypes.c_int32(-1)
    p = ctypes.c_void_p(1 << 24)
    assert L.nomas_kvcache_append_archive(ctypes.byref(d), p, p, 128, 5, host, ctypes.byref(n), None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_append_archive(ctypes.byref(d), p, p, 128, 2, host, None, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_append_archive(ctypes.byref(d), p, p, 64, 2, host, ctypes.byref(n), None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_append_archive(ctypes.byref(d), p, p, 128, 2, None, ctypes.byref(n), None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_restore_frames(ctypes.byref(d), host, 0, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_kvcache_restore_frames(ctypes.byref(d), None, 1, None) == nomas.NOMAS_E_INVALID
    assert d.frames_written == 6 and n.value == -1


def test_qkv_projection_rejects_before_launch():
    L = nomas.lib()
    p = ctypes.c_void_p(1 << 24)
    ok = dict(x=p, ldx=2048, n=100, hid=2048, w=p, ldw=2048, H=16, D=128, nv=0, tab=None, y=p, ldy=6144)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.nomas_qkv_projection(a["x"], a["ldx"], a["n"], a["hid"], a["w"], a["ldw"], a["H"], a["D"], a["nv"],
                                      a["tab"], a["y"], a["ldy"], None)
    assert call(hid=2000) == nomas.NOMAS_E_INVALID           # not a multiple of 64
    assert call(ldx=2040) == nomas.NOMAS_E_INVALID
    assert call(ldy=6140) == nomas.NOMAS_E_INVALID
    assert call(nv=101) == nomas.NOMAS_E_INVALID
    assert call(D=96) == nomas.NOMAS_E_UNSUPPORTED
    assert call(x=None) == nomas.NOMAS_E_INVALID
    assert call(tab=ctypes.c_void_p((1 << 24) + 8)) == nomas.NOMAS_E_INVALID
    assert L.nomas_rope3d_table(p, 128, 0, 1, 2, 2, 32, 48, 40, 10000.0, 0, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_rope3d_table(None, 128, 0, 1, 2, 2, 32, 48, 48, 10000.0, 0, None) == nomas.NOMAS_E_INVALID


def test_noalloc_limit_and_refusal_on_the_host():
    """The no-allocation attention call states its scratch size and refuses
    sizes beyond it before touching the device (placeholder addresses)."""
    L = nomas.lib()
    cap = L.nomas_segment_attention_noalloc_max_bytes()
    assert cap == 64 << 20
    # the full single-layer shape without splits fits
    assert L.nomas_segment_attention_workspace_bytes(7680, 256, 17280, 16, 128, 0, 1) <= cap
    _, d, rc = _desc(dtype=0, heads=16, dim=128, tpf=960, cap=18)
    assert rc == 0
    d.frames_written = 18
    fake = ctypes.c_void_p(1 << 20)
    rc = L.nomas_segment_attention_noalloc(fake, fake, fake, 2048, 7680, 256, ctypes.byref(d), fake, 2048, None,
                                           0.088, 8, None)
    assert rc == nomas.NOMAS_E_WORKSPACE and b"scratch" in L.nomas_last_error()


def test_projection_append_rejects_before_launch_and_keeps_descriptor():
    L, d, rc = _desc(dtype=1, heads=2, dim=64, tpf=24, cap=4)
    assert rc == 0
    p = ctypes.c_void_p(1 << 24)
    def call(H=2, D=64, nv=48, desc=d):
        return L.nomas_qkv_projection_append(p, 128, 64, 128, p, 128, H, D, nv, None, p, 384, None, 0, desc, None)
    assert call(H=3) == nomas.NOMAS_E_INVALID and b"heads" in L.nomas_last_error()
    assert call(nv=40) == nomas.NOMAS_E_INVALID and b"multiple" in L.nomas_last_error()
    assert call(nv=0) == nomas.NOMAS_E_INVALID
    assert call(desc=None) == nomas.NOMAS_E_INVALID
    assert d.frames_written == 0


def test_projection_vt_rejects_bad_transposed_output():
    L = nomas.lib()
    p = ctypes.c_void_p(1 << 24)
    def call(vt=p, ld_vt=64, n=64):
        return L.nomas_qkv_projection_vt(p, 128, n, 128, p, 128, 2, 64, 0, None, p, 384, vt, ld_vt, None)
    assert call(vt=None) == nomas.NOMAS_E_INVALID
    assert call(vt=ctypes.c_void_p((1 << 24) + 8)) == nomas.NOMAS_E_INVALID and b"v_t" in L.nomas_last_error()
    assert call(ld_vt=56) == nomas.NOMAS_E_INVALID      # fewer columns than rows
    assert call(ld_vt=68) == nomas.NOMAS_E_INVALID      # not a multiple of 8
    L2, d, rc = _desc(dtype=1, heads=2, dim=64, tpf=24, cap=4)
    assert L2.nomas_qkv_projection_append(p, 128, 64, 128, p, 128, 2, 64, 48, None, p, 384, p, 60, ctypes.byref(d),
                                          None) == nomas.NOMAS_E_INVALID
    assert d.frames_written == 0


def test_attention_frames_rejects_frames_not_retained():
    """Frame ranges outside the retained frames, a missing value input and a bad
    V^T are refused before anything is enqueued; the descriptor is unchanged."""
    L, d, rc = _desc(dtype=1, heads=2, dim=64, tpf=24, cap=4)
    assert rc == 0
    d.frames_written = 6                                   # retained: frames [2, 6)
    p = ctypes.c_void_p(1 << 24)
    ws = ctypes.c_void_p(1 << 26)
    def call(first, n, v=p, vt=None, ld_vt=0):
        return L.nomas_segment_attention_frames(p, p, v, 384, vt, ld_vt, 48, 16, ctypes.byref(d), first, n, p, 128,
                                                None, ctypes.c_float(0.125), 0, ws, 1 << 30, None)
    assert call(1, 3) == nomas.NOMAS_E_INVALID and b"retained" in L.nomas_last_error()
    assert call(3, 4) == nomas.NOMAS_E_INVALID            # runs past frames_written
    assert call(2, -1) == nomas.NOMAS_E_INVALID
    assert call(2, 4, v=None) == nomas.NOMAS_E_INVALID    # neither v_cur nor v_t
    assert call(2, 4, v=None, vt=p, ld_vt=64) == nomas.NOMAS_E_INVALID   # below round_up(n_q = 64, 128)
    assert call(2, 4, v=None, vt=p, ld_vt=132) == nomas.NOMAS_E_INVALID  # not a multiple of 8
    assert call(2, 4, v=None, vt=ctypes.c_void_p((1 << 24) + 2), ld_vt=128) == nomas.NOMAS_E_INVALID
    small = L.nomas_segment_attention_frames(p, p, p, 384, None, 0, 48, 16, ctypes.byref(d), 3, 2, p, 128, None,
                                             ctypes.c_float(0.125), 0, ws, 64, None)
    assert small == nomas.NOMAS_E_WORKSPACE
    assert d.frames_written == 6


def test_lds_stream_calibration_sizes_and_refusals():
    """The counter-calibration stream takes whole KiB and one sink word per MiB
    slice, and refuses other sizes and misaligned buffers before any launch."""
    L = nomas.lib()
    assert [L.nomas_calibrate_lds_stream_blocks(b) for b in (0, -1024, 1000, 1024, 1 << 20, (1 << 20) + 1024)] == \
        [-1, -1, -1, 1, 1, 2]
    dummy = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below is refused on the host
    assert L.nomas_calibrate_lds_stream(dummy, 1000, dummy, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_calibrate_lds_stream(None, 1024, dummy, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_calibrate_lds_stream(ctypes.c_void_p((1 << 20) + 8), 1024, dummy, None) == nomas.NOMAS_E_INVALID
    assert L.nomas_calibrate_lds_stream(dummy, 1024, ctypes.c_void_p((1 << 20) + 2), None) == nomas.NOMAS_E_INVALID
