"""Thin Python binding of libnomas.so (argument marshalling only).

Every function here has the name of the C entry point it forwards to, and does
nothing but check tensor dtypes/devices/strides, take device pointers, and pass
the caller's current HIP stream. All computation happens in the library's HIP
kernels; there is no fallback: if the library is missing or does not load, the
first call raises.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnomas.so")

NOMAS_OK, NOMAS_E_INVALID, NOMAS_E_UNSUPPORTED, NOMAS_E_WORKSPACE, NOMAS_E_HIP = range(5)
NOMAS_KV_BF16, NOMAS_KV_INT8 = 0, 1
NOMAS_SPARSE_KEY_BLOCK, NOMAS_SPARSE_QUERY_BLOCK = 128, 256


class NomasError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[nomas status {code}] {msg}")
        self.code = code


class KVCacheDesc(ctypes.Structure):
    """Mirror of ``nomas_kvcache`` in include/nomas.h."""
    _fields_ = [
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tokens_per_frame", ctypes.c_int32),
        ("capacity_frames", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("token_pitch", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("frames_written", ctypes.c_int64),
    ]


class Segment(ctypes.Structure):
    """Mirror of ``nomas_segment`` in include/nomas.h."""
    _fields_ = [("n_video", ctypes.c_int32), ("n_text", ctypes.c_int32), ("t0", ctypes.c_int32)]


_lib = None


def lib():
    """Load libnomas.so once (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m segment_autoregressive_dit_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    desc_p = ctypes.POINTER(KVCacheDesc)
    seg_p = ctypes.POINTER(Segment)
    sig = {
        "nomas_version": (i32, []),
        "nomas_calibrate_lds_stream_blocks": (i64, [i64]),
        "nomas_calibrate_lds_stream": (i32, [vp, i64, vp, vp]),
        "nomas_device_check_failures": (i64, [i32]),
        "nomas_last_error": (ctypes.c_char_p, []),
        "nomas_kvcache_token_pitch": (i64, [i32, i32]),
        "nomas_kvcache_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
        "nomas_kvcache_init": (i32, [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
        "nomas_kvcache_valid_frames": (i64, [desc_p]),
        "nomas_rope3d": (i32, [vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]),
        "nomas_kvcache_append": (i32, [desc_p, vp, vp, i64, i32, vp]),
        "nomas_segment_attention_workspace_bytes": (sz, [i32, i32, i64, i32, i32, i32, i32]),
        "nomas_segment_attention_splits": (i32, [i32, i32, i64, i32, i32, i32, i32]),
        "nomas_segment_attention": (i32, [vp, vp, vp, i64, i32, i32, desc_p, vp, i64, vp, f32, i32, vp, sz, vp]),
        "nomas_block_causal_attention_workspace_bytes": (sz, [seg_p, i32, i32, i32, i32]),
        "nomas_sparse_candidates": (i32, [i64]),
        "nomas_rope3d_table": (i32, [vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]),
        "nomas_qkv_projection": (i32, [vp, i64, i32, i32, vp, i64, i32, i32, i32, vp, vp, i64, vp]),
        "nomas_kvcache_record_bytes": (sz, [desc_p]),
        "nomas_kvcache_export_frames": (i32, [desc_p, i64, i32, vp, vp]),
        "nomas_kvcache_append_archive": (i32, [desc_p, vp, vp, i64, i32, vp, ctypes.POINTER(i32), vp]),
        "nomas_kvcache_restore_frames": (i32, [desc_p, vp, i32, vp]),
        "nomas_sparse_select_workspace_bytes": (sz, [i32, i64, i32, i32]),
        "nomas_sparse_select": (i32, [vp, i64, i32, desc_p, i32, vp, vp, sz, vp]),
        "nomas_segment_attention_sparse": (i32, [vp, vp, vp, i64, i32, i32, desc_p, vp, i32, vp, i64, vp, f32, i32,
                                                 vp, sz, vp]),
        "nomas_block_causal_attention": (i32, [vp, vp, vp, i64, seg_p, i32, i32, i32, i32, i32, vp, i64, vp, f32,
                                               vp, sz, vp]),
        "nomas_qkv_projection_append": (i32, [vp, i64, i32, i32, vp, i64, i32, i32, i32, vp, vp, i64, vp, i64, desc_p,
                                              vp]),
        "nomas_qkv_projection_vt": (i32, [vp, i64, i32, i32, vp, i64, i32, i32, i32, vp, vp, i64, vp, i64, vp]),
        "nomas_segment_attention_frames": (i32, [vp, vp, vp, i64, vp, i64, i32, i32, desc_p, i64, i32, vp, i64, vp, f32,
                                                 i32, vp, sz, vp]),
        "nomas_segment_attention_noalloc_max_bytes": (sz, []),
        "nomas_segment_attention_noalloc": (i32, [vp, vp, vp, i64, i32, i32, desc_p, vp, i64, vp, f32, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(code):
    if code != NOMAS_OK:
        raise NomasError(code, lib().nomas_last_error().decode())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(t, stream):
    """Mark a temporary allocated here as in use by ``stream`` when the caller
    names a stream other than the current one, so that the caching allocator
    does not hand its memory out again before the library's kernels on that
    stream are done with it."""
    if stream is not None and t is not None:
        t.record_stream(stream)
    return t


def _rows_view(t, name, heads, head_dim):
    """(pointer, row stride) of a bf16 device tensor laid out [rows, ...heads*head_dim]."""
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a bfloat16 CUDA tensor")
    if t.dim() == 3:
        if t.shape[1] != heads or t.shape[2] != head_dim or t.stride(2) != 1 or t.stride(1) != head_dim:
            raise ValueError(f"{name}: expected [rows, {heads}, {head_dim}] with contiguous heads")
    elif t.dim() == 2:
        if t.shape[1] < heads * head_dim or t.stride(1) != 1:
            raise ValueError(f"{name}: expected [rows, >= {heads * head_dim}] with unit inner stride")
    else:
        raise ValueError(f"{name}: expected a 2-D or 3-D tensor")
    return ctypes.c_void_p(t.data_ptr()), t.stride(0)


def _host_buffer(t, nbytes, name):
    if t.device.type != "cpu" or t.dtype != torch.uint8 or not t.is_contiguous() or t.numel() < nbytes:
        raise ValueError(f"{name} must be a contiguous uint8 host tensor of at least {nbytes} bytes")


def nomas_version():
    return lib().nomas_version()


def nomas_device_check_failures(reset=False):
    """Failed device-side index checks since the last reset (the checking
    build, libnomas_debug.so), or -1 for the normal build."""
    return lib().nomas_device_check_failures(int(bool(reset)))


def nomas_kvcache_bytes(n_heads, head_dim, tokens_per_frame, capacity_frames, kv_dtype, which):
    return lib().nomas_kvcache_bytes(n_heads, head_dim, tokens_per_frame, capacity_frames, kv_dtype, which)


class KVCache:
    """Device buffers + descriptor of one layer's ring cache (see nomas_kvcache)."""

    def __init__(self, n_heads, head_dim, tokens_per_frame, capacity_frames, int8, device="cuda"):
        L = lib()
        dt = NOMAS_KV_INT8 if int8 else NOMAS_KV_BF16
        nb = [L.nomas_kvcache_bytes(n_heads, head_dim, tokens_per_frame, capacity_frames, dt, w) for w in range(3)]
        if nb[0] == 0:
            _check(L.nomas_kvcache_init(ctypes.byref(KVCacheDesc()), n_heads, head_dim, tokens_per_frame,
                                        capacity_frames, dt, None, None, None, None))
        self.k = torch.empty(nb[0], dtype=torch.uint8, device=device)
        self.v = torch.empty(nb[1], dtype=torch.uint8, device=device)
        self.k_scale = torch.empty(nb[2] // 4, dtype=torch.float32, device=device) if int8 else None
        self.v_scale = torch.empty(nb[2] // 4, dtype=torch.float32, device=device) if int8 else None
        self.desc = KVCacheDesc()
        _check(L.nomas_kvcache_init(
            ctypes.byref(self.desc), n_heads, head_dim, tokens_per_frame, capacity_frames, dt,
            ctypes.c_void_p(self.k.data_ptr()), ctypes.c_void_p(self.v.data_ptr()),
            ctypes.c_void_p(self.k_scale.data_ptr()) if int8 else None,
            ctypes.c_void_p(self.v_scale.data_ptr()) if int8 else None))
        self.int8 = int8

    @property
    def frames_written(self):
        return self.desc.frames_written

    @property
    def valid_frames(self):
        return lib().nomas_kvcache_valid_frames(ctypes.byref(self.desc))

    @property
    def token_pitch(self):
        return self.desc.token_pitch

    @property
    def n_cached(self):
        return self.valid_frames * self.desc.tokens_per_frame

    def nomas_kvcache_record_bytes(self):
        return lib().nomas_kvcache_record_bytes(ctypes.byref(self.desc))

    def host_records(self, n_frames):
        """A pinned host buffer for n_frames archive records."""
        return torch.empty(max(1, n_frames) * self.nomas_kvcache_record_bytes(), dtype=torch.uint8, pin_memory=True)

    def nomas_kvcache_export_frames(self, first_frame, n_frames, host_dst, stream=None):
        """Records of retained frames [first_frame, +n_frames) -> host_dst (uint8 CPU tensor)."""
        _host_buffer(host_dst, n_frames * self.nomas_kvcache_record_bytes(), "host_dst")
        _check(lib().nomas_kvcache_export_frames(ctypes.byref(self.desc), first_frame, n_frames,
                                                 ctypes.c_void_p(host_dst.data_ptr()), _stream(stream)))

    def nomas_kvcache_append_archive(self, k_new, v_new, n_frames, host_evicted, stream=None):
        """Append that first exports the frames it overwrites; returns their count."""
        H, D = self.desc.n_heads, self.desc.head_dim
        kp, ld = _rows_view(k_new, "k_new", H, D)
        vp, ldv = _rows_view(v_new, "v_new", H, D)
        if ld != ldv:
            raise ValueError("k_new and v_new must share a row stride")
        if k_new.shape[0] < n_frames * self.desc.tokens_per_frame:
            raise ValueError("k_new/v_new hold fewer rows than n_frames frames")
        _host_buffer(host_evicted, n_frames * self.nomas_kvcache_record_bytes(), "host_evicted")
        n_ev = ctypes.c_int32(0)
        _check(lib().nomas_kvcache_append_archive(ctypes.byref(self.desc), kp, vp, ld, n_frames,
                                                  ctypes.c_void_p(host_evicted.data_ptr()), ctypes.byref(n_ev),
                                                  _stream(stream)))
        return n_ev.value

    def nomas_kvcache_restore_frames(self, host_src, n_frames, stream=None):
        _host_buffer(host_src, n_frames * self.nomas_kvcache_record_bytes(), "host_src")
        _check(lib().nomas_kvcache_restore_frames(ctypes.byref(self.desc), ctypes.c_void_p(host_src.data_ptr()),
                                                  n_frames, _stream(stream)))

    def nomas_kvcache_append(self, k_new, v_new, n_frames, stream=None):
        d = self.desc
        kp, ld = _rows_view(k_new, "k_new", d.n_heads, d.head_dim)
        vp, ldv = _rows_view(v_new, "v_new", d.n_heads, d.head_dim)
        if ld != ldv:
            raise ValueError("k_new and v_new must share a row stride")
        if k_new.shape[0] < n_frames * d.tokens_per_frame or v_new.shape[0] < n_frames * d.tokens_per_frame:
            raise ValueError("k_new/v_new hold fewer than n_frames*tokens_per_frame rows")
        _check(lib().nomas_kvcache_append(ctypes.byref(d), kp, vp, ld, n_frames, _stream(stream)))


def nomas_rope3d(q, k, t0, n_frames, grid_h, grid_w, band, n_heads, head_dim, theta=10000.0,
                 inverse=False, stream=None):
    """Rotate the first n_frames*grid_h*grid_w rows of q (and k) in place."""
    qp, ld = _rows_view(q, "q", n_heads, head_dim)
    kp = ctypes.c_void_p(0)
    if k is not None:
        kp, ldk = _rows_view(k, "k", n_heads, head_dim)
        if ldk != ld:
            raise ValueError("q and k must share a row stride")
        if k.shape[0] < n_frames * grid_h * grid_w:
            raise ValueError("k holds fewer rows than the segment's video tokens")
    if q.shape[0] < n_frames * grid_h * grid_w:
        raise ValueError("q holds fewer rows than the segment's video tokens")
    d_t, d_h, d_w = band
    _check(lib().nomas_rope3d(qp, kp, ld, n_heads, head_dim, t0, n_frames, grid_h, grid_w,
                              d_t, d_h, d_w, float(theta), int(bool(inverse)), _stream(stream)))


def nomas_calibrate_lds_stream(src, sink=None, stream=None):
    """Fetch every byte of the contiguous CUDA tensor ``src`` once by global ->
    LDS copies (the counter calibration of that access pattern); ``sink``:
    int32 [nomas_calibrate_lds_stream_blocks(bytes)], allocated if not given."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous CUDA tensor")
    nbytes = src.numel() * src.element_size()
    blocks = lib().nomas_calibrate_lds_stream_blocks(nbytes)
    if blocks < 1:
        raise ValueError("src must hold a positive multiple of 1024 bytes")
    if sink is None:
        sink = _on_stream(torch.empty(blocks, dtype=torch.int32, device=src.device), stream)
    elif sink.dtype != torch.int32 or not sink.is_cuda or not sink.is_contiguous() or sink.numel() < blocks:
        raise ValueError(f"sink must be a contiguous int32 CUDA tensor of at least {blocks} elements")
    _check(lib().nomas_calibrate_lds_stream(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                            _stream(stream)))
    return sink


def nomas_segment_attention_workspace_bytes(n_video, n_text, n_cached, n_heads, head_dim, kv_dtype, n_splits=0):
    return lib().nomas_segment_attention_workspace_bytes(n_video, n_text, n_cached, n_heads, head_dim, kv_dtype,
                                                         n_splits)


def nomas_segment_attention_splits(n_video, n_text, n_cached, n_heads, head_dim, kv_dtype, n_splits=0):
    return lib().nomas_segment_attention_splits(n_video, n_text, n_cached, n_heads, head_dim, kv_dtype, n_splits)


def workspace_for(cache, n_video, n_text, n_splits=0, device="cuda"):
    d = cache.desc
    nb = nomas_segment_attention_workspace_bytes(n_video, n_text, cache.n_cached, d.n_heads, d.head_dim, d.kv_dtype,
                                                 n_splits)
    return torch.empty(max(nb, 256), dtype=torch.uint8, device=device)


def nomas_segment_attention(q, k_cur, v_cur, n_video, n_text, cache, out=None, lse=None, softmax_scale=None,
                            n_splits=0, workspace=None, stream=None):
    """Attention of the current segment's rows against cache + current segment.

    Returns ``out`` ([n_q, H, D] bf16, allocated if not given)."""
    return _segment_attention(q, k_cur, v_cur, n_video, n_text, cache, None, out, lse, softmax_scale, n_splits,
                              workspace, stream)


def nomas_segment_attention_sparse(q, k_cur, v_cur, n_video, n_text, cache, block_list, out=None, lse=None,
                                   softmax_scale=None, n_splits=0, workspace=None, stream=None):
    """nomas_segment_attention restricted to the candidate blocks of ``block_list``
    (int32 [H, ceil(n_q/256), n_select], ascending lists of 128-row cache blocks)."""
    return _segment_attention(q, k_cur, v_cur, n_video, n_text, cache, block_list, out, lse, softmax_scale, n_splits,
                              workspace, stream)


def nomas_segment_attention_frames(q, k_cur, v_cur, n_video, n_text, cache, first_frame, n_frames, v_t=None,
                                   out=None, lse=None, softmax_scale=None, n_splits=0, workspace=None, stream=None):
    """Attention against the retained frames [first_frame, first_frame + n_frames)
    of ``cache`` and the current segment; with ``v_t`` (bf16 [H*D, ld_vt], the V^T
    nomas_qkv_projection_vt writes) the values come from it and ``v_cur`` may be
    None. Returns ``out``."""
    d = cache.desc
    H, D = d.n_heads, d.head_dim
    n_q = n_video + n_text
    qp, ld = _rows_view(q, "q", H, D)
    kp, ldk = _rows_view(k_cur, "k_cur", H, D)
    vp = None
    if v_cur is not None:
        vp, ldv = _rows_view(v_cur, "v_cur", H, D)
        if ldv != ld or v_cur.shape[0] < n_q:
            raise ValueError("v_cur must share q's row stride and hold n_video + n_text rows")
    if ld != ldk:
        raise ValueError("q, k_cur must share a row stride")
    for t, name in ((q, "q"), (k_cur, "k_cur")):
        if t.shape[0] < n_q:
            raise ValueError(f"{name} holds fewer than n_video + n_text rows")
    tp, ld_vt = None, 0
    if v_t is not None:
        if v_t.dtype != torch.bfloat16 or v_t.dim() != 2 or v_t.stride(1) != 1 or v_t.shape[0] != H * D:
            raise ValueError(f"v_t must be a 2-D bfloat16 tensor [{H * D}, ld_vt] with unit inner stride")
        tp, ld_vt = ctypes.c_void_p(v_t.data_ptr()), v_t.stride(0)
    if out is None:
        out = _on_stream(torch.empty((n_q, H, D), dtype=torch.bfloat16, device=q.device), stream)
    op, ldo = _rows_view(out, "out", H, D)
    if out.shape[0] < n_q:
        raise ValueError("out holds fewer than n_video + n_text rows")
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() < H * n_q:
            raise ValueError("lse must be a contiguous float32 tensor of n_heads*n_q elements")
        lp = ctypes.c_void_p(lse.data_ptr())
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if workspace is None:
        nb = nomas_segment_attention_workspace_bytes(n_video, n_text, max(0, n_frames) * d.tokens_per_frame, H, D,
                                                     d.kv_dtype, n_splits)
        workspace = _on_stream(torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device), stream)
    _check(lib().nomas_segment_attention_frames(qp, kp, vp, ld, tp, ld_vt, n_video, n_text, ctypes.byref(d),
                                                int(first_frame), int(n_frames), op, ldo, lp, scale, n_splits,
                                                ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                                _stream(stream)))
    return out


def nomas_segment_attention_noalloc_max_bytes():
    return lib().nomas_segment_attention_noalloc_max_bytes()


def nomas_segment_attention_noalloc(q, k_cur, v_cur, n_video, n_text, cache, out, lse=None, softmax_scale=None,
                                    n_splits=0, stream=None):
    """nomas_segment_attention without a workspace (the library's own scratch
    array, see nomas.h); nothing is allocated here either, so ``out`` is
    required. Returns ``out``."""
    d = cache.desc
    H, D = d.n_heads, d.head_dim
    n_q = n_video + n_text
    qp, ld = _rows_view(q, "q", H, D)
    kp, ldk = _rows_view(k_cur, "k_cur", H, D)
    vp, ldv = _rows_view(v_cur, "v_cur", H, D)
    if not (ld == ldk == ldv):
        raise ValueError("q, k_cur, v_cur must share a row stride")
    for t, name in ((q, "q"), (k_cur, "k_cur"), (v_cur, "v_cur"), (out, "out")):
        if t.shape[0] < n_q:
            raise ValueError(f"{name} holds fewer than n_video + n_text rows")
    op, ldo = _rows_view(out, "out", H, D)
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() < H * n_q:
            raise ValueError("lse must be a contiguous float32 tensor of n_heads*n_q elements")
        lp = ctypes.c_void_p(lse.data_ptr())
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().nomas_segment_attention_noalloc(qp, kp, vp, ld, n_video, n_text, ctypes.byref(d), op, ldo, lp, scale,
                                                 n_splits, _stream(stream)))
    return out


def nomas_sparse_candidates(n_cached):
    return lib().nomas_sparse_candidates(n_cached)


def nomas_sparse_select(q, n_q, cache, n_select, block_list=None, workspace=None, stream=None):
    """Candidate blocks per head and 256-row query block (see nomas.h); returns
    ``block_list`` (int32 [H, ceil(n_q/256), n_select])."""
    d = cache.desc
    H, D = d.n_heads, d.head_dim
    qp, ld = _rows_view(q, "q", H, D)
    if q.shape[0] < n_q:
        raise ValueError("q holds fewer than n_q rows")
    nqb = (n_q + NOMAS_SPARSE_QUERY_BLOCK - 1) // NOMAS_SPARSE_QUERY_BLOCK
    if block_list is None:
        block_list = _on_stream(torch.empty((H, nqb, max(n_select, 1)), dtype=torch.int32, device=q.device),
                                stream)[:, :, :n_select]
    if block_list.dtype != torch.int32 or not block_list.is_contiguous() or block_list.numel() < H * nqb * n_select:
        raise ValueError("block_list must be a contiguous int32 tensor of n_heads*n_qblocks*n_select elements")
    if workspace is None:
        nb = lib().nomas_sparse_select_workspace_bytes(n_q, cache.n_cached, H, D)
        workspace = _on_stream(torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device), stream)
    _check(lib().nomas_sparse_select(qp, ld, n_q, ctypes.byref(d), n_select, ctypes.c_void_p(block_list.data_ptr()),
                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
    return block_list


def _segment_attention(q, k_cur, v_cur, n_video, n_text, cache, block_list, out, lse, softmax_scale, n_splits,
                       workspace, stream):
    d = cache.desc
    H, D = d.n_heads, d.head_dim
    n_q = n_video + n_text
    qp, ld = _rows_view(q, "q", H, D)
    kp, ldk = _rows_view(k_cur, "k_cur", H, D)
    vp, ldv = _rows_view(v_cur, "v_cur", H, D)
    if not (ld == ldk == ldv):
        raise ValueError("q, k_cur, v_cur must share a row stride")
    for t, name in ((q, "q"), (k_cur, "k_cur"), (v_cur, "v_cur")):
        if t.shape[0] < n_q:
            raise ValueError(f"{name} holds fewer than n_video + n_text rows")
    if out is None:
        out = _on_stream(torch.empty((n_q, H, D), dtype=torch.bfloat16, device=q.device), stream)
    op, ldo = _rows_view(out, "out", H, D)
    if out.shape[0] < n_q:
        raise ValueError("out holds fewer than n_video + n_text rows")
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() < H * n_q:
            raise ValueError("lse must be a contiguous float32 tensor of n_heads*n_q elements")
        lp = ctypes.c_void_p(lse.data_ptr())
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if block_list is None:
        if workspace is None:
            workspace = _on_stream(workspace_for(cache, n_video, n_text, n_splits, q.device), stream)
        _check(lib().nomas_segment_attention(qp, kp, vp, ld, n_video, n_text, ctypes.byref(d), op, ldo, lp, scale,
                                             n_splits, ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                             _stream(stream)))
        return out
    nqb = (n_q + NOMAS_SPARSE_QUERY_BLOCK - 1) // NOMAS_SPARSE_QUERY_BLOCK
    if block_list.dtype != torch.int32 or block_list.dim() != 3 or block_list.shape[:2] != (H, nqb):
        raise ValueError(f"block_list must be int32 [{H}, {nqb}, n_select]")
    n_select = block_list.shape[2]
    if not block_list.is_contiguous():
        block_list = _on_stream(block_list.contiguous(), stream)
    if workspace is None:
        nb = nomas_segment_attention_workspace_bytes(n_video, n_text, n_select * NOMAS_SPARSE_KEY_BLOCK, H, D,
                                                     d.kv_dtype, n_splits)
        workspace = _on_stream(torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device), stream)
    _check(lib().nomas_segment_attention_sparse(qp, kp, vp, ld, n_video, n_text, ctypes.byref(d),
                                                ctypes.c_void_p(block_list.data_ptr()), n_select, op, ldo, lp, scale,
                                                n_splits, ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                                _stream(stream)))
    return out


def _segments(segments):
    """[(n_video, n_text, t0), ...] -> ctypes array of nomas_segment."""
    arr = (Segment * len(segments))()
    for i, (nv, nt, t0) in enumerate(segments):
        arr[i] = Segment(int(nv), int(nt), int(t0))
    return arr


def nomas_block_causal_attention_workspace_bytes(segments, tokens_per_frame, n_heads, head_dim):
    return lib().nomas_block_causal_attention_workspace_bytes(_segments(segments), len(segments), tokens_per_frame,
                                                              n_heads, head_dim)


def nomas_block_causal_attention(q, k, v, segments, tokens_per_frame, window_frames, n_heads, head_dim, out=None,
                                 lse=None, softmax_scale=None, workspace=None, stream=None):
    """Block-causal attention over several segments at once.

    ``segments``: [(n_video, n_text, t0), ...] in sequence order; q, k, v hold
    their rows [video_0; text_0; video_1; ...]. ``window_frames`` < 0: no window.
    Returns ``out`` ([n_rows, H, D] bf16, allocated if not given)."""
    H, D = n_heads, head_dim
    segs = _segments(segments)
    n_rows = sum(int(nv) + int(nt) for nv, nt, _ in segments)
    qp, ld = _rows_view(q, "q", H, D)
    kp, ldk = _rows_view(k, "k", H, D)
    vp, ldv = _rows_view(v, "v", H, D)
    if not (ld == ldk == ldv):
        raise ValueError("q, k, v must share a row stride")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.shape[0] < n_rows:
            raise ValueError(f"{name} holds fewer rows than the segments")
    if out is None:
        out = _on_stream(torch.empty((n_rows, H, D), dtype=torch.bfloat16, device=q.device), stream)
    op, ldo = _rows_view(out, "out", H, D)
    if out.shape[0] < n_rows:
        raise ValueError("out holds fewer rows than the segments")
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() < H * n_rows:
            raise ValueError("lse must be a contiguous float32 tensor of n_heads*n_rows elements")
        lp = ctypes.c_void_p(lse.data_ptr())
    if workspace is None:
        nb = nomas_block_causal_attention_workspace_bytes(segments, tokens_per_frame, H, D)
        workspace = _on_stream(torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device), stream)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().nomas_block_causal_attention(qp, kp, vp, ld, segs, len(segments), tokens_per_frame, window_frames,
                                              H, D, op, ldo, lp, scale, ctypes.c_void_p(workspace.data_ptr()),
                                              workspace.numel(), _stream(stream)))
    return out


def nomas_rope3d_table(head_dim, t0, n_frames, grid_h, grid_w, band, theta=10000.0, inverse=False, table=None,
                       stream=None):
    """(cos, sin) table [n_frames*grid_h*grid_w, head_dim/2, 2] float32 of a segment's video rows;
    None for a segment without video rows (nothing to rotate: pass rope_table=None)."""
    n = n_frames * grid_h * grid_w
    if n == 0:
        return None
    if table is None:
        table = _on_stream(torch.empty((n, head_dim // 2, 2), dtype=torch.float32, device="cuda"), stream)
    if table.dtype != torch.float32 or not table.is_cuda or not table.is_contiguous() or table.numel() < n * head_dim:
        raise ValueError("table must be a contiguous float32 CUDA tensor of n_rows*head_dim elements")
    d_t, d_h, d_w = band
    _check(lib().nomas_rope3d_table(ctypes.c_void_p(table.data_ptr()), head_dim, t0, n_frames, grid_h, grid_w, d_t,
                                    d_h, d_w, float(theta), int(bool(inverse)), _stream(stream)))
    return table


def new_vt(n_rows, n_heads, head_dim, device="cuda", stream=None):
    """A V^T buffer for nomas_qkv_projection_vt: bf16 [H*D, round_up(n_rows, 128)]."""
    return _on_stream(torch.empty((n_heads * head_dim, (n_rows + 127) // 128 * 128), dtype=torch.bfloat16,
                                  device=device), stream)


def nomas_qkv_projection(x, w, n_heads, head_dim, n_video=0, rope_table=None, qkv=None, stream=None, cache=None,
                         v_t=None):
    """qkv = [q | k | v] projection of x [n, hidden] by w [3*H*D, hidden] with RoPE
    on the video rows' q, k (when a table is given). Returns qkv [n, 3*H*D].
    With ``v_t`` (bf16 [H*D, ld_vt]) the values are also written transposed
    (nomas_qkv_projection_vt). With ``cache`` (a KVCache):
    nomas_qkv_projection_append, which also appends the n_video rows' keys and
    values to it."""
    for t, name in ((x, "x"), (w, "w")):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be a 2-D bfloat16 CUDA tensor with unit inner stride")
    n, hidden = x.shape
    n_ch = 3 * n_heads * head_dim
    if w.shape[0] != n_ch or w.shape[1] != hidden:
        raise ValueError(f"w must be [{n_ch}, {hidden}]")
    if qkv is None:
        qkv = _on_stream(torch.empty((n, n_ch), dtype=torch.bfloat16, device=x.device), stream)
    if qkv.dtype != torch.bfloat16 or qkv.dim() != 2 or qkv.stride(1) != 1 or qkv.shape[0] < n or qkv.shape[1] < n_ch:
        raise ValueError("qkv must be a 2-D bfloat16 tensor of at least [n, 3*H*D] with unit inner stride")
    tp = None
    if rope_table is not None:
        if rope_table.dtype != torch.float32 or not rope_table.is_contiguous() or \
                rope_table.numel() < n_video * head_dim:
            raise ValueError("rope_table must be a contiguous float32 tensor of n_video*head_dim elements")
        tp = ctypes.c_void_p(rope_table.data_ptr())
    args = (ctypes.c_void_p(x.data_ptr()), x.stride(0), n, hidden, ctypes.c_void_p(w.data_ptr()), w.stride(0),
            n_heads, head_dim, n_video, tp, ctypes.c_void_p(qkv.data_ptr()), qkv.stride(0))
    vt_args = (None, 0)
    if v_t is not None:
        if v_t.dtype != torch.bfloat16 or v_t.dim() != 2 or v_t.stride(1) != 1 or v_t.shape[0] != n_heads * head_dim \
                or v_t.shape[1] < n:
            raise ValueError(f"v_t must be a 2-D bfloat16 tensor of [{n_heads * head_dim}, >= n] with unit inner stride")
        vt_args = (ctypes.c_void_p(v_t.data_ptr()), v_t.stride(0))
    if cache is not None:
        _check(lib().nomas_qkv_projection_append(*args, *vt_args, ctypes.byref(cache.desc), _stream(stream)))
    elif v_t is not None:
        _check(lib().nomas_qkv_projection_vt(*args, *vt_args, _stream(stream)))
    else:
        _check(lib().nomas_qkv_projection(*args, _stream(stream)))
    return qkv


def nomas_qkv_projection_vt(x, w, n_heads, head_dim, n_video, rope_table, v_t, qkv=None, stream=None):
    """nomas_qkv_projection that also writes the values transposed into ``v_t``
    (see new_vt). Returns qkv."""
    return nomas_qkv_projection(x, w, n_heads, head_dim, n_video=n_video, rope_table=rope_table, qkv=qkv,
                                stream=stream, v_t=v_t)


def nomas_qkv_projection_append(x, w, n_heads, head_dim, n_video, rope_table, cache, qkv=None, stream=None,
                                v_t=None):
    """The final-step projection: nomas_qkv_projection that also appends the
    n_video rows' keys and values to ``cache`` (and, with ``v_t``, writes the
    values transposed). Returns qkv."""
    return nomas_qkv_projection(x, w, n_heads, head_dim, n_video=n_video, rope_table=rope_table, qkv=qkv,
                                stream=stream, cache=cache, v_t=v_t)
