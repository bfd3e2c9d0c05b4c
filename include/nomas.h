/*
 * nomas.h -- C ABI of libnomas.so: the segment-attention hot path of a
 * segment-autoregressive video diffusion transformer, for AMD MI355X (gfx950).
 *
 * The path, as the pages describe the model:
 *   - the DiT renders one video segment at a time and conditions it on a cache
 *     of earlier latents' keys and values ("Hy-Nomas: Was Tencent mit seinem frei
 *     formbaren interaktiven Weltmodell tatsaechlich macht", orcarouter.ai,
 *     section "Die Schleife");
 *   - 54 double-stream blocks, hidden 2048 = 16 heads x 128, 3D RoPE
 *     ("Hy-Nomas auf einer RTX 4090", inferencekey.com, section
 *     "Modell und Dateien");
 *   - on one GPU the cache keeps a window of the last 18 latent frames, stored
 *     INT8 and computed BF16 (same page, section "Das Single-GPU-Preset";
 *     blog.authon.dev config excerpt: kv_cache_quantization: int8,
 *     sliding_window.past_frames: 18);
 *   - segment-wise causal joint attention (madebyagents.com model page
 *     "Hy-Nomas", component "Segment-Autoregressive DiT").
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are HIP device pointers, (host) are host memory.
 *     bf16 data is passed as uint16_t bit patterns.
 *   - The caller owns all memory. The library never allocates, frees or
 *     synchronises; every compute call enqueues kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and returns.
 *     (One exception: nomas_segment_attention_noalloc uses a scratch array
 *     the library itself holds, for callers that cannot allocate.)
 *   - Every call returns a nomas_status. All arguments are checked on the host
 *     before anything is enqueued: on an error nothing is enqueued, the cache
 *     descriptor is unchanged, and nomas_last_error() describes the problem.
 *     NOMAS_E_HIP reports a failed kernel launch (hipGetErrorString text).
 *   - Inputs holding NaN or Inf give undefined results (not checked).
 *   - Activations are token-major: element (row r, head h, dim d) of a tensor
 *     with row stride `ld` (elements) is at base[r*ld + h*head_dim + d].
 *     `ld` >= n_heads*head_dim and a multiple of 8; base pointers 16-byte
 *     aligned. This lets Q, K and V be views into one fused QKV buffer.
 *   - Supported: head_dim in {64, 128}; n_heads >= 1.
 */
#ifndef NOMAS_H
#define NOMAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NOMAS_OK = 0,
  NOMAS_E_INVALID = 1,      /* bad argument (null, size, alignment, layout)   */
  NOMAS_E_UNSUPPORTED = 2,  /* valid but not implemented (e.g. head_dim 96)   */
  NOMAS_E_WORKSPACE = 3,    /* workspace missing or smaller than required     */
  NOMAS_E_HIP = 4           /* a HIP runtime call or kernel launch failed     */
} nomas_status;

typedef enum { NOMAS_KV_BF16 = 0, NOMAS_KV_INT8 = 1 } nomas_kv_dtype;

/*
 * Ring-buffer KV cache of one layer: a window of `capacity_frames` latent
 * frames of `tokens_per_frame` video tokens each. Caller-owned plain data;
 * fill it with nomas_kvcache_init. The library changes only frames_written,
 * in the calls that append frames (nomas_kvcache_append, ..._append_archive,
 * ..._restore_frames, nomas_qkv_projection_append). A caller may set
 * frames_written itself, e.g. to resume a session from archived records: with
 * frames_written = F - n, restoring the records of frames F - n .. F - 1 puts
 * each back in its original slot.
 *
 * Frame f of the session (f = 0, 1, ... in append order) is stored in slot
 * f mod capacity_frames while it is retained; the retained frames are the last
 * min(frames_written, capacity_frames) appended, so they always fill slots
 * [0, valid_frames) and token rows [0, valid_frames*tokens_per_frame).
 *
 * Device layouts (token_pitch = nomas_kvcache_token_pitch(...), a multiple of
 * 128 >= capacity_frames*tokens_per_frame; slot token s = slot*tpf + i):
 *   k        [n_heads][token_pitch][head_dim]   bf16 or int8, row-major
 *   v        [n_heads][head_dim][token_pitch]   bf16 or int8, TRANSPOSED: the
 *            tokens of one (head, dim) are contiguous, which is the operand
 *            order the attention kernel's value contraction reads
 *   k_scale, v_scale  [n_heads][token_pitch]   float32, INT8 only (else NULL)
 * INT8 entries are x ~= code * scale with one scale per (token, head) vector.
 */
typedef struct nomas_kvcache {
  int32_t n_heads;
  int32_t head_dim;
  int32_t tokens_per_frame;
  int32_t capacity_frames;
  int32_t kv_dtype;          /* nomas_kv_dtype */
  int32_t token_pitch;
  void* k;                   /* (device) */
  void* v;                   /* (device) */
  float* k_scale;            /* (device) INT8 only */
  float* v_scale;            /* (device) INT8 only */
  int64_t frames_written;    /* frames appended since init */
} nomas_kvcache;

/* Library version, (major << 16) | minor. */
int32_t nomas_version(void);

/* Checking build only (libnomas_debug.so, compiled with NOMAS_DEVICE_CHECKS):
 * the kernels test every cache slot, token range and tile row they address
 * against the buffer it must stay in, count each failed test on the device and
 * skip that access. Returns the count since the last reset on the current
 * device (reset != 0 clears it; the call synchronises with the device), or -1
 * in the normal build, whose kernels carry no checks. For debugging and test
 * harnesses. */
int64_t nomas_device_check_failures(int32_t reset);

/* Text of the last error on the calling thread ("" if none). Valid until the
 * next call into the library on that thread. */
const char* nomas_last_error(void);

/* Tokens reserved per head in the cache buffers: round_up(capacity*tpf, 128).
 * Returns -1 on invalid sizes. */
int64_t nomas_kvcache_token_pitch(int32_t tokens_per_frame, int32_t capacity_frames);

/* Bytes of one cache buffer: which = 0 -> k, 1 -> v, 2 -> one scale array
 * (0 for NOMAS_KV_BF16). Returns 0 on invalid arguments. */
size_t nomas_kvcache_bytes(int32_t n_heads, int32_t head_dim, int32_t tokens_per_frame,
                           int32_t capacity_frames, int32_t kv_dtype, int32_t which);

/* Fill `*c` (host) for caller-allocated device buffers of the sizes above, with
 * frames_written = 0. Scales must be NULL for BF16 and non-NULL for INT8.
 * Buffer contents need no initialisation. One head's K (or V) slice,
 * token_pitch * head_dim * element bytes, must stay below 2 GiB (the kernels
 * address it with 32-bit byte offsets): NOMAS_E_INVALID otherwise, also from
 * every later call handed a descriptor edited past that limit. */
int32_t nomas_kvcache_init(nomas_kvcache* c, int32_t n_heads, int32_t head_dim,
                           int32_t tokens_per_frame, int32_t capacity_frames, int32_t kv_dtype,
                           void* k, void* v, float* k_scale, float* v_scale);

/* Number of retained frames, min(frames_written, capacity_frames); -1 if c is NULL. */
int64_t nomas_kvcache_valid_frames(const nomas_kvcache* c);

/*
 * 3D rotary position embedding, in place, of the n_frames*grid_h*grid_w video
 * rows of q (and of k when k != NULL). Text rows are not passed and not rotated.
 * Row i (ordered frame, row, col) sits at t = t0 + i/(grid_h*grid_w),
 * h = (i/grid_w) % grid_h, w = i % grid_w. Head-dim bands [0,d_t), [d_t,d_t+d_h),
 * [d_t+d_h,head_dim) are rotated by t, h, w: channels (o+2j, o+2j+1) of a band
 * of width d turn by pos*theta^(-2j/d) (negated when inverse != 0).
 * Pages: "3D RoPE" in the model card's architecture list ("Hy-Nomas auf einer
 * RTX 4090", section "Modell und Dateien"); band split, pair order and theta are
 * this library's reading (arguments).
 * Arithmetic: per-pair frequency theta^(-2j/d) evaluated in double precision on
 * the host and rounded to float32; angle, sine/cosine and rotation in float32;
 * result rounded to bf16 (nearest even).
 * q, k: (device) [rows][ld] bf16. d_t + d_h + d_w == head_dim, each even.
 * t0 >= 0, n_frames >= 1, grid_h, grid_w >= 1, theta > 0.
 */
int32_t nomas_rope3d(uint16_t* q, uint16_t* k, int64_t ld, int32_t n_heads, int32_t head_dim,
                     int32_t t0, int32_t n_frames, int32_t grid_h, int32_t grid_w,
                     int32_t d_t, int32_t d_h, int32_t d_w, float theta, int32_t inverse,
                     void* stream);

/*
 * Append n_frames latent frames (n_frames*tokens_per_frame video rows of K and
 * V, token-major with row stride ld) to the ring cache `*c` (host descriptor),
 * evicting the oldest frames beyond the capacity; when n_frames > capacity only
 * the last capacity frames are written. Increments c->frames_written by
 * n_frames at enqueue time (stream order).
 * Pages: cache of earlier latents' K/V, "Die Schleife" (orcarouter.ai); window of
 * 18 latent frames and INT8 KV, "Das Single-GPU-Preset" (inferencekey.com).
 * BF16 cache: plain copy. INT8 cache, per (token, head) vector x of head_dim
 * values: m = max|x|; s = m/127 (float32, correctly rounded); code =
 * round-half-even(x/s) (float32 quotient, correctly rounded) clamped to
 * [-127, 127]; s = 0 and codes 0 when m = 0. Bit-exact by construction.
 * k_new, v_new: (device) bf16 [n_frames*tpf][ld]; ld >= n_heads*head_dim.
 */
int32_t nomas_kvcache_append(nomas_kvcache* c, const uint16_t* k_new, const uint16_t* v_new,
                             int64_t ld, int32_t n_frames, void* stream);

/*
 * Archive of frames leaving the window (the lifelong history the pages keep in
 * CPU memory: "Persistent Lifelong KV Cache", madebyagents.com "Hy-Nomas";
 * orcarouter.ai "Die Schleife"). Copies run on the DMA engines
 * (hipMemcpy2DAsync on `stream`), asynchronous to the host: the host buffer must
 * stay valid until the stream reaches them, and should be pinned
 * (hipHostMalloc) for the copies to overlap with compute.
 * A frame's record (nomas_kvcache_record_bytes) is its slot contents in cache
 * order: K [n_heads][tpf][head_dim], then V^T [n_heads][head_dim][tpf] (int8
 * codes or bf16 bits), then for INT8 the key scales [n_heads][tpf] and the
 * value scales [n_heads][tpf] (float32).
 */
size_t nomas_kvcache_record_bytes(const nomas_kvcache* c);   /* 0 if c is invalid */

/* Records of the retained frames [first_frame, first_frame + n_frames) (absolute
 * frame numbers, as counted by frames_written) -> host_dst (host, n_frames
 * records back to back). Frames that are not retained: NOMAS_E_INVALID. */
int32_t nomas_kvcache_export_frames(const nomas_kvcache* c, int64_t first_frame, int32_t n_frames,
                                    void* host_dst, void* stream);

/* nomas_kvcache_append of 1 <= n_frames <= capacity frames that first exports
 * the retained frames the append overwrites (the oldest ones) to host_evicted
 * (host, room for n_frames records); *n_evicted (host) receives their count,
 * they being frames [frames_written - valid, ... + *n_evicted) before the call. */
int32_t nomas_kvcache_append_archive(nomas_kvcache* c, const uint16_t* k_new, const uint16_t* v_new,
                                     int64_t ld, int32_t n_frames, void* host_evicted, int32_t* n_evicted,
                                     void* stream);

/* Appends 1 <= n_frames <= capacity archived records (host_src, back to back)
 * to the cache unchanged, like nomas_kvcache_append (frames_written advances;
 * the oldest frames are overwritten): e.g. to bring history back for attention. */
int32_t nomas_kvcache_restore_frames(nomas_kvcache* c, const void* host_src, int32_t n_frames, void* stream);

/* Workspace bytes nomas_segment_attention needs for these sizes, the cache's
 * kv_dtype (nomas_kv_dtype: it sets the key tile) and n_splits (0 = the
 * automatic choice, which depends only on these arguments, n_cached being the
 * cached token count at call time). 0 on invalid arguments. */
size_t nomas_segment_attention_workspace_bytes(int32_t n_video, int32_t n_text, int64_t n_cached,
                                               int32_t n_heads, int32_t head_dim, int32_t kv_dtype,
                                               int32_t n_splits);

/* The split count the call will use for these sizes (n_splits = 0 chooses; a
 * request above the number of key tiles is clamped to it). -1 on invalid
 * arguments. The automatic choice is 1 when the call's query-tile blocks (per
 * head, 256 queries each at head dim 128) fill the chip's resident block slots
 * (one per compute unit at head dim 128, two at 64; 256 compute units);
 * otherwise, with s splits the call runs ceil(blocks * s / slots) rounds of
 * blocks that each take 1/s of the keys, and it takes the smallest s within
 * 10 % of the shortest such makespan, keeping at least 16 key tiles per split. */
int32_t nomas_segment_attention_splits(int32_t n_video, int32_t n_text, int64_t n_cached,
                                       int32_t n_heads, int32_t head_dim, int32_t kv_dtype,
                                       int32_t n_splits);

/*
 * Block-causal segment attention of the current segment.
 * Queries: the n_q = n_video + n_text rows of q, video rows first then text.
 * Keys/values: the retained cache tokens (rows [0, valid_frames*tpf) of each
 * head of `*c`) followed by all n_q rows of k_cur/v_cur. INT8 cache entries enter
 * as code*scale: a key's codes convert to bf16 exactly and its scale multiplies
 * the float32 logit; a value's code*scale is formed in float32 and rounded once
 * to bf16.
 * Every query sees every such key: bidirectional inside the segment, and
 * earlier segments only through the cache (causal across segments).
 * out[r, h, :] = sum_j softmax_j(softmax_scale * <q[r,h,:], key_j>) value_j
 * lse[h*n_q + r] = log sum_j exp(softmax_scale * <q[r,h,:], key_j>) (if lse != NULL)
 * Pages: "segment-wise causal joint attention", madebyagents.com "Hy-Nomas";
 * the cache as attention context, orcarouter.ai "Die Schleife".
 * Arithmetic: bf16 MFMA products, float32 accumulation and softmax; with
 * n_splits > 1 the key range is cut into that many contiguous chunks whose
 * partial results are merged by their log-sum-exp in a fixed order (results are
 * bitwise reproducible run to run for a fixed n_splits).
 * q, k_cur, v_cur: (device) bf16 [n_q][ld_qkv]; out: (device) bf16
 * [n_q][ld_out]; lse: (device) float32 [n_heads][n_q] or NULL;
 * c: (host) descriptor; its n_heads and head_dim are those of q, k_cur, v_cur, out.
 * softmax_scale > 0 (1/sqrt(head_dim) is the model's). workspace: (device),
 * 256-byte aligned, >= nomas_segment_attention_workspace_bytes(...).
 * n_video + n_text >= 1, and (n_video + n_text) * ld_qkv * 2 bytes below 2 GiB
 * (32-bit byte ranges in the kernels): NOMAS_E_INVALID otherwise.
 */
int32_t nomas_segment_attention(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                int64_t ld_qkv, int32_t n_video, int32_t n_text,
                                const nomas_kvcache* c, uint16_t* out, int64_t ld_out, float* lse,
                                float softmax_scale, int32_t n_splits,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * nomas_segment_attention over a chosen range of the retained frames, with the
 * segment's values optionally given transposed.
 * Keys/values: the cached tokens of frames [first_frame, first_frame + n_frames)
 * (absolute frame numbers, as counted by frames_written; all must be retained:
 * frames_written - valid_frames <= first_frame, first_frame + n_frames <=
 * frames_written, n_frames >= 0), then all n_q rows of the current segment.
 * The range may wrap round the ring. Its use: a segment's final denoising step
 * whose projection has already written the segment into the cache
 * (nomas_qkv_projection_append) attends to the window before the segment,
 * [frames_written - n_seg - W, frames_written - n_seg) in a cache of capacity
 * W + n_seg. With every retained frame the result is bit-identical to
 * nomas_segment_attention's (the same key order).
 * v_t: NULL (values from v_cur, as nomas_segment_attention), or (device) bf16
 * V^T of the current segment [n_heads*head_dim][ld_vt] -- row h*head_dim + d
 * holds channel d of head h for rows 0 .. n_q-1, as nomas_qkv_projection_vt
 * writes it; then v_cur is not read (may be NULL), the in-call transpose is
 * skipped, and ld_vt >= n_q rounded up to a multiple of 128 (the key tiles
 * read whole blocks of columns; columns >= n_q are never used), a multiple of 8,
 * head_dim * ld_vt * 2 < 2^31.
 * Other arguments, results, arithmetic and workspace (sized for n_cached =
 * n_frames * tokens_per_frame) as nomas_segment_attention. Frames not retained
 * or a bad v_t: NOMAS_E_INVALID before anything is enqueued.
 * Pages: the window of past frames ("Das Single-GPU-Preset", inferencekey.com)
 * and attention to cached context ("Die Schleife", orcarouter.ai).
 */
int32_t nomas_segment_attention_frames(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                       int64_t ld_qkv, const uint16_t* v_t, int64_t ld_vt, int32_t n_video,
                                       int32_t n_text, const nomas_kvcache* c, int64_t first_frame,
                                       int32_t n_frames, uint16_t* out, int64_t ld_out, float* lse,
                                       float softmax_scale, int32_t n_splits, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * nomas_segment_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results, without the workspace. The call
 * allocates nothing; its workspace is a scratch array inside the library,
 * nomas_segment_attention_noalloc_max_bytes() bytes on every GPU it runs on,
 * held until the process ends.
 * Sizes whose workspace (nomas_segment_attention_workspace_bytes) exceeds that
 * limit give NOMAS_E_WORKSPACE before anything is enqueued; the limit covers
 * the full single-layer shape (16 x 128 heads, 7,936 queries) without splits.
 * `stream` must belong to the calling thread's current device (NOMAS_E_INVALID
 * otherwise). Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (other streams, other threads) race and must be ordered
 * by the caller. The first call on a device looks up the array's address there.
 */
size_t  nomas_segment_attention_noalloc_max_bytes(void);
int32_t nomas_segment_attention_noalloc(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                        int64_t ld_qkv, int32_t n_video, int32_t n_text, const nomas_kvcache* c,
                                        uint16_t* out, int64_t ld_out, float* lse, float softmax_scale,
                                        int32_t n_splits, void* stream);

/*
 * 3D RoPE angles of a segment's video rows as a table, for the fused projection
 * below (computed once per segment, reused by every layer and step):
 * table[i][p] = (cos, sin)(pos * theta^(-2j/d)) of pair p (band and law as in
 * nomas_rope3d, angle negated when inverse != 0) for video row i of the
 * segment. table: (device) float32 [n_frames*grid_h*grid_w][head_dim/2][2],
 * 16-byte aligned. Same angle arithmetic as nomas_rope3d (float32 pos*w, sincosf).
 */
int32_t nomas_rope3d_table(float* table, int32_t head_dim, int32_t t0, int32_t n_frames, int32_t grid_h,
                           int32_t grid_w, int32_t d_t, int32_t d_h, int32_t d_w, float theta, int32_t inverse,
                           void* stream);

/*
 * QKV projection of a DiT block with the 3D RoPE of the video rows fused in:
 * qkv[r, c] = bf16( (x[r, :] . w[c, :]) rotated ) for the 3*n_heads*head_dim
 * channels c = [query | key | value] (head h's head_dim channels together in
 * each part). The query and key channels of rows r < n_video are rotated in
 * pairs (2j, 2j+1) of each head by rope_table[r][j] (nomas_rope3d_table);
 * text rows (r >= n_video), value channels, and every row when rope_table is
 * NULL are not (rope_table 16-byte aligned). No bias. Pages: hidden size 2,048, 16 heads of 128, 3D RoPE
 * ("Hy-Nomas auf einer RTX 4090", inferencekey.com, "Modell und Dateien").
 * Arithmetic: bf16 MFMA products, float32 accumulation and rotation, one
 * rounding to bf16.
 * x: (device) bf16 [n_rows][ld_x]; w: (device) bf16 [3*n_heads*head_dim][ld_w];
 * hidden a positive multiple of 64, ld_x and ld_w >= hidden and multiples of 8;
 * qkv: (device) bf16 [n_rows][ld_qkv], ld_qkv >= 3*n_heads*head_dim and a
 * multiple of 4 (q, k, v for nomas_segment_attention are views at column
 * offsets 0, H*D, 2*H*D with ld_qkv as their row stride). No workspace.
 */
int32_t nomas_qkv_projection(const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden, const uint16_t* w,
                             int64_t ld_w, int32_t n_heads, int32_t head_dim, int32_t n_video,
                             const float* rope_table, uint16_t* qkv, int64_t ld_qkv, void* stream);

/*
 * nomas_qkv_projection that also writes the value channels transposed:
 * v_t[h*head_dim + d][r] = qkv[r, 2*n_heads*head_dim + h*head_dim + d] for every
 * row r < n_rows (the same bf16 values), the layout of attention's value
 * operand: nomas_segment_attention_frames takes it as v_t and skips its
 * transpose pass over the segment's values.
 * v_t: (device) bf16 [n_heads*head_dim][ld_vt], 16-byte aligned, ld_vt >= n_rows
 * and a multiple of 8; columns >= n_rows are not written. Other arguments,
 * results and errors as nomas_qkv_projection.
 */
int32_t nomas_qkv_projection_vt(const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden, const uint16_t* w,
                                int64_t ld_w, int32_t n_heads, int32_t head_dim, int32_t n_video,
                                const float* rope_table, uint16_t* qkv, int64_t ld_qkv, uint16_t* v_t,
                                int64_t ld_vt, void* stream);

/*
 * nomas_qkv_projection for a segment's final denoising step, fused with
 * nomas_kvcache_append: besides writing qkv exactly as nomas_qkv_projection
 * does, it appends the segment's n_video / tokens_per_frame frames to the ring
 * cache `*c` (host descriptor) from the projection's own outputs -- the key
 * channels of rows [0, n_video) as stored in qkv (rotated when rope_table is
 * given) and the value channels -- with the append's arithmetic: INT8 scale
 * m/127 and codes RNE(x/s) of the stored bf16 values, or bf16 copies; the same
 * slots, eviction and frames_written update. The cache's separate append pass
 * (a second read of the segment's keys and values) is not needed.
 * Pages: the projection as above; the cache and its INT8 window as in
 * nomas_kvcache_append ("Hy-Nomas auf einer RTX 4090", inferencekey.com,
 * "Modell und Dateien" and "Das Single-GPU-Preset").
 * c: n_heads and head_dim those of the projection; n_video a positive multiple
 * of its tokens_per_frame. v_t, ld_vt: NULL, or the V^T output of
 * nomas_qkv_projection_vt. Other arguments and errors as nomas_qkv_projection;
 * on an error nothing is enqueued and *c is unchanged. The final step's
 * attention then reads the frames before the segment
 * (nomas_segment_attention_frames), so the cache needs room for the window
 * plus the segment.
 */
int32_t nomas_qkv_projection_append(const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden,
                                    const uint16_t* w, int64_t ld_w, int32_t n_heads, int32_t head_dim,
                                    int32_t n_video, const float* rope_table, uint16_t* qkv, int64_t ld_qkv,
                                    uint16_t* v_t, int64_t ld_vt, nomas_kvcache* c, void* stream);

/*
 * Block-sparse segment attention. After two dense denoising steps the pages keep
 * 25 % of the candidate video blocks ("Hy-Nomas auf einer RTX 4090",
 * inferencekey.com, "Das Single-GPU-Preset", citing the tech report's 6.2); they
 * give no block size or selection rule. Reading: candidates are the cached video
 * keys in blocks of NOMAS_SPARSE_KEY_BLOCK consecutive cache rows (the last one
 * may be shorter); each block of NOMAS_SPARSE_QUERY_BLOCK consecutive query rows
 * of a head keeps its own list of candidates; the current segment's rows are
 * always attended.
 * block_list layout: int32 [n_heads][ceil(n_q / NOMAS_SPARSE_QUERY_BLOCK)][n_select],
 * each list ascending, entries unique in [0, candidates).
 */
#define NOMAS_SPARSE_KEY_BLOCK 128
#define NOMAS_SPARSE_QUERY_BLOCK 256

/* Candidate blocks of n_cached cache rows: ceil(n_cached / 128); -1 if n_cached < 0. */
int32_t nomas_sparse_candidates(int64_t n_cached);

/* Workspace bytes of nomas_sparse_select (0 on invalid arguments). */
size_t nomas_sparse_select_workspace_bytes(int32_t n_q, int64_t n_cached, int32_t n_heads, int32_t head_dim);

/*
 * Selection rule (a reading): per head and query block, candidate block c
 * scores mean_q . mean_k(c) in float32 (means of the block's query rows and of
 * the candidate's cached keys as attention sees them: bf16 values, or
 * code*scale for INT8); the n_select highest scores are kept, equal scores
 * going to the lower index, and written to block_list in ascending order.
 * q: (device) bf16 [n_q][ld_q] (the queries the attention will use); c: (host)
 * descriptor of the cache; n_select in [0, candidates], at most 8192
 * candidates; block_list: (device) as above (untouched when n_select = 0).
 * workspace: (device) 256-byte aligned, >= nomas_sparse_select_workspace_bytes.
 */
int32_t nomas_sparse_select(const uint16_t* q, int64_t ld_q, int32_t n_q, const nomas_kvcache* c,
                            int32_t n_select, int32_t* block_list, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * nomas_segment_attention restricted, for each head and query block, to the
 * n_select candidate blocks of block_list (plus the whole current segment).
 * Arguments and results as nomas_segment_attention; block_list as above, read
 * on the device (a list that breaks the stated form gives undefined results;
 * every access still stays inside the cache buffers). Workspace: as for
 * nomas_segment_attention_workspace_bytes with n_cached = n_select*128.
 */
int32_t nomas_segment_attention_sparse(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                       int64_t ld_qkv, int32_t n_video, int32_t n_text, const nomas_kvcache* c,
                                       const int32_t* block_list, int32_t n_select, uint16_t* out,
                                       int64_t ld_out, float* lse, float softmax_scale, int32_t n_splits,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * One segment of a multi-segment call: n_video video rows (frames t0, t0+1, ...,
 * tokens_per_frame rows each, in (frame, row, col) order) followed by n_text
 * text rows.
 */
typedef struct {
  int32_t n_video;
  int32_t n_text;
  int32_t t0;
} nomas_segment;

/* Workspace bytes nomas_block_causal_attention needs (0 on invalid arguments). */
size_t nomas_block_causal_attention_workspace_bytes(const nomas_segment* segs, int32_t n_segments,
                                                    int32_t tokens_per_frame, int32_t n_heads,
                                                    int32_t head_dim);

/*
 * Block-causal attention over several segments at once (the whole-sequence
 * form of the segment-wise causal joint attention, as in training): the joint
 * sequence is the segments' rows in order, [video_0; text_0; video_1; text_1;
 * ...], and q, k, v hold all of them.
 * A key row j is visible to a query row i iff j is in i's segment, or j is a
 * video row of an earlier segment whose frame is >= t0(seg(i)) - window_frames
 * (window_frames < 0: every earlier video row). Text rows of earlier segments
 * are never visible.
 * out[r, h, :] = sum_j softmax_j(softmax_scale * <q[r,h,:], k[j,h,:]>) v[j,h,:]
 * over the visible j; lse[h*n_rows + r] its log-sum-exp (if lse != NULL).
 * Pages: "segment-wise causal joint attention", madebyagents.com "Hy-Nomas";
 * the cached call nomas_segment_attention reproduces segment s's rows of this
 * with the cache holding the window of earlier frames.
 * segs: (host) n_segments in [1, 64] entries; each n_video a multiple of
 * tokens_per_frame, n_text >= 0, n_video + n_text >= 1, t0 >= 0.
 * q, k, v: (device) bf16 [n_rows][ld_qkv]; out: (device) bf16 [n_rows][ld_out];
 * lse: (device) float32 [n_heads][n_rows] or NULL. head_dim 64 or 128.
 * n_rows * ld_qkv * 2 bytes below 2 GiB (NOMAS_E_INVALID otherwise).
 * workspace: (device), 256-byte aligned, >= the bytes above. Arithmetic as in
 * nomas_segment_attention (bf16 MFMA products, float32 accumulation and softmax;
 * bitwise reproducible run to run).
 */
int32_t nomas_block_causal_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv,
                                     const nomas_segment* segs, int32_t n_segments,
                                     int32_t tokens_per_frame, int32_t window_frames, int32_t n_heads,
                                     int32_t head_dim, uint16_t* out, int64_t ld_out, float* lse,
                                     float softmax_scale, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* ---- Counter calibration (a measurement aid, not a step of the method) -----
 *
 * For the callers that profile the library: rocprofv3's FETCH_SIZE scales
 * differently for different access patterns, and the attention and projection
 * kernels fetch their tiles with global -> LDS copies (16 bytes per lane). This
 * call fetches exactly `bytes` bytes of src that way, each byte once, and
 * writes one 32-bit word per 1 MiB slice to sink (its values mean nothing), so
 * FETCH_SIZE of one launch over a known size gives that pattern's scale.
 * src: (device) 16-byte aligned, bytes > 0 and a multiple of 1024; sink:
 * (device) 4-byte aligned, nomas_calibrate_lds_stream_blocks(bytes) words.
 * Errors: NOMAS_E_INVALID for other sizes or alignments (nothing enqueued).
 */
int64_t nomas_calibrate_lds_stream_blocks(int64_t bytes);   /* -1 for an invalid size */
int32_t nomas_calibrate_lds_stream(const void* src, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NOMAS_H */
