"""Planted mistakes in the oracle (CPU only). Each plausible slip -- a dropped
term, a wrong sign, a swapped index, a wrong rounding, an off-by-one in a mask --
is planted in one oracle function through monkeypatch, and at least one pin of
tests/test_oracle_*.py must then fail. This shows the pins bind the oracle's
arithmetic instead of restating it."""

import math
import sys

import numpy as np
import pytest

if sys.version_info < (3, 11):
    from exceptiongroup import BaseExceptionGroup

import test_oracle_attention as PA
import test_oracle_formats as PF
import test_oracle_qkv as PK
import test_oracle_quant as PQ
import test_oracle_ring as PG
import test_oracle_rope as PR
import test_oracle_sparse as PS
from oracle import attention, formats, qkv, quant, ring, rope, sparse


def _some_pin_fails(pins):
    # only a failed assertion counts: a planted slip that merely crashes would
    # say nothing about the pins (a property-based pin that finds several
    # distinct failing examples reports them together, as a group)
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return True
        except BaseExceptionGroup as eg:
            if all(isinstance(e, AssertionError) for e in eg.exceptions):
                return True
            raise
    return False


ROPE_PINS = [PR.test_positions_match_explicit_loops, PR.test_pair_norms_preserved, PR.test_inverse_by_negated_angle,
             PR.test_zero_position_is_identity, PR.test_one_axis_is_complex_multiplication,
             PR.test_band_layout_unit_vectors, PR.test_relative_shift_invariance]
QUANT_PINS = [PQ.test_roundtrip_within_half_step, PQ.test_special_cases, PQ.test_ties_round_to_even,
              PQ.test_every_code_is_exact_in_bf16, PQ.test_dequantised_values_are_exact_products] + \
             [lambda m=m: PQ.test_exhaustive_against_exact_rational(m)
              for m in (0x3F80, 0x4080, 0x40A0, 0x42A0, 0x3A83, 0x0081, 0x3F96, 0x3FB4, 0x3A8F)]
ATTN_PINS = [PA.test_probability_rows_sum_to_one, PA.test_ones_values_give_ones,
             PA.test_constant_keys_give_mean_and_frame_histogram, PA.test_single_key_and_dominant_logit,
             PA.test_key_permutation_invariance, PA.test_brute_force_tiny, PA.test_brute_force_tiny_workload_rows,
             PA.test_rows_helper_matches_full, PA.test_block_causal_row_subset, PA.test_window_changes_result] + \
            [lambda s=s: PA.test_split_merge_equals_unsplit(s) for s in (2, 3, 7)] + \
            [lambda i=i, w=w: PA.test_cached_equals_full_block_causal(i, w) for i in (False, True) for w in (None, 4, 3)]
RING_PINS = [PG.test_window_is_last_capacity_frames, PG.test_append_larger_than_capacity_keeps_tail,
             PG.test_evicted_then_retained_is_every_frame_in_order]
SPARSE_PINS = [PS.test_all_blocks_selected_is_dense, PS.test_no_blocks_selected_is_segment_only,
               PS.test_selected_rows_only_matter, PS.test_planted_blocks_are_chosen,
               PS.test_ties_go_to_lower_index_and_lists_ascend, PS.test_selection_invariances,
               PS.test_short_last_block_mean_is_over_its_own_rows, PS.test_each_head_uses_its_own_list]
QKV_PINS = [PK.test_brute_force_projection, PK.test_identity_weights_give_rope_of_the_input, PK.test_one_rounding_after_the_rotation,
            PK.test_rotation_preserves_pair_norms_and_values_are_unrotated]
FORMAT_PINS = [PF.test_to_bf16_matches_torch_on_float32_patterns, PF.test_to_bf16_single_rounding_from_float64_brute_force]


# ---- RoPE slips
def _rope_variant(pair, swap_sin=False):
    def rope3d(x, t, h, w, d_t, d_h, d_w, theta=10000.0, sign=1.0):
        x = np.asarray(x, dtype=np.float64)
        out = x.copy()
        offset = 0
        for pos, width in ((t, d_t), (h, d_h), (w, d_w)):
            if width:
                phi = sign * rope.angles(pos, width, theta)
                c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
                if pair == "adjacent":
                    iu = np.arange(offset, offset + width, 2)
                    iv = iu + 1
                else:                                   # halves of the band
                    iu = np.arange(offset, offset + width // 2)
                    iv = iu + width // 2
                u, v = x[:, :, iu], x[:, :, iv]
                if swap_sin:
                    out[:, :, iu], out[:, :, iv] = u * c + v * s, -u * s + v * c
                else:
                    out[:, :, iu], out[:, :, iv] = u * c - v * s, u * s + v * c
            offset += width
        return out
    return rope3d


_ORIG_ROPE3D = rope.rope3d


def _rope_ignores_sign(x, t, h, w, d_t, d_h, d_w, theta=10000.0, sign=1.0):
    return _ORIG_ROPE3D(x, t, h, w, d_t, d_h, d_w, theta)


def _angles_half_exponent(pos, width, theta=10000.0):
    j = np.arange(width // 2, dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * (theta ** (-1.0 * j / width))[None, :]


def _angles_base_1000(pos, width, theta=10000.0):
    j = np.arange(width // 2, dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * (1000.0 ** (-2.0 * j / width))[None, :]


def _positions_hw_swapped(t0, n_frames, grid_h, grid_w):
    i = np.arange(n_frames * grid_h * grid_w, dtype=np.int64)
    return t0 + i // (grid_h * grid_w), i % grid_h, (i // grid_h) % grid_w


# ---- quantisation slips
def _quantise_variant(div=127.0, rounding="even", f32_quotient=True, f32_scale=True):
    def q(x):
        x = np.asarray(x, dtype=np.float64)
        m = np.max(np.abs(x), axis=-1)
        s = (m / div).astype(np.float32)
        s64 = s.astype(np.float64) if f32_scale else m / div
        safe = np.where(s64 > 0, s64, 1.0)[..., None]
        r = x / safe
        if f32_quotient:
            r = r.astype(np.float32).astype(np.float64)
        r = np.rint(r) if rounding == "even" else np.sign(r) * np.floor(np.abs(r) + 0.5)
        r = np.where((s64 > 0)[..., None], np.clip(r, -127, 127), 0.0)
        return r.astype(np.int8), s
    return q


def _quantise_scale_per_token(x):
    """One scale per token across all heads (instead of per token and head)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim < 2:
        return quant_orig(x)
    m = np.max(np.abs(x), axis=(-2, -1), keepdims=True)
    s = (m / 127.0).astype(np.float32)
    s64 = s.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    r = (x / safe).astype(np.float32).astype(np.float64)
    q = np.where(s64 > 0, np.clip(np.rint(r), -127, 127), 0.0)
    return q.astype(np.int8), np.broadcast_to(s[..., 0], x.shape[:-1]).astype(np.float32)


def _dequantise_to_bf16(q, s):
    return formats.to_bf16(np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None])


def _to_bf16_ties_away(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x8000) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


quant_orig = quant.quantise


# ---- attention slips
def _attention_variant(slip):
    orig = attention.segment_attention

    def seg(q, k_cur, v_cur, k_past=None, v_past=None, scale=None, return_probs=False):
        if slip == "no_scale":
            scale = 1.0
        if slip == "drop_past":
            k_past = v_past = None
        if slip == "keys_as_values":
            v_cur, v_past = k_cur, k_past
        res = orig(q, k_cur, v_cur, k_past, v_past, scale, return_probs)
        if slip == "lse_log2":
            return (res[0], res[1] / math.log(2.0)) + tuple(res[2:])
        return res
    return seg


_ORIG_ROWS = attention.segment_attention_rows


def _rows_heads_misread(q_rows, row_heads, k, v, scale):
    """Every sampled row attended with head 0's keys and values."""
    return _ORIG_ROWS(q_rows, np.zeros_like(np.asarray(row_heads)), k, v, scale)


_ORIG_BCF = attention.block_causal_full


def _block_causal_raw_past(segments, *args, **kwargs):
    """Earlier segments' video keys/values as written, not as the cache holds them."""
    segs = [{k: v for k, v in sg.items() if k not in ("k_past", "v_past")} for sg in segments]
    return _ORIG_BCF(segs, *args, **kwargs)


def _softmax_no_normalisation(s):
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p, m[..., 0]


def _split_unnormalised_weights(q, k, v, n_splits, scale):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    bounds = np.linspace(0, k.shape[0], n_splits + 1).round().astype(int)
    parts = [attention.segment_attention(q, k[a:b], v[a:b], scale=scale)
             for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    out = sum(o * np.exp(l).T[:, :, None] for o, l in parts)      # weight not divided by the total
    lse = np.log(sum(np.exp(l) for _, l in parts))
    return out, lse


def _block_causal_window_off_by_one():
    orig = attention.block_causal_full

    def full(segments, window_frames=None, scale=None, rows=None, return_lse=False):
        w = None if window_frames is None else window_frames - 1      # frame > t0 - W instead of >=
        return orig(segments, w, scale, rows, return_lse)
    return full


# ---- sparse-selection slips
def _select_variant(slip):
    def select(q, k_past, n_select):
        sc = sparse.block_scores(q, k_past)
        H, nqb, nc = sc.shape
        out = np.empty((H, nqb, n_select), np.int32)
        for h in range(H):
            for b in range(nqb):
                if slip == "lowest":
                    order = sorted(range(nc), key=lambda c: (sc[h, b, c], c))
                else:                                   # ties to the higher index
                    order = sorted(range(nc), key=lambda c: (-sc[h, b, c], -c))
                out[h, b] = sorted(order[:n_select])
        return out
    return select


def _block_means_sum(x, block):
    x = np.asarray(x, np.float64)
    nb = (x.shape[0] + block - 1) // block
    return np.stack([x[b * block:(b + 1) * block].sum(axis=0) for b in range(nb)])   # sum, not mean


def _sparse_attention_drops_last_partial(q, k_cur, v_cur, k_past, v_past, lists, scale):
    n_full = (k_past.shape[0] // sparse.KEY_BLOCK) * sparse.KEY_BLOCK
    return _orig_sparse_attention(q, k_cur, v_cur, k_past[:n_full], v_past[:n_full],
                                  np.where(lists * sparse.KEY_BLOCK < n_full, lists, 0), scale)


_orig_sparse_attention = sparse.sparse_segment_attention


# ---- QKV-projection slips
def _qkv_variant(slip):
    orig = qkv.qkv_projection

    def proj(x, w, n_heads, head_dim, n_video=0, rope=None):
        if slip == "rope_on_values":
            q, k, v = orig(x, w, n_heads, head_dim, n_video, rope)
            if rope is not None and n_video > 0:
                r = dict(rope)
                args = (r["t0"], r["n_frames"], r["grid_h"], r["grid_w"], r["d_t"], r["d_h"], r["d_w"])
                v = v.copy()
                v[:n_video] = formats.to_bf16(qkv.rope3d_segment(v[:n_video], *args))
            return q, k, v
        if slip == "round_before_rope":
            # the product rounded to bf16 before the rotation as well (two roundings)
            x64, w64 = np.asarray(x, np.float64), np.asarray(w, np.float64)
            H, D = n_heads, head_dim
            y = formats.to_bf16(x64 @ w64.T)
            q, k, v = (y[:, i * H * D:(i + 1) * H * D].reshape(-1, H, D).copy() for i in range(3))
            if rope is not None and n_video > 0:
                r = dict(rope)
                args = (r["t0"], r["n_frames"], r["grid_h"], r["grid_w"], r["d_t"], r["d_h"], r["d_w"])
                q[:n_video] = qkv.rope3d_segment(q[:n_video], *args)
                k[:n_video] = qkv.rope3d_segment(k[:n_video], *args)
            return formats.to_bf16(q), formats.to_bf16(k), formats.to_bf16(v)
        # q and k channel blocks exchanged
        q, k, v = orig(x, w, n_heads, head_dim, n_video, rope)
        return k, q, v
    return proj


# ---- ring slip
class _RingKeepsOldest(ring.RingModel):
    def append(self, payloads):
        for p in payloads:
            self.frames.append((self.frames_written, p))
            self.frames_written += 1
            while len(self.frames) > self.capacity:
                self.evicted.append(self.frames.pop())               # evicts the newest


class _RingOneShort(ring.RingModel):
    def append(self, payloads):
        for p in payloads:
            self.frames.append((self.frames_written, p))
            self.frames_written += 1
            while len(self.frames) >= self.capacity:              # keeps capacity-1 frames
                self.evicted.append(self.frames.pop(0))


class _RingSlotsFromOne(ring.RingModel):
    def expected_slots(self):
        return {(f + 1) % self.capacity: (f, p) for f, p in self.frames}


def _block_means_full_divisor(x, block):
    """Short last block averaged over a full block's row count."""
    x = np.asarray(x, np.float64)
    nb = (x.shape[0] + block - 1) // block
    return np.stack([x[b * block:(b + 1) * block].sum(axis=0) / block for b in range(nb)])


def _positions_without_t0(t0, n_frames, grid_h, grid_w):
    return _ORIG_POSITIONS(0, n_frames, grid_h, grid_w)


_ORIG_POSITIONS = rope.video_positions


_ORIG_SPARSE_ATTN = sparse.sparse_segment_attention


def _sparse_lists_of_head0(q, k_cur, v_cur, k_past, v_past, lists, scale):
    """Every head attends to head 0's block list."""
    lists = np.asarray(lists)
    return _ORIG_SPARSE_ATTN(q, k_cur, v_cur, k_past, v_past, np.broadcast_to(lists[:1], lists.shape), scale)


# ---- format slip
def _to_bf16_truncate(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


MUTANTS = {
    "rope: rotation sense reversed": (rope, "rope3d", _rope_variant("adjacent", swap_sin=True), ROPE_PINS),
    "rope: pairs as band halves": (rope, "rope3d", _rope_variant("halves"), ROPE_PINS),
    "rope: frequency exponent j/d": (rope, "angles", _angles_half_exponent, ROPE_PINS),
    "rope: inverse rotation not inverted": (rope, "rope3d", _rope_ignores_sign, ROPE_PINS),
    "rope: frequency base 1000 whatever theta": (rope, "angles", _angles_base_1000, ROPE_PINS),
    "rope: h and w positions swapped": (rope, "video_positions", _positions_hw_swapped, ROPE_PINS),
    "rope: frame positions from 0 instead of t0": (rope, "video_positions", _positions_without_t0, ROPE_PINS),
    "quant: scale absmax/128": (quant, "quantise", _quantise_variant(div=128.0), QUANT_PINS),
    "quant: ties away from zero": (quant, "quantise", _quantise_variant(rounding="away"), QUANT_PINS),
    "quant: quotient not rounded to fp32": (quant, "quantise", _quantise_variant(f32_quotient=False), QUANT_PINS),
    "quant: codes against the unrounded scale": (quant, "quantise", _quantise_variant(f32_scale=False), QUANT_PINS),
    "quant: one scale per token across heads": (quant, "quantise", _quantise_scale_per_token, QUANT_PINS),
    "quant: dequantised values rounded to bf16": (quant, "dequantise", _dequantise_to_bf16, QUANT_PINS),
    "attention: scale dropped": (attention, "segment_attention", _attention_variant("no_scale"), ATTN_PINS),
    "attention: cached keys dropped": (attention, "segment_attention", _attention_variant("drop_past"), ATTN_PINS),
    "attention: keys used as values": (attention, "segment_attention", _attention_variant("keys_as_values"), ATTN_PINS),
    "attention: log-sum-exp in log2 units": (attention, "segment_attention", _attention_variant("lse_log2"), ATTN_PINS),
    "attention: sampled rows read with head 0": (attention, "segment_attention_rows", _rows_heads_misread, ATTN_PINS),
    "attention: earlier segments' keys raw, not as cached": (attention, "block_causal_full", _block_causal_raw_past,
                                                             ATTN_PINS),
    "attention: softmax not normalised": (attention, "_softmax_rows", _softmax_no_normalisation, ATTN_PINS),
    "attention: split weights not normalised": (attention, "split_attention", _split_unnormalised_weights, ATTN_PINS),
    "attention: window mask off by one": (attention, "block_causal_full", _block_causal_window_off_by_one(), ATTN_PINS),
    "sparse: lowest scores selected": (sparse, "select_blocks", _select_variant("lowest"), SPARSE_PINS),
    "sparse: ties to the higher index": (sparse, "select_blocks", _select_variant("ties_high"), SPARSE_PINS),
    "sparse: block sums instead of means": (sparse, "block_means", _block_means_sum, SPARSE_PINS),
    "sparse: short last block over a full count": (sparse, "block_means", _block_means_full_divisor, SPARSE_PINS),
    "sparse: every head takes head 0's list": (sparse, "sparse_segment_attention", _sparse_lists_of_head0,
                                               SPARSE_PINS),
    "sparse: short last block dropped": (sparse, "sparse_segment_attention", _sparse_attention_drops_last_partial,
                                          SPARSE_PINS),
    "qkv: RoPE applied to values": (qkv, "qkv_projection", _qkv_variant("rope_on_values"), QKV_PINS),
    "qkv: q and k blocks exchanged": (qkv, "qkv_projection", _qkv_variant("qk_swapped"), QKV_PINS),
    "qkv: rounded to bf16 before the rotation too": (qkv, "qkv_projection", _qkv_variant("round_before_rope"),
                                                     QKV_PINS),
    "ring: evicts the newest frame": (ring, "RingModel", _RingKeepsOldest, RING_PINS),
    "ring: window one frame short": (ring, "RingModel", _RingOneShort, RING_PINS),
    "ring: slots counted from one": (ring, "RingModel", _RingSlotsFromOne, RING_PINS),
    "formats: bf16 by truncation": (formats, "to_bf16", _to_bf16_truncate, FORMAT_PINS),
    "formats: bf16 ties away from zero": (formats, "to_bf16", _to_bf16_ties_away, FORMAT_PINS),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    module, attr, fn, pins = MUTANTS[name]
    monkeypatch.setattr(module, attr, fn)
    if module is ring:      # the pins hold their own reference to the class
        monkeypatch.setattr(PG, "RingModel", fn, raising=False)
        monkeypatch.setattr(PA, "RingModel", fn, raising=False)
    assert _some_pin_fails(pins), f"no pin caught the planted mistake: {name}"


def test_unmodified_oracle_passes_the_pins():
    assert not _some_pin_fails(ROPE_PINS + QUANT_PINS + ATTN_PINS + RING_PINS + FORMAT_PINS + SPARSE_PINS + QKV_PINS)
