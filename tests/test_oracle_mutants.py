"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

Every mutant below is a plausible slip — a dropped factor, a flipped sign,
a swapped index or band, a strict instead of non-strict comparison, a
transposed normalisation — patched into ``oracle`` for the duration of one
check.  The pins in test_oracle_rope / test_oracle_attention must reject it.
"""
import numpy as np
import pytest

import test_oracle_attention as TA
import test_oracle_block_sparse as TS
import test_oracle_qkv as TQ
import test_oracle_ring as TG
import test_oracle_rope as TR
from oracle import attention as A
from oracle import block_sparse as S
from oracle import qkv as Q
from oracle import ring as G
from oracle import rope3d as R

_orig_token_freqs = R.token_freqs
_orig_positions = R.positions


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _mut_angles_dropped_two(d_b, theta):
    j = np.arange(d_b // 2, dtype=np.float64)
    return np.power(np.float64(theta), -1.0 * j / d_b)


def _mut_freqs_conj(tables, pos):
    return np.conj(_orig_token_freqs(tables, pos))


def _mut_freqs_band_order(tables, pos):
    ft, fh, fw = tables
    return np.concatenate([fh[pos[:, 1]], ft[pos[:, 0]], fw[pos[:, 2]]], axis=1)


def _mut_positions_hw_swapped(F, H, W, s, off, n):
    p = _orig_positions(F, H, W, s, off, n).copy()
    i = np.arange(off, off + n) % (H * W)
    p[:, 1], p[:, 2] = i % H, i // H
    return p


def _mut_positions_no_start(F, H, W, s, off, n):
    p = _orig_positions(F, H, W, s, off, n).copy()
    p[:, 0] -= s
    return p


def _mut_visible_strict(q_rows, q_pos, kv_len, C):
    qc = (q_pos + np.asarray(q_rows)) // C
    kc = np.arange(kv_len) // C
    return kc[None, :] < qc[:, None]


_orig_attn = A.chunk_causal_attention


def _mut_attn_col_softmax(q, kc, vc, q_pos, kv_len, C, scale, rows=None, block=256):
    q = np.asarray(q, dtype=np.float64)
    b, lq, nh, d = q.shape
    rows = np.arange(lq) if rows is None else np.asarray(rows)
    out = np.empty((b, len(rows), nh, d))
    for bi in range(b):
        for h in range(nh):
            s = scale * (q[bi, rows, h] @ kc[bi, :kv_len, h].T)
            s = np.where(A.visible(rows, q_pos, kv_len, C), s, -np.inf)
            p = np.exp(s - s.max(axis=0, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[bi, :, h] = p @ vc[bi, :kv_len, h]
    return out


def _mut_attn_no_scale(q, kc, vc, q_pos, kv_len, C, scale, rows=None, block=256):
    return _orig_attn(q, kc, vc, q_pos, kv_len, C, 1.0, rows=rows, block=block)


_orig_project = Q.qkv_project


def _mut_qkv_k_v_swapped(x, w, bias, nh, d):
    q, k, v = _orig_project(x, w, bias, nh, d)
    return q, v, k


def _mut_qkv_d_major(x, w, bias, nh, d):
    """Rows of each group read as head_dim-major instead of head-major."""
    x = np.asarray(x, dtype=np.float64)
    y = x @ np.asarray(w, dtype=np.float64).T
    if bias is not None:
        y = y + bias
    b, n = x.shape[:2]
    hd = nh * d
    return tuple(y[..., i * hd:(i + 1) * hd].reshape(b, n, d, nh).transpose(0, 1, 3, 2)
                 for i in range(3))


def _mut_qkv_no_bias(x, w, bias, nh, d):
    return _orig_project(x, w, None, nh, d)


_orig_held = G.held_frames
_orig_ring_positions = G.positions


def _mut_slot_ring_over_sinks(t, sink, window):
    return np.mod(np.asarray(t, dtype=np.int64), sink + window)


def _mut_slot_offset_not_subtracted(t, sink, window):
    t = np.asarray(t, dtype=np.int64)
    return np.where(t < sink, t, sink + np.mod(t, window))


def _mut_held_one_short(F, s, sink, window):
    h = _orig_held(F, s, sink, window)
    end = s + F
    return h[h != max(sink, end - window)] if end - window >= sink else h


def _mut_held_no_sinks(F, s, sink, window):
    h = _orig_held(F, s, sink, window)
    return h[h >= sink]


_orig_frame_row = G.frame_row


def _mut_frame_row_block_transposed(h, w, H, W, bh=0, bw=0):
    if not bh:
        return _orig_frame_row(h, w, H, W)
    h, w = np.asarray(h), np.asarray(w)
    block = (h // bh) * (W // bw) + w // bw
    return block * (bh * bw) + (w % bw) * bh + h % bh


def _mut_ring_time_is_slot(F, H, W, s, off, n, sink, window):
    p = _orig_ring_positions(F, H, W, s, off, n, sink, window).copy()
    p[:, 0] = p[:, 3] // (H * W)
    return p


_orig_key_blocks = S.key_blocks
_orig_block_sparse = S.block_sparse_attention


def _mut_blocks_repeats_kept(persist, local, n_kb):
    ids = np.concatenate([np.asarray(persist).reshape(-1), np.asarray(local).reshape(-1)])
    return np.sort(ids[(ids >= 0) & (ids < n_kb)])


def _mut_blocks_no_persistent(persist, local, n_kb):
    return _orig_key_blocks(np.zeros(0, dtype=np.int64), local, n_kb)


def _mut_blocks_padding_kept(persist, local, n_kb):
    ids = np.concatenate([np.asarray(persist).reshape(-1), np.asarray(local).reshape(-1)])
    return np.unique(ids[ids < n_kb])


def _mut_local_of_next_block(q, kc, vc, kv, blk, persist, local, scale):
    return _orig_block_sparse(q, kc, vc, kv, blk, persist, np.roll(local, 1, axis=2), scale)


ROPE_PINS = [
    (TR.test_rotation_matches_gptj_interleaved_rope_per_band, ((8, 8, 8),)),
    (TR.test_unit_vector_closed_form, ()),
    (TR.test_brute_force_rotation_loops_tiny, ()),
    (TR.test_positions_brute_force_grid, (3, 5, 7, 9)),
    (TR.test_start_frame_worked_example, ()),
    (TR.test_shard_equals_unsharded_algorithm2, (8,)),
]

QKV_PINS = [
    (TQ.test_projection_brute_force, ()),
    (TQ.test_identity_projection, ()),
    (TQ.test_one_hot_row_lands_in_its_slot, (1, 2, 7)),
]

RING_PINS = [
    (TG.test_slot_map_and_held_set_match_a_fifo_store, (2, 5, 2)),
    (TG.test_positions_rows, ()),
    (TG.test_rolled_rollout_matches_brute_force_over_a_full_cache, (1, 4, 3)),
    (TG.test_time_shift_moves_slots_not_outputs, ()),
    (TG.test_sinks_survive_and_memory_is_bounded, ()),
    (TG.test_blockified_frame_rows, (4, 6, 2, 3)),
]

SPARSE_PINS = [
    (TS.test_brute_force_tiny, (4, 10, 24)),
    (TS.test_brute_force_tiny, (3, 8, 20)),
    (TS.test_every_block_selected_is_dense_attention, ()),
    (TS.test_identical_keys_average_v_and_empty_gives_zero, ()),
    (TS.test_padding_repeats_and_order_change_nothing, ()),
    (TS.test_persistent_only_is_attention_over_the_gathered_rows, ()),
]

ATTN_PINS = [
    (TA.test_brute_force_tiny, (64, 32, 96, 32)),
    (TA.test_matches_torch_sdpa_fp64_with_bool_mask, ()),
    (TA.test_closed_forms, ()),
]


@pytest.mark.parametrize("attr,mutant", [
    ("band_angles", _mut_angles_dropped_two),
    ("token_freqs", _mut_freqs_conj),
    ("token_freqs", _mut_freqs_band_order),
    ("positions", _mut_positions_hw_swapped),
    ("positions", _mut_positions_no_start),
])
def test_rope_mutant_is_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(R, attr, mutant)
    assert any(_fails(fn, *args) for fn, args in ROPE_PINS), f"{mutant.__name__} survived"


@pytest.mark.parametrize("attr,mutant", [
    ("visible", _mut_visible_strict),
    ("chunk_causal_attention", _mut_attn_col_softmax),
    ("chunk_causal_attention", _mut_attn_no_scale),
])
def test_attention_mutant_is_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(A, attr, mutant)
    assert any(_fails(fn, *args) for fn, args in ATTN_PINS), f"{mutant.__name__} survived"


@pytest.mark.parametrize("mutant", [_mut_qkv_k_v_swapped, _mut_qkv_d_major, _mut_qkv_no_bias])
def test_qkv_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(Q, "qkv_project", mutant)
    assert any(_fails(fn, *args) for fn, args in QKV_PINS), f"{mutant.__name__} survived"


@pytest.mark.parametrize("attr,mutant", [
    ("frame_slot", _mut_slot_ring_over_sinks),
    ("frame_slot", _mut_slot_offset_not_subtracted),
    ("held_frames", _mut_held_one_short),
    ("held_frames", _mut_held_no_sinks),
    ("positions", _mut_ring_time_is_slot),
    ("frame_row", _mut_frame_row_block_transposed),
])
def test_ring_mutant_is_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(G, attr, mutant)
    assert any(_fails(fn, *args) for fn, args in RING_PINS), f"{mutant.__name__} survived"


@pytest.mark.parametrize("attr,mutant", [
    ("key_blocks", _mut_blocks_repeats_kept),
    ("key_blocks", _mut_blocks_no_persistent),
    ("key_blocks", _mut_blocks_padding_kept),
    ("block_sparse_attention", _mut_local_of_next_block),
])
def test_block_sparse_mutant_is_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(S, attr, mutant)
    assert any(_fails(fn, *args) for fn, args in SPARSE_PINS), f"{mutant.__name__} survived"


def test_unmutated_oracle_passes_every_pin():
    for fn, args in ROPE_PINS + ATTN_PINS + QKV_PINS + RING_PINS + SPARSE_PINS:
        assert not _fails(fn, *args), fn.__name__
