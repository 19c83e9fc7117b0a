"""Pins of the rolling-window cache oracle to facts outside it.

``oracle.ring`` is tied to:

* a literal FIFO simulation of a fixed-size frame store (pure Python: sink
  frames kept, the oldest other frame evicted, the newcomer taking the
  freed slot) that must agree with the closed-form slot map and held set;
* the plain cache (``oracle.rope3d`` / ``oracle.attention``, pinned on
  their own) whenever nothing has been evicted;
* brute-force attention (Python loops, math.exp) over the rows of the
  simulated held frames, read from a cache that keeps every frame in
  global order, across a rollout that wraps the ring several times;
* the RoPE relative-position property: shifting every frame of a rollout by
  the same amount moves every slot but leaves the attention output alone;
* sink rows that survive a long rollout, and the memory bound.
CPU only.
"""
import collections
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import ring as G
from oracle import rope3d as R


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


class FifoStore:
    """A store of sink + window frame slots filled in arrival order."""

    def __init__(self, sink, window):
        self.sink, self.window = sink, window
        self.slot_of = {}
        self.recent = collections.deque()
        self.free = list(range(sink, sink + window))

    def put(self, t):
        if t in self.slot_of:          # rewritten by a later denoising step
            return self.slot_of[t]
        if t < self.sink:
            slot = t
        else:
            if len(self.recent) == self.window:
                old = self.recent.popleft()
                slot = self.slot_of.pop(old)
            else:
                slot = self.free.pop(0)
            self.recent.append(t)
        self.slot_of[t] = slot
        return slot


@pytest.mark.parametrize("sink,window,F", [(0, 7, 3), (0, 6, 3), (2, 5, 2), (1, 4, 3),
                                          (3, 3, 3), (0, 1, 1), (4, 9, 2)])
def test_slot_map_and_held_set_match_a_fifo_store(sink, window, F):
    store = FifoStore(sink, window)
    for c in range(40 // F):
        s = c * F
        for t in range(s, s + F):
            assert store.put(t) == int(G.frame_slot(t, sink, window)), (t, sink, window)
        held = G.held_frames(F, s, sink, window)
        assert sorted(store.slot_of) == list(held)
        assert len(held) == min(s + F, sink + window)
        assert len(set(G.frame_slot(held, sink, window).tolist())) == len(held)


def test_positions_rows():
    F, H, W, s, off, n, sink, window = 2, 3, 4, 8, 5, 17, 1, 4
    p = G.positions(F, H, W, s, off, n, sink, window)
    plain = R.positions(F, H, W, s, off, n)
    np.testing.assert_array_equal(p[:, :3], plain[:, :3])
    for i in range(n):
        t, h, w = plain[i, :3]
        slot = t if t < sink else sink + (t - sink) % window
        assert p[i, 3] == slot * H * W + h * W + w


def test_no_eviction_is_the_plain_cache():
    d = (8, 8, 8)
    nh, D, F, H, W = 2, 24, 2, 3, 3
    tables = R.rope3d_tables(*d, 10000.0, 32, 8, 8)
    n_chunks, hw = 4, 9
    cap = n_chunks * F * hw
    kr, vr = np.zeros((1, cap, nh, D)), np.zeros((1, cap, nh, D))
    kp, vp = np.zeros_like(kr), np.zeros_like(vr)
    for c in range(n_chunks):
        s = c * F
        q, k, v = (_rand((1, F * hw, nh, D), 10 * c + i) for i in range(3))
        np.testing.assert_array_equal(G.positions(F, H, W, s, 0, F * hw, 0, n_chunks * F),
                                      R.positions(F, H, W, s, 0, F * hw))
        qr = G.rope3d_apply_append(q, k, v, kr, vr, tables, F, H, W, s, 0, 0, n_chunks * F)
        qp = R.rope3d_apply_append(q, k, v, kp, vp, tables, F, H, W, s, 0)
        np.testing.assert_array_equal(qr, qp)
        np.testing.assert_array_equal(kr, kp)
        o_ring = G.ring_attention(qr, kr, vr, F, H, W, s, 0, n_chunks * F, 0.2)
        o_plain = A.chunk_causal_attention(qp, kp, vp, s * hw, (s + F) * hw, F * hw, 0.2)
        np.testing.assert_allclose(o_ring, o_plain, rtol=0, atol=1e-13)


def _brute_attention(q_rot, k_rows, v_rows, scale):
    """Per query and head: softmax over the given key rows, in Python loops."""
    b, n, nh, d = q_rot.shape
    out = np.zeros_like(q_rot)
    for bi in range(b):
        for i in range(n):
            for h in range(nh):
                logits = [scale * sum(q_rot[bi, i, h, e] * kr[bi, h, e] for e in range(d))
                          for kr in k_rows]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                z = sum(w)
                for e in range(d):
                    out[bi, i, h, e] = sum(w[j] * v_rows[j][bi, h, e] for j in range(len(w))) / z
    return out


@pytest.mark.parametrize("sink,window,F", [(0, 5, 2), (1, 4, 3)])
def test_rolled_rollout_matches_brute_force_over_a_full_cache(sink, window, F):
    d = (4, 4, 4)
    nh, D, H, W, hw = 2, 12, 2, 2, 4
    tables = R.rope3d_tables(*d, 10000.0, 64, 4, 4)
    n_chunks = 7                               # wraps the ring several times
    full_k = np.zeros((1, n_chunks * F * hw, nh, D))
    full_v = np.zeros_like(full_k)
    kr = np.full((1, (sink + window) * hw, nh, D), np.nan)
    vr = kr.copy()
    store = FifoStore(sink, window)
    for c in range(n_chunks):
        s = c * F
        for step in range(2):                  # denoising steps rewrite the chunk
            q, k, v = (_rand((1, F * hw, nh, D), 100 * c + 10 * step + i) for i in range(3))
            # reference: plain cache in global order, FIFO store for the held set
            qp = R.rope3d_apply_append(q, k, v, full_k, full_v, tables, F, H, W, s, 0)
            for t in range(s, s + F):
                store.put(t)
            held = sorted(store.slot_of)
            k_rows = [full_k[:, t * hw + j] for t in held for j in range(hw)]
            v_rows = [full_v[:, t * hw + j] for t in held for j in range(hw)]
            expect = _brute_attention(qp, k_rows, v_rows, 0.35)
            qr = G.rope3d_apply_append(q, k, v, kr, vr, tables, F, H, W, s, 0, sink, window)
            got = G.ring_attention(qr, kr, vr, F, H, W, s, sink, window, 0.35)
            np.testing.assert_allclose(got, expect, rtol=0, atol=1e-12)


def test_time_shift_moves_slots_not_outputs():
    """RoPE relative positions: a rollout shifted by 5 frames attends the same."""
    d = (8, 4, 4)
    nh, D, F, H, W, hw, window = 2, 16, 2, 2, 3, 6, 4
    tables = R.rope3d_tables(*d, 10000.0, 64, 4, 4)
    outs = []
    for shift in (0, 5):
        kr = np.zeros((1, window * hw, nh, D))
        vr = np.zeros_like(kr)
        for c in range(5):
            s = shift + c * F
            q, k, v = (_rand((1, F * hw, nh, D), 7 * c + i) for i in range(3))
            qr = G.rope3d_apply_append(q, k, v, kr, vr, tables, F, H, W, s, 0, 0, window)
            o = G.ring_attention(qr, kr, vr, F, H, W, s, 0, window, 0.3)
        outs.append(o)
    assert G.frame_slot(5 + 8, 0, window) != G.frame_slot(8, 0, window)
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-12)


def test_sinks_survive_and_memory_is_bounded():
    d = (4, 4, 4)
    nh, D, F, H, W, hw, sink, window = 1, 12, 3, 2, 2, 4, 2, 6
    tables = R.rope3d_tables(*d, 10000.0, 128, 4, 4)
    kr = np.zeros((1, (sink + window) * hw, nh, D))
    vr = np.zeros_like(kr)
    first = None
    for c in range(30):
        s = c * F
        q, k, v = (_rand((1, F * hw, nh, D), c + 3 * i) for i in range(3))
        G.rope3d_apply_append(q, k, v, kr, vr, tables, F, H, W, s, 0, sink, window)
        if c == 0:
            first = kr[:, :sink * hw].copy()
        np.testing.assert_array_equal(kr[:, :sink * hw], first)
        assert len(G.held_rows(F, H, W, s, sink, window)) <= (sink + window) * hw


def test_sharded_writes_compose():
    """Slices written from their offsets fill the same ring rows as one call."""
    d = (4, 4, 4)
    nh, D, F, H, W, s, sink, window = 2, 12, 3, 3, 5, 21, 1, 5
    tables = R.rope3d_tables(*d, 10000.0, 64, 4, 8)
    n = F * H * W
    q, k, v = (_rand((1, n, nh, D), 50 + i) for i in range(3))
    cap = (sink + window) * H * W
    k1, v1 = np.zeros((1, cap, nh, D)), np.zeros((1, cap, nh, D))
    q1 = G.rope3d_apply_append(q, k, v, k1, v1, tables, F, H, W, s, 0, sink, window)
    k2, v2 = np.zeros_like(k1), np.zeros_like(v1)
    parts = []
    for a, b in ((0, 11), (11, 30), (30, n)):
        parts.append(G.rope3d_apply_append(q[:, a:b], k[:, a:b], v[:, a:b], k2, v2, tables,
                                           F, H, W, s, a, sink, window))
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), q1)
    np.testing.assert_array_equal(k2, k1)
    np.testing.assert_array_equal(v2, v1)


@pytest.mark.parametrize("H,W,bh,bw", [(8, 16, 8, 8), (4, 6, 2, 3), (6, 4, 1, 4), (4, 4, 4, 4)])
def test_blockified_frame_rows(H, W, bh, bw):
    """Blockify: a permutation of each frame's rows in which every (bh x bw)
    tile occupies consecutive rows, tiles in row-major order, tokens
    row-major inside a tile (brute-force enumeration)."""
    rows = {}
    expect_block = 0
    for hb in range(H // bh):
        for wb in range(W // bw):
            members = [(hb * bh + dh, wb * bw + dw) for dh in range(bh) for dw in range(bw)]
            for j, (h, w) in enumerate(members):
                rows[(h, w)] = expect_block * bh * bw + j
            expect_block += 1
    got = {(h, w): int(G.frame_row(h, w, H, W, bh, bw)) for h in range(H) for w in range(W)}
    assert got == rows
    assert sorted(got.values()) == list(range(H * W))
    p = G.positions(2, H, W, 6, 3, 2 * H * W - 3, 1, 3, bh, bw)
    plain = G.positions(2, H, W, 6, 3, 2 * H * W - 3, 1, 3)
    np.testing.assert_array_equal(p[:, :3], plain[:, :3])
    np.testing.assert_array_equal(p[:, 3] // (H * W), plain[:, 3] // (H * W))   # same slots


def test_blockify_leaves_ring_attention_unchanged():
    """Blockify only permutes rows inside the held frames: attention over the
    held memory is the same up to rounding."""
    d = (4, 4, 4)
    nh, D, F, H, W, sink, window = 2, 12, 2, 4, 4, 1, 3
    tables = R.rope3d_tables(*d, 10000.0, 64, 4, 4)
    outs = []
    for bh, bw in ((0, 0), (2, 2)):
        cap = (sink + window) * H * W
        kr, vr = np.zeros((1, cap, nh, D)), np.zeros((1, cap, nh, D))
        for c in range(5):
            q, k, v = (_rand((1, F * H * W, nh, D), 40 + 3 * c + i) for i in range(3))
            qr = G.rope3d_apply_append(q, k, v, kr, vr, tables, F, H, W, c * F, 0, sink, window,
                                       bh, bw)
        outs.append(G.ring_attention(qr, kr, vr, F, H, W, (5 - 1) * F, sink, window, 0.3))
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-13)


def test_errors():
    with pytest.raises(ValueError):
        G.held_frames(3, 0, 0, 2)            # window smaller than a chunk
    with pytest.raises(ValueError):
        G.positions(1, 2, 2, 0, 0, 4, -1, 3)
    with pytest.raises(ValueError):
        G.positions(1, 4, 6, 0, 0, 4, 0, 3, 4, 4)       # 4 does not divide 6
    with pytest.raises(ValueError):
        G.rope3d_apply_append(np.zeros((1, 4, 1, 12)), np.zeros((1, 4, 1, 12)),
                              np.zeros((1, 4, 1, 12)), np.zeros((1, 4, 1, 12)),
                              np.zeros((1, 4, 1, 12)), R.rope3d_tables(4, 4, 4, 1e4, 8, 4, 4),
                              1, 2, 2, 0, 0, 0, 2)
