"""Pins of the RoPE/position/append oracle to facts outside the oracle.

Each test ties ``oracle.rope3d`` to something it does not compute itself:
a third-party interleaved-RoPE implementation (GPT-J's, from the
``transformers`` package), the start-frame worked example printed in
Yuan & Li §3.3.2 item 1, brute-force grid enumeration, Algorithm 2's
broadcast construction over the full chunk (the unsharded run), and the
textbook RoPE invariants (identity at 0, norm preservation, composition,
relative position).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import rope3d as R
from rope_chunk_causal_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tables(d=(8, 8, 8), theta=10000.0, mx=(64, 32, 32)):
    return R.rope3d_tables(d[0], d[1], d[2], theta, mx[0], mx[1], mx[2])


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# --------------------------------------------------------------------------
# positions
# --------------------------------------------------------------------------

def test_start_frame_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "start_frames_tau3.json")))
    tau = g["tau"]
    for k, s in enumerate(g["start_frame_of_block"]):
        assert s == k * tau
        pos = R.positions(tau, 2, 3, s, 0, tau * 6)
        # local frame f of block k has global time index f + s
        np.testing.assert_array_equal(pos[:, 0], s + np.repeat(np.arange(tau), 6))
    # block 2, local frame 1 -> global frame 7
    pos = R.positions(3, 2, 3, 6, 6, 6)
    assert set(pos[:, 0].tolist()) == {7}


@pytest.mark.parametrize("F,H,W,s", [(2, 4, 4, 0), (2, 4, 4, 4), (3, 30, 52, 6),
                                     (3, 5, 7, 9), (1, 1, 1, 3)])
def test_positions_brute_force_grid(F, H, W, s):
    """Flat-index formula == nested row-major enumeration of the (F,H,W) grid."""
    rows = []
    for f in range(F):
        for h in range(H):
            for w in range(W):
                rows.append((s + f, h, w))
    brute = np.array(rows, dtype=np.int64)
    n = F * H * W
    pos = R.positions(F, H, W, s, 0, n)
    np.testing.assert_array_equal(pos[:, :3], brute)
    # cache rows: global frame-major order from frame 0
    np.testing.assert_array_equal(pos[:, 3], (brute[:, 0] * H + brute[:, 1]) * W + brute[:, 2])


@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_positions_shard_rule(P):
    """A rank's slice computed from its offset == that slice of the full chunk."""
    F, H, W, s = 3, 30, 52, 9
    L = F * H * W
    full = R.positions(F, H, W, s, 0, L)
    bounds = [(r * L) // P for r in range(P + 1)]
    for r in range(P):
        a, b = bounds[r], bounds[r + 1]
        np.testing.assert_array_equal(R.positions(F, H, W, s, a, b - a), full[a:b])


def test_positions_shard_boundaries_mid_row_and_frame():
    F, H, W, s = 3, 30, 52, 9
    p1 = R.positions(F, H, W, s, 585, 1)[0]     # rank 1 of 8 starts mid-row
    assert tuple(p1[:3]) == (9, 11, 13)
    p2 = R.positions(F, H, W, s, 1170, 585)      # rank 2 straddles frame 1560
    assert p2[1559 - 1170, 0] == 9 and p2[1560 - 1170, 0] == 10
    assert tuple(p2[1560 - 1170, 1:3]) == (0, 0)


# --------------------------------------------------------------------------
# tables and rotation against an independent interleaved-RoPE implementation
# --------------------------------------------------------------------------

def _gptj_rotate(x_band, pos_1d, dim):
    """GPT-J's interleaved rotary (transformers) on one band; x_band [n, heads, dim]."""
    torch = pytest.importorskip("torch")
    gptj = pytest.importorskip("transformers.models.gptj.modeling_gptj")
    emb = gptj.create_sinusoidal_positions(int(pos_1d.max()) + 1, dim)  # fp32 sin|cos
    e = emb[torch.as_tensor(pos_1d)][None]                              # [1, n, dim]
    sin, cos = torch.split(e, dim // 2, dim=-1)
    t = torch.as_tensor(x_band, dtype=torch.float32)[None]
    return gptj.apply_rotary_pos_emb(t, sin, cos)[0].double().numpy()


@pytest.mark.parametrize("d", [(8, 8, 8), (44, 42, 42), (4, 6, 2)])
def test_rotation_matches_gptj_interleaved_rope_per_band(d):
    """Per band, the oracle equals GPT-J's interleaved RoPE at that band's coordinate.

    Pins the pair layout (adjacent pairs), the sign of the rotation, the
    per-band schedule theta^(-2j/d_b) and the t, h, w band order.
    """
    F, H, W, s = 3, 5, 7, 6
    n = F * H * W
    D = sum(d)
    tables = _tables(d, mx=(16, 8, 8))
    pos = R.positions(F, H, W, s, 0, n)
    x = _rand((1, n, 3, D), 7)
    y = R.rope3d_apply(x, tables, pos)[0]
    off = 0
    for b, db in enumerate(d):
        ref = _gptj_rotate(x[0, :, :, off:off + db], pos[:, b], db)
        np.testing.assert_allclose(y[:, :, off:off + db], ref, atol=2e-5, rtol=0)
        off += db


def test_unit_vector_closed_form():
    """x = e_{2j} rotates to (cos phi_j, sin phi_j) in slots (2j, 2j+1)."""
    d = (8, 8, 8)
    tables = _tables(d)
    pos = np.array([[5, 3, 2, 0]], dtype=np.int64)
    coord = {0: 5, 1: 3, 2: 2}
    for j in range(12):
        x = np.zeros((1, 1, 1, 24))
        x[..., 2 * j] = 1.0
        y = R.rope3d_apply(x, tables, pos)[0, 0, 0]
        band, jj = divmod(j, 4)
        phi = coord[band] * 10000.0 ** (-2.0 * jj / 8)
        assert abs(y[2 * j] - math.cos(phi)) < 1e-15
        assert abs(y[2 * j + 1] - math.sin(phi)) < 1e-15
        others = np.delete(y, [2 * j, 2 * j + 1])
        assert not others.any()


def test_table_known_values():
    ft, fh, fw = _tables((44, 42, 42), mx=(1024, 64, 64))
    assert ft.shape == (1024, 22) and fh.shape == (64, 21) and fw.shape == (64, 21)
    assert np.all(ft[0] == 1.0)                     # position 0: identity
    assert ft[1, 0] == complex(math.cos(1.0), math.sin(1.0))   # theta_0 = 1
    # lowest frequency of a band of d_b dims is theta^(-(d_b-2)/d_b)
    np.testing.assert_allclose(np.angle(fh[1, -1]), 10000.0 ** (-40.0 / 42), rtol=1e-14)
    np.testing.assert_allclose(np.abs(ft), 1.0, atol=1e-15)


def test_identity_at_origin_and_bandwise_identity():
    tables = _tables()
    x = _rand((2, 1, 3, 24), 1)
    y = R.rope3d_apply(x, tables, np.array([[0, 0, 0, 0]]))
    assert np.array_equal(x, y)
    # h = 0: the h band is unchanged exactly, the others move
    y = R.rope3d_apply(x, tables, np.array([[4, 0, 3, 0]]))
    assert np.array_equal(y[..., 8:16], x[..., 8:16])
    assert not np.allclose(y[..., 0:8], x[..., 0:8])
    assert not np.allclose(y[..., 16:24], x[..., 16:24])


def test_norm_preserved_per_pair():
    tables = _tables((44, 42, 42), mx=(1024, 64, 64))
    pos = R.positions(3, 30, 52, 1020, 0, 3 * 30 * 52)[:: 37]
    x = _rand((1, len(pos), 2, 128), 3)
    y = R.rope3d_apply(x, tables, pos)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13, atol=1e-15)


def test_composition():
    """R(a) R(b) = R(a + b) for 3D positions a, b."""
    tables = _tables(mx=(64, 32, 32))
    x = _rand((1, 1, 2, 24), 5)
    a = np.array([[3, 2, 7, 0]])
    b = np.array([[9, 5, 1, 0]])
    ab = a + b
    y = R.rope3d_apply(R.rope3d_apply(x, tables, a), tables, b)
    np.testing.assert_allclose(y, R.rope3d_apply(x, tables, ab), atol=1e-13)


def test_relative_position_invariant():
    """<R(p) q, R(p') k> depends only on p - p' (any 3D shift)."""
    tables = _tables(mx=(64, 32, 32))
    q = _rand((1, 1, 1, 24), 11)
    k = _rand((1, 1, 1, 24), 12)
    p, pp = np.array([[7, 2, 5, 0]]), np.array([[3, 6, 1, 0]])
    base = np.sum(R.rope3d_apply(q, tables, p) * R.rope3d_apply(k, tables, pp))
    for shift in ([1, 0, 0], [0, 3, 0], [0, 0, 9], [20, 7, 4]):
        sh = np.array([shift + [0]])
        v = np.sum(R.rope3d_apply(q, tables, p + sh) * R.rope3d_apply(k, tables, pp + sh))
        assert abs(v - base) < 1e-12
    # and it does change with the difference
    v = np.sum(R.rope3d_apply(q, tables, p + np.array([[1, 0, 0, 0]])) *
               R.rope3d_apply(k, tables, pp))
    assert abs(v - base) > 1e-6


def _algorithm2_full_chunk(x, tables, F, H, W, s):
    """Algorithm 2's construction: broadcast the three tables over (F,H,W), cat, multiply."""
    ft, fh, fw = tables
    ct, ch, cw = ft.shape[1], fh.shape[1], fw.shape[1]
    f = np.concatenate([
        np.broadcast_to(ft[s:s + F].reshape(F, 1, 1, ct), (F, H, W, ct)),
        np.broadcast_to(fh[:H].reshape(1, H, 1, ch), (F, H, W, ch)),
        np.broadcast_to(fw[:W].reshape(1, 1, W, cw), (F, H, W, cw)),
    ], axis=-1).reshape(F * H * W, 1, -1)
    b, n, nh, d = x.shape
    xc = x.reshape(b, n, nh, -1, 2)
    y = (xc[..., 0] + 1j * xc[..., 1]) * f[None]
    return np.stack([y.real, y.imag], axis=-1).reshape(b, n, nh, d)


@pytest.mark.parametrize("P", [1, 2, 8])
def test_shard_equals_unsharded_algorithm2(P):
    """Shard r from (Delta = r*L/P, s) is bit-equal to the unsharded run's slice."""
    F, H, W, s = 3, 6, 10, 9
    L = F * H * W
    tables = _tables((8, 8, 8), mx=(16, 8, 16))
    x = _rand((2, L, 3, 24), 21)
    full = _algorithm2_full_chunk(x, tables, F, H, W, s)
    for r in range(P):
        a, b = (r * L) // P, ((r + 1) * L) // P
        pos = R.positions(F, H, W, s, a, b - a)
        shard = R.rope3d_apply(x[:, a:b], tables, pos)
        assert np.array_equal(shard, full[:, a:b])


def test_brute_force_rotation_loops_tiny():
    """Explicit per-element 2x2 rotations with math.cos/sin == complex form."""
    wl = synth.WORKLOADS["tiny"]
    d_t, d_h, d_w = synth.wan_band_split(wl.head_dim)
    tables = _tables((d_t, d_h, d_w))
    pos = R.positions(2, 4, 4, 4, 0, 32)
    x = synth.to_f64(synth.normal((1, 32, 2, 24), 1, "f32"), "f32")
    y = R.rope3d_apply(x, tables, pos)
    bands = [(0, d_t), (d_t, d_h), (d_t + d_h, d_w)]
    for i in range(32):
        for h in range(2):
            for b, (off, db) in enumerate(bands):
                for j in range(db // 2):
                    phi = pos[i, b] * math.pow(10000.0, -2.0 * j / db)
                    c, sn = math.cos(phi), math.sin(phi)
                    x0 = x[0, i, h, off + 2 * j]
                    x1 = x[0, i, h, off + 2 * j + 1]
                    assert abs(y[0, i, h, off + 2 * j] - (x0 * c - x1 * sn)) < 1e-14
                    assert abs(y[0, i, h, off + 2 * j + 1] - (x0 * sn + x1 * c)) < 1e-14


# --------------------------------------------------------------------------
# KV-cache write
# --------------------------------------------------------------------------

def test_append_rows_and_untouched_neighbours():
    F, H, W, s, delta, n = 2, 4, 4, 4, 5, 20
    tables = _tables(mx=(16, 8, 8))
    q, k, v = (_rand((2, n, 2, 24), i) for i in (1, 2, 3))
    cap = (s + F) * H * W + 3
    kc = np.full((2, cap, 2, 24), 7.0)
    vc = np.full((2, cap, 2, 24), -7.0)
    qr = R.rope3d_apply_append(q, k, v, kc, vc, tables, F, H, W, s, delta)
    row0 = s * H * W + delta
    pos = R.positions(F, H, W, s, delta, n)
    np.testing.assert_array_equal(qr, R.rope3d_apply(q, tables, pos))
    np.testing.assert_array_equal(kc[:, row0:row0 + n], R.rope3d_apply(k, tables, pos))
    np.testing.assert_array_equal(vc[:, row0:row0 + n], v)      # V is not rotated
    assert np.all(kc[:, :row0] == 7.0) and np.all(kc[:, row0 + n:] == 7.0)
    assert np.all(vc[:, :row0] == -7.0) and np.all(vc[:, row0 + n:] == -7.0)


def test_append_cache_too_small_raises():
    tables = _tables(mx=(16, 8, 8))
    q = np.zeros((1, 4, 1, 24))
    kc = np.zeros((1, 10, 1, 24))
    with pytest.raises(ValueError):
        R.rope3d_apply_append(q, q, q, kc, kc.copy(), tables, 1, 2, 2, 2, 0)
