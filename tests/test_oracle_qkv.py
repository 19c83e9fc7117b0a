"""Pins of the fused QKV + Causal-RoPE oracle to facts outside it.

``oracle.qkv`` is tied to: a brute-force per-element sum over the model
dimension (pure Python loops on a tiny case), the identity projection (q, k,
v become x, 2x, 3x), one-hot weights that pin the stacking order of the
q, k, v row groups and the head-major layout inside each, a bias-only
projection, and the RoPE oracle applied to the identity projection (which
fixes the glue between the projection and the rotation).  CPU only.
"""
import numpy as np
import pytest

from oracle import qkv as Q
from oracle import rope3d as R


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def test_projection_brute_force():
    B, n, K, H, D = 2, 3, 5, 2, 4
    x = _rand((B, n, K), 1)
    w = _rand((3 * H * D, K), 2)
    b = _rand((3 * H * D,), 3)
    q, k, v = Q.qkv_project(x, w, b, H, D)
    out = (q, k, v)
    for bi in range(B):
        for i in range(n):
            for which in range(3):
                for h in range(H):
                    for d in range(D):
                        o = which * H * D + h * D + d
                        s = b[o]
                        for c in range(K):
                            s += x[bi, i, c] * w[o, c]
                        assert abs(out[which][bi, i, h, d] - s) <= 1e-12 * (1 + abs(s))


def test_identity_projection():
    B, n, H, D = 1, 7, 3, 8
    x = _rand((B, n, H * D), 4)
    eye = np.eye(H * D)
    w = np.concatenate([eye, 2 * eye, 3 * eye])
    q, k, v = Q.qkv_project(x, w, None, H, D)
    xr = x.reshape(B, n, H, D)
    np.testing.assert_array_equal(q, xr)
    np.testing.assert_array_equal(k, 2 * xr)
    np.testing.assert_array_equal(v, 3 * xr)


@pytest.mark.parametrize("which,h,d", [(0, 0, 0), (0, 1, 5), (1, 0, 3), (1, 2, 7), (2, 2, 0)])
def test_one_hot_row_lands_in_its_slot(which, h, d):
    B, n, K, H, D = 1, 2, 6, 3, 8
    x = _rand((B, n, K), 5)
    w = np.zeros((3 * H * D, K))
    w[which * H * D + h * D + d, 2] = 1.0
    out = Q.qkv_project(x, w, None, H, D)
    for t in range(3):
        expect = np.zeros((B, n, H, D))
        if t == which:
            expect[:, :, h, d] = x[:, :, 2]
        np.testing.assert_array_equal(out[t], expect)


def test_bias_only():
    B, n, K, H, D = 2, 4, 3, 2, 4
    b = _rand((3 * H * D,), 6)
    q, k, v = Q.qkv_project(np.zeros((B, n, K)), np.zeros((3 * H * D, K)), b, H, D)
    for t, y in enumerate((q, k, v)):
        np.testing.assert_array_equal(y, np.broadcast_to(b[t * H * D:(t + 1) * H * D].reshape(H, D),
                                                          (B, n, H, D)))


def test_fused_equals_rope_of_identity_projection():
    """With W = [I; I; I] the fused path is RoPE + append of x itself."""
    d = (8, 8, 8)
    H, D = 2, sum(d)
    F, Hg, Wg, s, off, n = 2, 4, 4, 2, 5, 20
    tables = R.rope3d_tables(*d, 10000.0, 16, 8, 8)
    x = _rand((1, n, H * D), 7)
    eye = np.eye(H * D)
    w = np.concatenate([eye, eye, eye])
    cap = (s + F) * Hg * Wg
    kc, vc = np.zeros((1, cap, H, D)), np.zeros((1, cap, H, D))
    q = Q.qkv_rope_append(x, w, None, H, D, kc, vc, tables, F, Hg, Wg, s, off)
    pos = R.positions(F, Hg, Wg, s, off, n)
    xr = x.reshape(1, n, H, D)
    rot = R.rope3d_apply(xr, tables, pos)
    np.testing.assert_array_equal(q, rot)
    np.testing.assert_array_equal(kc[:, pos[:, 3]], rot)
    np.testing.assert_array_equal(vc[:, pos[:, 3]], xr)
    untouched = np.setdiff1d(np.arange(cap), pos[:, 3])
    assert not kc[:, untouched].any() and not vc[:, untouched].any()


def test_shape_errors():
    with pytest.raises(ValueError):
        Q.qkv_project(np.zeros((1, 2, 4)), np.zeros((5, 4)), None, 1, 2)
