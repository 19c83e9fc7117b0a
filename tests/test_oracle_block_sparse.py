"""Pins of the block-sparse attention oracle to facts outside it.

``oracle.block_sparse`` is tied to: brute force (Python loops over every
cache row, keeping the rows whose block a Python set holds), PyTorch's fp64
scaled_dot_product_attention with a boolean token mask built from the
lists, the dense chunk-causal oracle when every block is selected, closed
forms (identical keys average V; an empty selection gives zeros), and the
rule that padding, out-of-range entries, repeats and list order change
nothing.  CPU only.
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import block_sparse as S


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _lists(seed, B, nh, n_qb, n_kb, n_p, n_l):
    g = np.random.Generator(np.random.PCG64(seed))
    persist = g.integers(-1, n_kb + 2, size=(B, nh, n_p))
    local = g.integers(-1, n_kb + 2, size=(B, nh, n_qb, n_l))
    return persist, local


def _brute(q, kc, vc, kv, blk, persist, local, scale):
    B, n_q, nh, d = q.shape
    n_kb = kv // blk
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(nh):
            for i in range(n_q):
                qb = i // blk
                chosen = {int(x) for x in persist[b, h] if 0 <= x < n_kb}
                chosen |= {int(x) for x in local[b, h, qb] if 0 <= x < n_kb}
                keys = [j for j in range(kv) if j // blk in chosen]
                if not keys:
                    continue
                logits = [scale * sum(q[b, i, h, e] * kc[b, j, h, e] for e in range(d)) for j in keys]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                z = sum(w)
                for e in range(d):
                    out[b, i, h, e] = sum(w[t] * vc[b, keys[t], h, e] for t in range(len(keys))) / z
    return out


@pytest.mark.parametrize("blk,n_q,kv", [
    (4, 10, 24),     # 3 query blocks (last short), 6 key blocks
    (3, 8, 20),      # blocks of an odd size (as 48 = 3 x 16): 3 query blocks, 6 key blocks + 2 rows
    (6, 13, 30),     # 3 query blocks (last of 1 row), 5 key blocks
])
def test_brute_force_tiny(blk, n_q, kv):
    B, nh, d = 2, 2, 4
    n_qb, n_kb = -(-n_q // blk), kv // blk
    q, kc, vc = _rand((B, n_q, nh, d), 1), _rand((B, kv + 3, nh, d), 2), _rand((B, kv + 3, nh, d), 3)
    persist, local = _lists(4, B, nh, n_qb, n_kb, 2, 3)
    got = S.block_sparse_attention(q, kc, vc, kv, blk, persist, local, 0.4)
    np.testing.assert_allclose(got, _brute(q, kc, vc, kv, blk, persist, local, 0.4),
                               rtol=0, atol=1e-12)


def test_matches_torch_sdpa_with_a_token_mask():
    torch = pytest.importorskip("torch")
    B, nh, d, blk, n_q, kv = 1, 3, 8, 8, 40, 96
    q, kc, vc = _rand((B, n_q, nh, d), 5), _rand((B, kv, nh, d), 6), _rand((B, kv, nh, d), 7)
    g = np.random.Generator(np.random.PCG64(8))
    persist = g.integers(0, 12, size=(B, nh, 3))
    local = g.integers(0, 12, size=(B, nh, 5, 4))
    got = S.block_sparse_attention(q, kc, vc, kv, blk, persist, local, 0.3)
    mask = np.zeros((B, nh, n_q, kv), dtype=bool)
    for h in range(nh):
        for i in range(n_q):
            for x in list(persist[0, h]) + list(local[0, h, i // blk]):
                mask[0, h, i, x * blk:(x + 1) * blk] = True
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(kc), t(vc), attn_mask=torch.from_numpy(mask), scale=0.3)
    np.testing.assert_allclose(got, ref.numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-12)


def test_every_block_selected_is_dense_attention():
    B, nh, d, blk = 1, 2, 8, 4
    n_q, kv = 12, 36
    q, kc, vc = _rand((B, n_q, nh, d), 9), _rand((B, kv, nh, d), 10), _rand((B, kv, nh, d), 11)
    persist = np.tile(np.arange(0, 9, 2), (B, nh, 1))                 # even blocks
    local = np.tile(np.arange(1, 9, 2), (B, nh, 3, 1))                 # odd blocks
    got = S.block_sparse_attention(q, kc, vc, kv, blk, persist, local, 0.25)
    # the query chunk is the last chunk of the cache: every key visible
    dense = A.chunk_causal_attention(q, kc, vc, kv - n_q, kv, n_q, 0.25)
    np.testing.assert_allclose(got, dense, rtol=0, atol=1e-13)


def test_identical_keys_average_v_and_empty_gives_zero():
    B, nh, d, blk, n_q, kv = 1, 1, 6, 4, 8, 16
    q = _rand((B, n_q, nh, d), 12)
    kc = _rand((B, kv, nh, d), 13)
    kc[0, 8:12] = kc[0, 8]                     # block 2: four identical keys
    vc = _rand((B, kv, nh, d), 14)
    persist = np.full((B, nh, 1), -1)
    local = np.array([[[[2, -1]], [[-1, 99]]]]).reshape(B, nh, 2, 2)
    got = S.block_sparse_attention(q, kc, vc, kv, blk, persist, local, 1.0)
    np.testing.assert_allclose(got[0, :4, 0], np.tile(vc[0, 8:12, 0].mean(axis=0), (4, 1)),
                               rtol=0, atol=1e-14)
    assert not got[0, 4:].any()                # block 1 selects nothing valid


def test_padding_repeats_and_order_change_nothing():
    B, nh, d, blk, n_q, kv = 1, 2, 8, 4, 16, 40
    q, kc, vc = _rand((B, n_q, nh, d), 15), _rand((B, kv, nh, d), 16), _rand((B, kv, nh, d), 17)
    persist = np.array([3, 7]).reshape(1, 1, 2).repeat(nh, axis=1)
    local = np.array([[0, 5], [1, 2], [9, 4], [6, 8]]).reshape(1, 1, 4, 2).repeat(nh, axis=1)
    ref = S.block_sparse_attention(q, kc, vc, kv, blk, persist, local, 0.5)
    messy_p = np.array([7, -1, 3, 7, 10, -5]).reshape(1, 1, 6).repeat(nh, axis=1)
    messy_l = np.array([[5, 0, 3, -1, 5], [2, 1, 1, 44, -1], [4, 9, 7, 4, -1],
                        [8, 6, 8, 6, 10]]).reshape(1, 1, 4, 5).repeat(nh, axis=1)
    got = S.block_sparse_attention(q, kc, vc, kv, blk, messy_p, messy_l, 0.5)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_persistent_only_is_attention_over_the_gathered_rows():
    B, nh, d, blk, n_q, kv = 2, 2, 8, 8, 24, 64
    q, kc, vc = _rand((B, n_q, nh, d), 18), _rand((B, kv, nh, d), 19), _rand((B, kv, nh, d), 20)
    persist = np.array([[[6, 1, 4], [0, 2, 7]], [[5, 3, 3], [7, 7, 7]]])
    local = np.full((B, nh, 3, 1), -1)
    got = S.block_sparse_attention(q, kc, vc, kv, blk, persist, local, 0.2)
    for b in range(B):
        for h in range(nh):
            blocks = sorted(set(persist[b, h].tolist()))
            rows = np.concatenate([np.arange(x * blk, (x + 1) * blk) for x in blocks])
            g = len(rows)
            ref = A.chunk_causal_attention(q[b:b + 1, :, h:h + 1], kc[b:b + 1, rows][:, :, h:h + 1],
                                           vc[b:b + 1, rows][:, :, h:h + 1], 0, g, g, 0.2)
            np.testing.assert_allclose(got[b:b + 1, :, h:h + 1], ref, rtol=0, atol=1e-13)


def test_shape_errors():
    with pytest.raises(ValueError):
        S.block_sparse_attention(np.zeros((1, 8, 1, 4)), np.zeros((1, 8, 1, 4)),
                                 np.zeros((1, 8, 1, 4)), 8, 4, np.zeros((1, 1, 1), int),
                                 np.zeros((1, 1, 3, 1), int), 1.0)
