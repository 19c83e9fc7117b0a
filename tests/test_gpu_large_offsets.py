"""GPU parity: K/V caches past 4 GiB per batch entry, on the bf16 head_dim-128
kernels (dense chunk-causal and block-sparse).

64 heads make a cache row 16 KB, so rows from 262144 on sit more than 4 GiB
into a batch entry; the caches hold 264192 rows (4.33 GB each for K and V)
and two batch entries, so entry 1 also starts 4.33 GB in.  Two heads carry
seeded data (the others are zeros).  The keys past 4 GiB get a common
component along the queries' shared direction, so they carry most of the
softmax weight: an address that wrapped at 4 GiB would read other rows and
miss the reference by the size of the output itself (rel L2 ~ 1), far past
the 1e-2 bound.  Block-sparse lists select blocks on both sides of 4 GiB.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import Bf16Rows, check_attn, say, to_dev, to_host_f64, torch
from oracle import attention as A
from oracle import block_sparse as S
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu

NH, D, B, NQ = 64, 128, 2, 128
ROWS_4G = (1 << 32) // (NH * D * 2)          # first row past 4 GiB in an entry
CAP = ROWS_4G + 2048
HEADS = (0, NH - 1)                          # heads with data


@pytest.fixture(scope="module")
def big():
    t = torch()
    g = np.random.Generator(np.random.PCG64(901))
    u = g.standard_normal(D)
    u /= np.linalg.norm(u)
    qf = synth.bf16_bits_to_f32(synth.normal((B, NQ, len(HEADS), D), 902, "bf16")) + 4.0 * u
    q = synth.f32_to_bf16_bits(qf.astype(np.float32))
    kf = synth.bf16_bits_to_f32(synth.normal((B, CAP, len(HEADS), D), 903, "bf16"))
    kf[:, ROWS_4G:] += 16.0 * u
    k = synth.f32_to_bf16_bits(kf.astype(np.float32))
    v = synth.normal((B, CAP, len(HEADS), D), 904, "bf16")
    say("caches past 4 GiB per entry", B, CAP, NH, D)
    dq = t.zeros((B, NQ, NH, D), dtype=t.bfloat16, device="cuda")
    dk = t.zeros((B, CAP, NH, D), dtype=t.bfloat16, device="cuda")
    dv = t.zeros_like(dk)
    for i, h in enumerate(HEADS):
        dq[:, :, h] = to_dev(np.ascontiguousarray(q[:, :, i]), "bf16")
        dk[:, :, h] = to_dev(np.ascontiguousarray(k[:, :, i]), "bf16")
        dv[:, :, h] = to_dev(np.ascontiguousarray(v[:, :, i]), "bf16")
    t.cuda.synchronize()
    yield dict(q=q, k=k, v=v, dq=dq, dk=dk, dv=dv)
    del dq, dk, dv
    t.cuda.empty_cache()


def test_dense_attention_cache_past_4gib(big):
    t = torch()
    out = t.full((B, NQ, NH, D), float("nan"), dtype=t.bfloat16, device="cuda")
    say("dense attention, keys past 4 GiB", CAP)
    rcc.chunk_causal_attn(big["dq"], big["dk"], big["dv"], out, CAP - NQ, CAP, NQ,
                          1.0 / math.sqrt(D))
    t.cuda.synchronize()
    assert bool(t.isfinite(out).all())
    ref = A.chunk_causal_attention(synth.to_f64(big["q"], "bf16"), Bf16Rows(big["k"]),
                                   Bf16Rows(big["v"]), CAP - NQ, CAP, NQ, 1.0 / math.sqrt(D))
    got = to_host_f64(out[:, :, list(HEADS)])
    say("dense past 4 GiB", check_attn(got, ref, "dense, cache > 4 GiB"))
    # the heads without data attend zero keys: the mean of zero values
    assert bool((out[:, :, 1:NH - 1] == 0).all())


@pytest.mark.parametrize("blk", [64, 48])
def test_block_sparse_cache_past_4gib(big, blk):
    """Blocks of 64 (a tile inside one block) and of 48 (tiles that span two
    blocks; block ROWS_4G // 48 itself straddles the 4 GiB line)."""
    t = torch()
    far = ROWS_4G // blk                     # the block holding the first row past 4 GiB
    n_kb = CAP // blk
    n_qb = -(-NQ // blk)
    persist = np.array([far, far + 4, 17], dtype=np.int32)
    local = np.array([[n_kb - 1, far + 14, n_kb + 5, -1], [far + 2, 3, n_kb - 1, n_kb - 1],
                      [far + 1, 0, far + 3, -1]], dtype=np.int32)[:n_qb]
    P = np.broadcast_to(persist, (B, NH, 3)).copy()
    Lc = np.broadcast_to(local, (B, NH, n_qb, 4)).copy()
    out = t.full((B, NQ, NH, D), float("nan"), dtype=t.bfloat16, device="cuda")
    say("block-sparse, blocks past 4 GiB", CAP, "block", blk)
    rcc.block_sparse_attn(big["dq"], big["dk"], big["dv"], out, CAP, blk, t.from_numpy(P).cuda(),
                          t.from_numpy(Lc).cuda(), 1.0 / math.sqrt(D))
    t.cuda.synchronize()
    assert bool(t.isfinite(out).all())
    ref = S.block_sparse_attention(synth.to_f64(big["q"], "bf16"), Bf16Rows(big["k"]),
                                   Bf16Rows(big["v"]), CAP, blk, P[:, :len(HEADS)],
                                   Lc[:, :len(HEADS)], 1.0 / math.sqrt(D))
    got = to_host_f64(out[:, :, list(HEADS)])
    say("sparse past 4 GiB", check_attn(got, ref, "block-sparse, cache > 4 GiB"))
