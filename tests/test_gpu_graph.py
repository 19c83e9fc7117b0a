"""The hot-path step captured in a HIP graph (torch.cuda.CUDAGraph over the
caller's stream) replays to the same bits as the eager calls.

The step is rope3d_apply_append then chunk_causal_attn on a 480P-shaped
chunk (smaller grid, same head shape); a second graph holds the fused QKV
projection and block-sparse attention with 64- and 48-row blocks; a third,
an attention launch whose unchecked sweep fails its certificate and sweeps
again checked.  Each graph is replayed several times
with eager work and synchronisations between replays, and every replay's
q', cache and attention output are compared with the eager result bit for
bit.  The library records no memset or allocation, so replays need nothing
reset.
"""
import math

import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import say, to_dev, torch
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_bitwise():
    t = torch()
    F, H, W, s, nh, D = 3, 10, 16, 6, 4, 128
    L, hw = F * H * W, H * W
    cfg = rcc.rope_cfg(44, 42, 42, 64, 16, 16)
    tables = rcc.rope3d_tables(cfg)
    g = rcc.grid(F, H, W, s, 0)
    q, k, v = (to_dev(synth.normal((1, L, nh, D), 90 + i, "bf16"), "bf16") for i in range(3))
    cap = (s + F) * hw
    kc0 = to_dev(synth.normal((1, cap, nh, D), 95, "bf16"), "bf16")
    vc0 = to_dev(synth.normal((1, cap, nh, D), 96, "bf16"), "bf16")
    scale = 1.0 / math.sqrt(D)

    def step(kc, vc, qo, out):
        rcc.rope3d_apply_append(tables, g, q, k, v, qo, kc, vc)
        rcc.chunk_causal_attn(qo, kc, vc, out, s * hw, cap, L, scale)

    say("graph: eager reference")
    e_kc, e_vc = kc0.clone(), vc0.clone()
    e_qo, e_out = t.empty_like(q), t.empty_like(q)
    step(e_kc, e_vc, e_qo, e_out)
    t.cuda.synchronize()

    kc, vc = kc0.clone(), vc0.clone()
    qo, out = t.empty_like(q), t.empty_like(q)
    graph = t.cuda.CUDAGraph()
    say("graph: capture")
    with t.cuda.graph(graph):
        step(kc, vc, qo, out)
    t.cuda.synchronize()
    i16 = t.int16
    for r in range(4):
        for x in (qo, out):
            x.fill_(float("nan"))
        kc.copy_(kc0)
        vc.copy_(vc0)
        scratch = t.empty_like(q)                     # eager work between replays
        step(kc0.clone(), vc0.clone(), scratch, t.empty_like(q))
        t.cuda.synchronize()
        say("graph: replay", r)
        graph.replay()
        t.cuda.synchronize()
        for got, ref in ((qo, e_qo), (kc, e_kc), (vc, e_vc), (out, e_out)):
            assert bool((got.view(i16) == ref.view(i16)).all()), r


def test_graph_of_fused_qkv_and_block_sparse_replays_bitwise():
    """The fused QKV projection writing q' and the cache, then block-sparse
    attention of q' over the cache with [1,8,8]-sized (64) and [3,4,4]-sized
    (48) blocks, captured together; replays match the eager calls bit for
    bit."""
    t = torch()
    import numpy as np
    F, H, W, s, nh, D, K = 2, 8, 16, 2, 2, 128, 256
    L, hw = F * H * W, H * W
    cfg = rcc.rope_cfg(44, 42, 42, 16, 16, 16)
    tables = rcc.rope3d_tables(cfg)
    g = rcc.grid(F, H, W, s, 0)
    x = to_dev(synth.normal((1, L, K), 120, "bf16"), "bf16")
    wq = (to_dev(synth.normal((3 * nh * D, K), 121, "bf16"), "bf16").float() /
          math.sqrt(K)).to(t.bfloat16)
    cap = (s + F) * hw
    kc0 = to_dev(synth.normal((1, cap, nh, D), 122, "bf16"), "bf16")
    vc0 = to_dev(synth.normal((1, cap, nh, D), 123, "bf16"), "bf16")
    lists = {}
    gen = np.random.Generator(np.random.PCG64(124))
    for blk in (64, 48):
        n_qb, n_kb = -(-L // blk), cap // blk
        p = gen.choice(n_kb, size=(1, nh, 2), replace=False).astype(np.int32)
        loc = gen.integers(-1, n_kb, size=(1, nh, n_qb, 3)).astype(np.int32)
        lists[blk] = (t.from_numpy(p).cuda(), t.from_numpy(loc).cuda())
    scale = 1.0 / math.sqrt(D)

    def step(kc, vc, qo, outs):
        rcc.qkv_rope_append(tables, g, x, wq, None, qo, kc, vc)
        for blk, o in zip((64, 48), outs):
            rcc.block_sparse_attn(qo, kc, vc, o, cap, blk, *lists[blk], scale)

    say("graph (qkv + block-sparse): eager reference")
    e_kc, e_vc, e_qo = kc0.clone(), vc0.clone(), t.empty(1, L, nh, D, device="cuda",
                                                        dtype=t.bfloat16)
    e_outs = [t.empty_like(e_qo) for _ in range(2)]
    step(e_kc, e_vc, e_qo, e_outs)
    t.cuda.synchronize()
    assert all(bool(t.isfinite(o).all()) for o in e_outs)

    kc, vc, qo = kc0.clone(), vc0.clone(), t.empty_like(e_qo)
    outs = [t.empty_like(e_qo) for _ in range(2)]
    graph = t.cuda.CUDAGraph()
    say("graph (qkv + block-sparse): capture")
    with t.cuda.graph(graph):
        step(kc, vc, qo, outs)
    t.cuda.synchronize()
    i16 = t.int16
    for r in range(3):
        for y in [qo] + outs:
            y.fill_(float("nan"))
        kc.copy_(kc0)
        vc.copy_(vc0)
        step(kc0.clone(), vc0.clone(), t.empty_like(e_qo), [t.empty_like(e_qo) for _ in range(2)])
        t.cuda.synchronize()
        say("graph (qkv + block-sparse): replay", r)
        graph.replay()
        t.cuda.synchronize()
        for got, ref in [(qo, e_qo), (kc, e_kc), (vc, e_vc)] + list(zip(outs, e_outs)):
            assert bool((got.view(i16) == ref.view(i16)).all()), r


def test_graph_replay_of_the_certificate_fallback():
    """Dense attention on scores that jump past the fp32 exponent range late
    in the key range: the unchecked sweep fails its certificate and every
    workgroup sweeps again with every step checked.  Captured in a graph,
    the launch (the decision and the second sweep included) replays to the
    eager bits."""
    t = torch()
    import numpy as np
    lq, kv, d = 256, 2048, 128
    g = np.random.Generator(np.random.PCG64(130))
    u = g.standard_normal(d)
    u /= np.linalg.norm(u)
    q = synth.bf16_bits_to_f32(synth.normal((1, lq, 2, d), 131, "bf16")) + 6.0 * u
    k = synth.bf16_bits_to_f32(synth.normal((1, kv, 2, d), 132, "bf16"))
    k[0, 1900:1903] += 400.0 * u
    dq = to_dev(synth.f32_to_bf16_bits(q.astype(np.float32)), "bf16")
    dk = to_dev(synth.f32_to_bf16_bits(k.astype(np.float32)), "bf16")
    dv = to_dev(synth.normal((1, kv, 2, d), 133, "bf16"), "bf16")
    scale = 1.0 / math.sqrt(d)
    say("graph (certificate fallback): eager reference")
    ref = t.empty_like(dq)
    rcc.chunk_causal_attn(dq, dk, dv, ref, kv - lq, kv, kv, scale)
    t.cuda.synchronize()
    assert bool(t.isfinite(ref).all())
    out = t.empty_like(dq)
    graph = t.cuda.CUDAGraph()
    say("graph (certificate fallback): capture")
    with t.cuda.graph(graph):
        rcc.chunk_causal_attn(dq, dk, dv, out, kv - lq, kv, kv, scale)
    t.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        scratch = t.empty_like(dq)
        rcc.chunk_causal_attn(dq, dk, dv, scratch, kv - lq, kv, kv, scale)
        t.cuda.synchronize()
        say("graph (certificate fallback): replay", r)
        graph.replay()
        t.cuda.synchronize()
        assert bool((out.view(t.int16) == ref.view(t.int16)).all()), r

