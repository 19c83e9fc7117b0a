"""The hot-path step captured in a HIP graph (torch.cuda.CUDAGraph over the
caller's stream) replays to the same bits as the eager calls.

The step is rope3d_apply_append then chunk_causal_attn on a 480P-shaped
chunk (smaller grid, same head shape).  The graph is replayed several times
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
