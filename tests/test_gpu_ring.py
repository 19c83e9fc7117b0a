"""GPU parity: the rolling-window ring (positions, RoPE + ring write, fused
QKV + ring write, attention over the held memory) vs ``oracle.ring``.

Every case drives a rollout long enough to wrap the ring, so rows are
evicted and overwritten.  The oracle keeps its own ring from the same seeded
inputs; for attention it stores the rotated k at the ring's storage
precision (bf16, nearest-even), as the GPU ring does.  Rules: positions
bit-exact; fp32 RoPE within 1e-5; bf16 RoPE within max(1e-2, half a bf16
ulp); attention max 2e-2 / mean 2e-3.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import check_attn, check_bf16_rope, say, to_dev, to_host_f64, torch, wave_rows
from oracle import qkv as Q
from oracle import ring as G
from oracle import rope3d as R
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu


def _bf16(x64: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x64.astype(np.float32))).astype(np.float64)


@pytest.mark.parametrize("F,H,W,s,off,n,sink,window,bh,bw", [
    (3, 30, 52, 237, 0, 4680, 0, 21, 0, 0),        # last chunk of a 1 min rollout
    (3, 30, 52, 237, 2 * 585, 585, 3, 18, 0, 0),   # one SP rank's slice, with sinks
    (2, 4, 5, 0, 0, 40, 1, 4, 0, 0),               # sink frame written
    (2, 4, 5, 9, 7, 20, 1, 4, 0, 0),
    (1, 3, 3, 1000, 0, 9, 5, 1, 0, 0),             # window of one frame
    (3, 32, 56, 57, 0, 5376, 3, 12, 8, 8),         # [1,8,8] blocks of a 896x512 frame
    (3, 32, 56, 57, 1000, 1337, 0, 6, 4, 8),       # a slice, non-square blocks
    (2, 6, 9, 4, 5, 90, 1, 3, 3, 3),
])
def test_ring_positions_bit_exact(F, H, W, s, off, n, sink, window, bh, bw):
    say("ring positions", F, H, W, s, off, n, sink, window, bh, bw)
    got = rcc.ring_positions(rcc.grid(F, H, W, s, off), rcc.ring(sink, window, bh, bw), n)
    torch().cuda.synchronize()
    ref = G.positions(F, H, W, s, off, n, sink, window, bh, bw)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), ref)


def test_ring_rollout_tiny_fp32_every_element():
    """fp32 generic path: sink 1, window 4 frames, chunks of 2 frames, 8 chunks x 2 steps."""
    t = torch()
    d, nh, F, H, W, sink, window = (8, 8, 8), 2, 2, 4, 4, 1, 4
    D, hw = sum(d), H * W
    cfg = rcc.rope_cfg(*d, 32, 8, 8)
    tables = rcc.rope3d_tables(cfg)
    otab = R.rope3d_tables(*d, 10000.0, 32, 8, 8)
    cap = (sink + window) * hw
    kr = t.full((1, cap, nh, D), float("nan"), device="cuda")
    vr = t.full_like(kr, float("nan"))
    okr, ovr = np.full((1, cap, nh, D), np.nan), np.full((1, cap, nh, D), np.nan)
    scale = 1.0 / math.sqrt(D)
    for c in range(8):
        s = c * F
        for step in range(2):
            host = [synth.normal((1, F * hw, nh, D), 1000 * c + 10 * step + i, "f32")
                    for i in range(3)]
            dq, dk, dv = (to_dev(x, "f32") for x in host)
            qo, out = t.empty_like(dq), t.full_like(dq, float("nan"))
            g, r = rcc.grid(F, H, W, s, 0), rcc.ring(sink, window)
            say("ring tiny fp32 chunk", c, "step", step)
            rcc.rope3d_apply_append_ring(tables, g, r, dq, dk, dv, qo, kr, vr)
            rcc.chunk_causal_attn_ring(g, r, qo, kr, vr, out, scale)
            t.cuda.synchronize()
            q, k, v = (x.astype(np.float64) for x in host)
            oq = G.rope3d_apply_append(q, k, v, okr, ovr, otab, F, H, W, s, 0, sink, window)
            assert np.abs(to_host_f64(qo) - oq).max() <= 1e-5
            held = G.held_rows(F, H, W, s, sink, window)
            assert held.max() < rcc.ring_held_tokens(g, r) == len(held)
            assert np.abs(to_host_f64(kr)[:, held] - okr[:, held]).max() <= 1e-5
            assert np.array_equal(to_host_f64(vr)[:, held], ovr[:, held])
            ref = G.ring_attention(oq, okr, ovr, F, H, W, s, sink, window, scale)
            check_attn(to_host_f64(out), ref, f"tiny c{c}s{step}")


def test_ring_rollout_bf16_d128_small():
    """bf16 / head_dim 128 fast path on a small grid: no sinks, window of 7 frames."""
    t = torch()
    d, nh, F, H, W, sink, window = (44, 42, 42), 2, 3, 4, 9, 0, 7
    D, hw = 128, 36
    cfg = rcc.rope_cfg(*d, 64, 8, 16)
    tables = rcc.rope3d_tables(cfg)
    otab = R.rope3d_tables(*d, 10000.0, 64, 8, 16)
    cap = window * hw
    kr = t.zeros((2, cap, nh, D), dtype=t.bfloat16, device="cuda")
    vr = t.zeros_like(kr)
    okr, ovr = np.zeros((2, cap, nh, D)), np.zeros((2, cap, nh, D))
    scale = 1.0 / math.sqrt(D)
    for c in range(9):
        s = c * F
        host = [synth.normal((2, F * hw, nh, D), 77 + 10 * c + i, "bf16") for i in range(3)]
        dq, dk, dv = (to_dev(x, "bf16") for x in host)
        qo, out = t.empty_like(dq), t.full_like(dq, float("nan"))
        g, r = rcc.grid(F, H, W, s, 0), rcc.ring(sink, window)
        say("ring bf16 d128 chunk", c)
        rcc.rope3d_apply_append_ring(tables, g, r, dq, dk, dv, qo, kr, vr)
        rcc.chunk_causal_attn_ring(g, r, qo, kr, vr, out, scale)
        t.cuda.synchronize()
        q, k, v = (synth.to_f64(x, "bf16") for x in host)
        oq = G.rope3d_apply_append(q, k, v, okr, ovr, otab, F, H, W, s, 0, sink, window)
        check_bf16_rope(to_host_f64(qo), oq, f"c{c} q'")
        held = G.held_rows(F, H, W, s, sink, window)
        check_bf16_rope(to_host_f64(kr)[:, held], okr[:, held], f"c{c} k ring")
        ref = G.ring_attention(_bf16(oq), _bf16(okr), ovr, F, H, W, s, sink, window, scale)
        check_attn(to_host_f64(out), ref, f"c{c} attn")


@pytest.mark.parametrize("name,sink,window,last", [
    ("480p_rolling_20s", 0, 21, 78),     # last chunk of the 20 s rollout
    ("480p_rolling_1min", 3, 18, 237),   # last chunk of 1 min, 3 sink frames
])
def test_480p_long_rollout_ring(name, sink, window, last):
    """Real shapes: write enough chunks to wrap the ring, then check every row
    of the held memory, every token of the last chunk's q', and its attention
    on a row of every 32-row wave of every head (the whole NaN-poisoned
    output finite)."""
    t = torch()
    wl = synth.WORKLOADS[name]
    nh, D, F, L, hw = wl.n_heads, wl.head_dim, wl.frames, wl.chunk_tokens, wl.hw
    rs = wl.rope
    cfg = rcc.rope_cfg(rs.d_t, rs.d_h, rs.d_w, rs.max_t, rs.max_h, rs.max_w, rs.theta)
    tables = rcc.rope3d_tables(cfg)
    otab = R.rope3d_tables(rs.d_t, rs.d_h, rs.d_w, rs.theta, rs.max_t, rs.max_h, rs.max_w)
    cap = (sink + window) * hw
    kr = t.zeros((1, cap, nh, D), dtype=t.bfloat16, device="cuda")
    vr = t.zeros_like(kr)
    okr, ovr = np.zeros((1, cap, nh, D)), np.zeros((1, cap, nh, D))
    r = rcc.ring(sink, window)
    # the sink chunk (if any), then 4 chunks more than the window holds
    starts = ([0] if sink else []) + list(range(last - F * (window // F + 3), last + 1, F))
    scale = 1.0 / math.sqrt(D)
    for s in starts:
        host = [synth.normal((1, L, nh, D), synth.seed_for(name, s, 3, x), "bf16")
                for x in ("q", "k", "v")]
        dq, dk, dv = (to_dev(x, "bf16") for x in host)
        qo = t.empty_like(dq)
        g = rcc.grid(F, wl.height, wl.width, s, 0)
        say(name, "ring write s", s)
        rcc.rope3d_apply_append_ring(tables, g, r, dq, dk, dv, qo, kr, vr)
        q, k, v = (synth.to_f64(x, "bf16") for x in host)
        oq = G.rope3d_apply_append(q, k, v, okr, ovr, otab, F, wl.height, wl.width, s, 0,
                                   sink, window)
    out = t.full_like(qo, float("nan"))
    say(name, "ring attention s", last)
    rcc.chunk_causal_attn_ring(g, r, qo, kr, vr, out, scale)
    t.cuda.synchronize()
    assert rcc.ring_held_tokens(g, r) == cap
    check_bf16_rope(to_host_f64(kr), okr, "k ring")
    assert np.array_equal(to_host_f64(vr), ovr)
    check_bf16_rope(to_host_f64(qo), oq, "q'")
    assert bool(t.isfinite(out).all()), f"{name}: non-finite attention output"
    tok = wave_rows(L, 9)
    ref = G.ring_attention(_bf16(oq), _bf16(okr), ovr, F, wl.height, wl.width, last, sink,
                           window, scale, rows=tok)
    check_attn(to_host_f64(out[:, tok]), ref, f"{name} attn")


@pytest.mark.parametrize("bh,bw", [(0, 0), (2, 5)])
def test_qkv_ring_write(bh, bw):
    """Fused projection into the ring: rollout of 6 chunks over a 1 + 3 frame
    ring, frames row-major or blockified into 2 x 5 tiles."""
    t = torch()
    d, nh, F, H, W, sink, window, K = (12, 10, 10), 2, 2, 4, 5, 1, 3, 64
    D, hw = 32, 20
    cfg = rcc.rope_cfg(*d, 32, 8, 8)
    tables = rcc.rope3d_tables(cfg)
    otab = R.rope3d_tables(*d, 10000.0, 32, 8, 8)
    cap = (sink + window) * hw
    kr = t.full((1, cap, nh, D), 7.0, dtype=t.bfloat16, device="cuda")
    vr = t.full_like(kr, 7.0)
    okr, ovr = np.full((1, cap, nh, D), 7.0), np.full((1, cap, nh, D), 7.0)
    wb = synth.normal((3 * nh * D, K), 5, "bf16", scale=1.0 / math.sqrt(K))
    bias = synth.normal((3 * nh * D,), 6, "f32", scale=0.5)
    w, bdev = to_dev(wb, "bf16"), to_dev(bias, "f32")
    for c in range(6):
        s = c * F
        for off, n in ((0, 23), (23, F * hw - 23)):       # two SP-style slices
            xb = synth.normal((1, n, K), 40 + 10 * c + off, "bf16")
            qo = t.empty((1, n, nh, D), dtype=t.bfloat16, device="cuda")
            say("qkv ring chunk", c, "slice", off, n)
            rcc.qkv_rope_append_ring(tables, rcc.grid(F, H, W, s, off),
                                     rcc.ring(sink, window, bh, bw), to_dev(xb, "bf16"), w, bdev,
                                     qo, kr, vr)
            t.cuda.synchronize()
            q, k, v = Q.qkv_project(synth.to_f64(xb, "bf16"), synth.to_f64(wb, "bf16"),
                                    bias.astype(np.float64), nh, D)
            oq = G.rope3d_apply_append(q, k, v, okr, ovr, otab, F, H, W, s, off, sink, window,
                                       bh, bw)
            check_bf16_rope(to_host_f64(qo), oq, f"c{c} q'")
        check_bf16_rope(to_host_f64(kr), okr, f"c{c} k ring")
        check_bf16_rope(to_host_f64(vr), ovr, f"c{c} v ring")


def test_ring_without_eviction_matches_the_plain_cache_bitwise():
    """A ring that never wraps holds exactly the plain cache; the calls agree bit for bit."""
    t = torch()
    wl = synth.WORKLOADS["480p_step"]
    rs = wl.rope
    nh, D, F, L, hw = wl.n_heads, wl.head_dim, wl.frames, wl.chunk_tokens, wl.hw
    cfg = rcc.rope_cfg(rs.d_t, rs.d_h, rs.d_w, rs.max_t, rs.max_h, rs.max_w, rs.theta)
    tables = rcc.rope3d_tables(cfg)
    cap = 3 * L
    caches = [t.zeros((1, cap, nh, D), dtype=t.bfloat16, device="cuda") for _ in range(4)]
    r = rcc.ring(0, 9)
    for s in (0, 3, 6):
        dq, dk, dv = (to_dev(synth.normal((1, L, nh, D), 500 + s + i, "bf16"), "bf16")
                      for i in range(3))
        q1, q2 = t.empty_like(dq), t.empty_like(dq)
        o1, o2 = t.empty_like(dq), t.empty_like(dq)
        g = rcc.grid(F, wl.height, wl.width, s, 0)
        say("ring vs plain s", s)
        rcc.rope3d_apply_append(tables, g, dq, dk, dv, q1, caches[0], caches[1])
        rcc.rope3d_apply_append_ring(tables, g, r, dq, dk, dv, q2, caches[2], caches[3])
        rcc.chunk_causal_attn(q1, caches[0], caches[1], o1, s * hw, (s + F) * hw, L,
                              1.0 / math.sqrt(D))
        rcc.chunk_causal_attn_ring(g, r, q2, caches[2], caches[3], o2, 1.0 / math.sqrt(D))
        t.cuda.synchronize()
        i16 = t.int16
        assert bool((q1.view(i16) == q2.view(i16)).all())
        assert bool((caches[0].view(i16) == caches[2].view(i16)).all())
        assert bool((caches[1].view(i16) == caches[3].view(i16)).all())
        assert bool((o1.view(i16) == o2.view(i16)).all())


def test_ring_errors_reported_without_launch():
    t = torch()
    cfg = rcc.rope_cfg(12, 10, 10, 16, 16, 16)
    tables = rcc.rope3d_tables(cfg)
    q = t.zeros((1, 32, 2, 32), dtype=t.bfloat16, device="cuda")
    kr = t.zeros((1, 48, 2, 32), dtype=t.bfloat16, device="cuda")
    with pytest.raises(rcc.RccError) as e:      # window smaller than the chunk
        rcc.rope3d_apply_append_ring(tables, rcc.grid(2, 4, 4, 0), rcc.ring(0, 1),
                                     q, q, q, q.clone(), kr, kr.clone())
    assert e.value.status == rcc.RCC_ERR_SHAPE
    with pytest.raises(rcc.RccError) as e:      # ring of 4 frames needs 64 rows
        rcc.rope3d_apply_append_ring(tables, rcc.grid(2, 4, 4, 8), rcc.ring(1, 3),
                                     q, q, q, q.clone(), kr, kr.clone())
    assert e.value.status == rcc.RCC_ERR_RANGE
    assert bool((kr == 0).all())
