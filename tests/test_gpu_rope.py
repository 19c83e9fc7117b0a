"""GPU parity: rope3d_tables, rope3d_positions and rope3d_apply_append vs the oracle.

Runs the HIP library through its C ABI (ctypes binding) on seeded inputs and
compares element by element with the fp64 oracle: positions bit-exact,
fp32 RoPE within 1e-5, bf16 RoPE within max(1e-2, half a bf16 ulp).
"""
import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import check_bf16_rope, say, to_dev, to_host_f64, torch
from oracle import rope3d as R
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu


def _cfg(wl, max_t=None):
    r = wl.rope
    return rcc.rope_cfg(r.d_t, r.d_h, r.d_w, max_t or r.max_t, r.max_h, r.max_w, r.theta)


def _oracle_tables(cfg):
    return R.rope3d_tables(cfg.d_t, cfg.d_h, cfg.d_w, cfg.theta, cfg.max_t, cfg.max_h, cfg.max_w)


def _flat_oracle_table(cfg):
    out = []
    for f in _oracle_tables(cfg):
        out.append(np.stack([f.real, f.imag], axis=-1).reshape(-1))
    return np.concatenate(out)


@pytest.mark.parametrize("dims,mx", [((44, 42, 42), (1024, 64, 128)), ((8, 8, 8), (16, 4, 4)),
                                     ((2, 4, 6), (7, 3, 5))])
def test_tables_match_oracle(dims, mx):
    cfg = rcc.rope_cfg(*dims, *mx)
    say("tables", dims, mx)
    t = rcc.rope3d_tables(cfg)
    torch().cuda.synchronize()
    got = t.buf.cpu().double().numpy()
    ref = _flat_oracle_table(cfg)
    assert got.shape == ref.shape
    # fp64 cos/sin rounded once to fp32: within one fp32 rounding of the oracle
    np.testing.assert_allclose(got, ref, rtol=0, atol=6e-8)
    exact = np.mean(got == ref.astype(np.float32).astype(np.float64))
    assert exact > 0.999


@pytest.mark.parametrize("F,H,W,s,off,n", [
    (2, 4, 4, 0, 0, 32), (2, 4, 4, 4, 0, 32), (3, 30, 52, 6, 0, 4680),
    (3, 30, 52, 9, 585, 585), (3, 30, 52, 9, 1170, 585), (3, 30, 52, 9, 4095, 585),
    (3, 45, 80, 18, 0, 10800), (5, 7, 3, 1000, 13, 77), (1, 1, 1, 0, 0, 1)])
def test_positions_bit_exact(F, H, W, s, off, n):
    say("positions", F, H, W, s, off, n)
    thw = rcc.rope3d_positions(rcc.grid(F, H, W, s, off), n)
    torch().cuda.synchronize()
    ref = R.positions(F, H, W, s, off, n)
    assert np.array_equal(thw.cpu().numpy().astype(np.int64), ref)


def _run_apply(wl, s, off, n, batch, in_dt, out_dt, seed, cap=None, poison=True):
    """Run rope3d_apply_append; returns host inputs, device outputs and cfg."""
    t = torch()
    cfg = _cfg(wl)
    tables = rcc.rope3d_tables(cfg)
    shape = (batch, n, wl.n_heads, wl.head_dim)
    q = synth.normal(shape, seed, in_dt)
    k = synth.normal(shape, seed + 1, in_dt)
    v = synth.normal(shape, seed + 2, in_dt)
    cap = cap or (s + wl.frames) * wl.hw + 7
    tdt = t.bfloat16 if out_dt == "bf16" else t.float32
    fill = float("nan") if poison else 0.0
    qo = t.full(shape, fill, dtype=tdt, device="cuda")
    kc = t.full((batch, cap, wl.n_heads, wl.head_dim), 3.0, dtype=tdt, device="cuda")
    vc = t.full((batch, cap, wl.n_heads, wl.head_dim), -3.0, dtype=tdt, device="cuda")
    dq, dk, dv = to_dev(q, in_dt), to_dev(k, in_dt), to_dev(v, in_dt)
    rcc.rope3d_apply_append(tables, rcc.grid(wl.frames, wl.height, wl.width, s, off),
                            dq, dk, dv, qo, kc, vc)
    t.cuda.synchronize()
    return cfg, (q, k, v), (qo, kc, vc), cap


def _oracle_apply(cfg, wl, s, off, host, in_dt, cap=None, tokens=None):
    """Oracle q', k', v and positions for the call's tokens (optionally a subset)."""
    n = host[0].shape[1]
    pos = R.positions(wl.frames, wl.height, wl.width, s, off, n)
    if tokens is not None:
        host = [x[:, tokens] for x in host]
        pos = pos[tokens]
    q, k, v = (synth.to_f64(x, in_dt) for x in host)
    tabs = _oracle_tables(cfg)
    return R.rope3d_apply(q, tabs, pos), R.rope3d_apply(k, tabs, pos), v, pos


@pytest.mark.parametrize("s", [0, 2, 4])
def test_apply_append_tiny_fp32(s):
    wl = synth.WORKLOADS["tiny"]
    say("apply tiny fp32 s=", s)
    cfg, host, (qo, kc, vc), cap = _run_apply(wl, s, 0, 32, 1, "f32", "f32", 11 + s)
    rq, rk, rv, pos = _oracle_apply(cfg, wl, s, 0, host, "f32", cap)
    gq, gk, gv = to_host_f64(qo), to_host_f64(kc), to_host_f64(vc)
    rows = pos[:, 3]
    assert np.abs(gq - rq).max() <= 1e-5
    assert np.abs(gk[:, rows] - rk).max() <= 1e-5
    assert np.array_equal(gv[:, rows], rv)                     # V copied bit-exactly
    other = np.setdiff1d(np.arange(cap), rows)
    assert np.all(gk[:, other] == 3.0) and np.all(gv[:, other] == -3.0)


@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"),
                                          ("f32", "f32")])
def test_apply_append_480p_chunk(in_dt, out_dt):
    """Full 4680-token 480P chunk at frames 6..8, all four dtype pairs."""
    wl = synth.WORKLOADS["480p_step"]
    s = 6
    say("apply 480p", in_dt, out_dt)
    cfg, host, (qo, kc, vc), cap = _run_apply(wl, s, 0, wl.chunk_tokens, 1, in_dt, out_dt, 22)
    rq, rk, rv, pos = _oracle_apply(cfg, wl, s, 0, host, in_dt, cap)
    rows = pos[:, 3]
    gq = to_host_f64(qo)
    gk = to_host_f64(kc)
    gv = to_host_f64(vc)
    if out_dt == "f32":
        assert np.abs(gq - rq).max() <= 1e-5
        assert np.abs(gk[:, rows] - rk).max() <= 1e-5
        if in_dt == "bf16":
            assert np.array_equal(gv[:, rows], rv)
    else:
        st = check_bf16_rope(gq, rq, "q'")
        check_bf16_rope(gk[:, rows], rk, "k cache")
        ref_v = synth.to_f64(synth.f32_to_bf16_bits(rv.astype(np.float32)), "bf16")
        assert np.array_equal(gv[:, rows], ref_v)
        say("bf16 rope stats", st)
    assert np.all(gk[:, :rows[0]] == 3.0) and np.all(gk[:, rows[-1] + 1:] == 3.0)
    assert np.all(gv[:, :rows[0]] == -3.0) and np.all(gv[:, rows[-1] + 1:] == -3.0)


@pytest.mark.parametrize("heads,D,dt", [(1, 64, "bf16"), (3, 128, "bf16"), (5, 48, "f32"),
                                         (7, 24, "f32")])
def test_apply_append_odd_heads_ragged_tokens(heads, D, dt):
    """Odd head counts, several head dims, a 51-token slice starting mid-frame
    (offset 6 of a 5 x 7 frame, crossing the frame boundary) and batch 2: the
    flat thread -> (token, 16-byte chunk) map must cover every element once
    with a ragged last workgroup."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name="odd", n_heads=heads, head_dim=D,
                             frames=2, height=5, width=7)
    s, off, n = 3, 6, 51
    say("apply odd heads", heads, D, dt)
    cfg, host, (qo, kc, vc), cap = _run_apply(wl, s, off, n, 2, dt, dt, 70 + heads)
    rq, rk, rv, pos = _oracle_apply(cfg, wl, s, off, host, dt, cap)
    rows = pos[:, 3]
    gq, gk, gv = to_host_f64(qo), to_host_f64(kc), to_host_f64(vc)
    if dt == "f32":
        assert np.abs(gq - rq).max() <= 1e-5
        assert np.abs(gk[:, rows] - rk).max() <= 1e-5
    else:
        check_bf16_rope(gq, rq, "q'")
        check_bf16_rope(gk[:, rows], rk, "k cache")
    assert np.array_equal(gv[:, rows], rv)
    other = np.setdiff1d(np.arange(cap), rows)
    assert np.all(gk[:, other] == 3.0) and np.all(gv[:, other] == -3.0)


def test_sp_shards_bit_equal_unsharded_and_match_oracle():
    """Each of 8 ranks' 585-token slice (Delta = 585 r) equals the unsharded run."""
    t = torch()
    wl = synth.WORKLOADS["480p_sp_shard"]
    s, L, P = 9, wl.chunk_tokens, synth.SP_DEGREE
    cfg = _cfg(wl)
    tables = rcc.rope3d_tables(cfg)
    shape = (1, L, wl.n_heads, wl.head_dim)
    host = [synth.normal(shape, 40 + i, "bf16") for i in range(3)]
    dq, dk, dv = (to_dev(x, "bf16") for x in host)
    cap = (s + wl.frames) * wl.hw
    g_full = rcc.grid(wl.frames, wl.height, wl.width, s, 0)
    outs = []
    for _ in range(2):  # full run, then the 8 shards
        outs.append([t.full(shape, float("nan"), dtype=t.bfloat16, device="cuda"),
                     t.zeros((1, cap, wl.n_heads, wl.head_dim), dtype=t.bfloat16, device="cuda"),
                     t.zeros((1, cap, wl.n_heads, wl.head_dim), dtype=t.bfloat16, device="cuda")])
    say("sp full")
    rcc.rope3d_apply_append(tables, g_full, dq, dk, dv, *outs[0])
    n = L // P
    for r in range(P):
        say("sp shard", r)
        sl = slice(r * n, (r + 1) * n)
        qo_r = t.empty((1, n, wl.n_heads, wl.head_dim), dtype=t.bfloat16, device="cuda")
        rcc.rope3d_apply_append(tables, rcc.grid(wl.frames, wl.height, wl.width, s, r * n),
                                dq[:, sl].contiguous(), dk[:, sl].contiguous(),
                                dv[:, sl].contiguous(), qo_r, outs[1][1], outs[1][2])
        outs[1][0][:, sl] = qo_r
    t.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert t.equal(a.view(t.int16), b.view(t.int16))
    # and the shard of rank 2 (straddles a frame boundary) against the oracle
    rq, rk, _, pos = _oracle_apply(cfg, wl, s, 2 * n, [x[:, 2 * n:3 * n] for x in host], "bf16", cap)
    check_bf16_rope(to_host_f64(outs[1][0][:, 2 * n:3 * n]), rq, "rank2 q'")
    check_bf16_rope(to_host_f64(outs[1][1])[:, pos[:, 3]], rk, "rank2 k")


def test_sp_shard_batched_64():
    """Rank-2 shard with 64 chunks batched (the bandwidth configuration): every
    token of every batch entry, and every other cache row keeps its canary."""
    wl = synth.WORKLOADS["480p_sp_shard"]
    s, n, r = 9, 585, 2
    say("sp shard batch 64")
    cfg, host, (qo, kc, vc), cap = _run_apply(wl, s, r * n, n, 64, "bf16", "bf16", 40,
                                              cap=(s + 3) * wl.hw)
    rq, rk, rv, pos = _oracle_apply(cfg, wl, s, r * n, host, "bf16", cap)
    check_bf16_rope(to_host_f64(qo), rq, "b64 q'")
    gk, gv = to_host_f64(kc), to_host_f64(vc)
    check_bf16_rope(gk[:, pos[:, 3]], rk, "b64 k")
    assert np.array_equal(gv[:, pos[:, 3]], rv)
    other = np.setdiff1d(np.arange(cap), pos[:, 3])
    assert np.all(gk[:, other] == 3.0) and np.all(gv[:, other] == -3.0)


def test_apply_720p_every_token():
    """Wan-14B 720P chunk (40 heads, 10800 tokens) at frames 18..20: every token,
    and every cache row outside the chunk keeps its canary."""
    wl = synth.WORKLOADS["720p_step"]
    s = 18
    say("apply 720p")
    cfg, host, (qo, kc, vc), cap = _run_apply(wl, s, 0, wl.chunk_tokens, 1, "bf16", "bf16", 60)
    rq, rk, rv, pos = _oracle_apply(cfg, wl, s, 0, host, "bf16", cap)
    check_bf16_rope(to_host_f64(qo), rq, "720p q'")
    gk, gv = to_host_f64(kc), to_host_f64(vc)
    check_bf16_rope(gk[:, pos[:, 3]], rk, "720p k")
    assert np.array_equal(gv[:, pos[:, 3]], rv)
    other = np.setdiff1d(np.arange(cap), pos[:, 3])
    assert np.all(gk[:, other] == 3.0) and np.all(gv[:, other] == -3.0)


def test_in_place_q_and_determinism():
    t = torch()
    wl = synth.WORKLOADS["480p_step"]
    cfg = _cfg(wl)
    tables = rcc.rope3d_tables(cfg)
    shape = (1, 1000, wl.n_heads, wl.head_dim)
    host = [synth.normal(shape, 70 + i, "bf16") for i in range(3)]
    g = rcc.grid(3, 30, 52, 3, 1234)
    cap = 6 * wl.hw
    res = []
    for inplace in (False, False, True):
        dq, dk, dv = (to_dev(x, "bf16") for x in host)
        qo = dq if inplace else t.empty_like(dq)
        kc = t.zeros((1, cap, wl.n_heads, wl.head_dim), dtype=t.bfloat16, device="cuda")
        vc = t.zeros_like(kc)
        say("inplace", inplace)
        rcc.rope3d_apply_append(tables, g, dq, dk, dv, qo, kc, vc)
        t.cuda.synchronize()
        res.append((qo.view(t.int16).cpu(), kc.view(t.int16).cpu()))
    for a in res[1:]:
        assert t.equal(a[0], res[0][0]) and t.equal(a[1], res[0][1])


def test_zero_tokens_is_a_no_op():
    t = torch()
    wl = synth.WORKLOADS["tiny"]
    cfg = _cfg(wl)
    tables = rcc.rope3d_tables(cfg)
    e = t.empty((1, 0, 2, 24), device="cuda")
    kc = t.full((1, 96, 2, 24), 5.0, device="cuda")
    rcc.rope3d_apply_append(tables, rcc.grid(2, 4, 4, 2, 32), e, e, e, e, kc, kc.clone())
    t.cuda.synchronize()
    assert bool((kc == 5.0).all())


def test_errors_reported_without_launch():
    t = torch()
    wl = synth.WORKLOADS["tiny"]
    cfg = _cfg(wl)
    tables = rcc.rope3d_tables(cfg)
    x = t.zeros((1, 32, 2, 24), device="cuda")
    kc = t.full((1, 64, 2, 24), 9.0, device="cuda")
    with pytest.raises(rcc.RccError) as e:   # s + F > max_t
        rcc.rope3d_apply_append(tables, rcc.grid(2, 4, 4, 15, 0), x, x, x, x.clone(), kc, kc)
    assert e.value.status == rcc.RCC_ERR_RANGE
    with pytest.raises(rcc.RccError) as e:   # cache too small for rows 64..95
        rcc.rope3d_apply_append(tables, rcc.grid(2, 4, 4, 4, 0), x, x, x, x.clone(), kc, kc)
    assert e.value.status == rcc.RCC_ERR_RANGE
    with pytest.raises(rcc.RccError) as e:   # Delta + n beyond the chunk
        rcc.rope3d_apply_append(tables, rcc.grid(2, 4, 4, 0, 1), x, x, x, x.clone(), kc, kc)
    assert e.value.status == rcc.RCC_ERR_RANGE
    t.cuda.synchronize()
    assert bool((kc == 9.0).all())
