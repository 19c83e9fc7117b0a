"""GPU parity: qkv_rope_append (fused QKV projection + Causal-RoPE + cache write)
vs the oracle.

Seeded bf16 inputs: x ~ N(0, 1) and w_qkv ~ N(0, 1/model_dim) (so outputs are
~N(0, 1), as in a trained projection), optional fp32 bias.  The oracle
projects in fp64 from the same bf16 values, rotates and writes its own cache.
q_out and the written cache rows must meet the bf16 RoPE rule (max(1e-2,
half a bf16 ulp)) on every token, including the full 480P chunk and the
64-chunk SP-rank batch; every cache row outside the slice must keep its
sentinel.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import check_bf16_rope, say, to_dev, to_host_f64, torch
from oracle import qkv as Q
from oracle import rope3d as R
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _run(B, n, nh, dims, K, F, H, W, s, off, mx, bias, seed, sample=None):
    t = torch()
    D = sum(dims)
    cfg = rcc.rope_cfg(*dims, *mx)
    tables = rcc.rope3d_tables(cfg)
    otab = R.rope3d_tables(*dims, cfg.theta, *mx)
    xb = synth.normal((B, n, K), seed, "bf16")
    wb = synth.normal((3 * nh * D, K), seed + 1, "bf16", scale=1.0 / math.sqrt(K))
    bias_np = synth.normal((3 * nh * D,), seed + 2, "f32", scale=0.5) if bias else None
    cap = (s + F) * H * W + 5
    say("qkv", B, n, nh, dims, K, (F, H, W, s, off), "bias" if bias else "")
    x, w = to_dev(xb, "bf16"), to_dev(wb, "bf16")
    bdev = to_dev(bias_np, "f32") if bias else None
    qo = t.full((B, n, nh, D), float("nan"), dtype=t.bfloat16, device="cuda")
    kc = t.full((B, cap, nh, D), SENTINEL, dtype=t.bfloat16, device="cuda")
    vc = t.full_like(kc, SENTINEL)
    rcc.qkv_rope_append(tables, rcc.grid(F, H, W, s, off), x, w, bdev, qo, kc, vc)
    t.cuda.synchronize()

    tok = np.arange(n) if sample is None else sample
    xo = synth.to_f64(xb, "bf16")[:, tok]
    wo = synth.to_f64(wb, "bf16")
    q, k, v = Q.qkv_project(xo, wo, None if bias_np is None else bias_np.astype(np.float64), nh, D)
    pos = R.positions(F, H, W, s, off, n)[tok]
    rq = R.rope3d_apply(q, otab, pos)
    rk = R.rope3d_apply(k, otab, pos)
    check_bf16_rope(to_host_f64(qo[:, tok]), rq, "q_out")
    check_bf16_rope(to_host_f64(kc[:, pos[:, 3]]), rk, "k_cache")
    check_bf16_rope(to_host_f64(vc[:, pos[:, 3]]), v, "v_cache")
    # every row outside the slice keeps the sentinel
    rows = R.positions(F, H, W, s, off, n)[:, 3]
    untouched = t.from_numpy(np.setdiff1d(np.arange(cap), rows)).cuda()
    if untouched.numel():
        assert bool((kc[:, untouched] == SENTINEL).all())
        assert bool((vc[:, untouched] == SENTINEL).all())
    return qo, kc, vc


@pytest.mark.parametrize("B,n,nh,dims,K,F,H,W,s,off,bias", [
    (1, 40, 2, (12, 10, 10), 64, 2, 4, 5, 2, 0, False),        # ragged token and feature tiles
    (3, 100, 2, (12, 10, 10), 64, 2, 10, 10, 4, 37, True),     # tiles span batch entries
    (2, 300, 3, (44, 42, 42), 128, 3, 10, 12, 6, 50, True),    # head_dim 128, several tiles
    (1, 1, 1, (12, 10, 10), 32, 1, 1, 1, 0, 0, False),          # one token, one K step
    (1, 257, 4, (16, 8, 8), 160, 2, 16, 16, 0, 0, False),       # K not a multiple of 64
    (1, 200, 3, (40, 44, 44), 128, 2, 10, 10, 3, 0, True),      # head_dim 128, other bands
])
def test_small_shapes_every_token(B, n, nh, dims, K, F, H, W, s, off, bias):
    _run(B, n, nh, dims, K, F, H, W, s, off, (16, 16, 16), bias, seed=11)


@pytest.mark.parametrize("n,nh,F,H,W", [
    (3700, 12, 3, 30, 52),   # 18 feature tiles: 384-token tiles fill the CUs in one round
    (9000, 5, 6, 30, 52),    # 1920 features: a ragged last feature tile
])
def test_384_token_tiles_every_token(n, nh, F, H, W):
    """Shapes the host runs with 384-token tiles, compared on every token."""
    _run(1, n, nh, (44, 42, 42), nh * 128, F, H, W, 2, 0, (16, 32, 64), True, 61)


def test_480p_chunk_every_token():
    wl = synth.WORKLOADS["480p_step"]
    r = wl.rope
    _run(1, wl.chunk_tokens, wl.n_heads, (r.d_t, r.d_h, r.d_w), wl.n_heads * wl.head_dim,
         wl.frames, wl.height, wl.width, wl.start_frames[0], 0, (r.max_t, r.max_h, r.max_w),
         True, 71)


def test_sp_shard_batch64_every_token():
    wl = synth.WORKLOADS["480p_sp_shard"]
    r = wl.rope
    n = wl.chunk_tokens // synth.SP_DEGREE
    _run(64, n, wl.n_heads, (r.d_t, r.d_h, r.d_w), wl.n_heads * wl.head_dim, wl.frames,
         wl.height, wl.width, wl.start_frames[0], 2 * n, (r.max_t, r.max_h, r.max_w), False, 81)


def test_deterministic():
    a = _run(2, 300, 3, (44, 42, 42), 128, 3, 10, 12, 6, 50, (16, 16, 16), True, 91)
    b = _run(2, 300, 3, (44, 42, 42), 128, 3, 10, 12, 6, 50, (16, 16, 16), True, 91)
    for x, y in zip(a, b):
        assert bool((x.view(torch().int16) == y.view(torch().int16)).all())


def test_zero_tokens_is_a_no_op():
    t = torch()
    cfg = rcc.rope_cfg(12, 10, 10, 16, 16, 16)
    tables = rcc.rope3d_tables(cfg)
    x = t.zeros((1, 0, 64), dtype=t.bfloat16, device="cuda")
    w = t.zeros((3 * 2 * 32, 64), dtype=t.bfloat16, device="cuda")
    qo = t.zeros((1, 0, 2, 32), dtype=t.bfloat16, device="cuda")
    kc = t.full((1, 64, 2, 32), SENTINEL, dtype=t.bfloat16, device="cuda")
    vc = t.full_like(kc, SENTINEL)
    rcc.qkv_rope_append(tables, rcc.grid(2, 4, 4, 0, 0), x, w, None, qo, kc, vc)
    t.cuda.synchronize()
    assert bool((kc == SENTINEL).all()) and bool((vc == SENTINEL).all())


def test_errors_reported_without_launch():
    t = torch()
    cfg = rcc.rope_cfg(12, 10, 10, 16, 16, 16)
    tables = rcc.rope3d_tables(cfg)
    x = t.zeros((1, 8, 48), dtype=t.bfloat16, device="cuda")        # model_dim 48: not 32k
    w = t.zeros((3 * 2 * 32, 48), dtype=t.bfloat16, device="cuda")
    qo = t.zeros((1, 8, 2, 32), dtype=t.bfloat16, device="cuda")
    kc = t.zeros((1, 64, 2, 32), dtype=t.bfloat16, device="cuda")
    with pytest.raises(rcc.RccError) as e:
        rcc.qkv_rope_append(tables, rcc.grid(2, 4, 4, 0, 0), x, w, None, qo, kc, kc.clone())
    assert e.value.status == rcc.RCC_ERR_SHAPE
    with pytest.raises(TypeError):
        rcc.qkv_rope_append(tables, rcc.grid(2, 4, 4, 0, 0), x.float(), w, None, qo, kc,
                            kc.clone())
