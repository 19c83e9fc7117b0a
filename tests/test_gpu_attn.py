"""GPU parity: chunk_causal_attn vs the fp64 oracle.

Element-by-element comparison on seeded inputs: max abs <= 2e-2, mean abs
<= 2e-3 (bf16 operands, fp32 accumulation) plus a relative L2 bound.  Small
cases are compared in full; the full-size 480P/720P steps on sampled query
rows (every head, first/last rows, tile edges).  The oracle sees exactly the
values the kernel's matrix cores see: for fp32 inputs, their bf16 rounding.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import Bf16Rows, check_attn, say, to_dev, to_host_f64, torch
from oracle import attention as A
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu


def _bf16_round(x32: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x32)).astype(np.float64)


def _attn_case(b, lq, nh, d, cap, q_pos, kv, C, in_dt, out_dt, seed, q_scale=1.0,
               rows=None, label=""):
    t = torch()
    q = synth.normal((b, lq, nh, d), seed, in_dt, scale=q_scale)
    k = synth.normal((b, cap, nh, d), seed + 1, in_dt)
    v = synth.normal((b, cap, nh, d), seed + 2, in_dt)
    out = t.full((b, lq, nh, d), float("nan"),
                 dtype=t.bfloat16 if out_dt == "bf16" else t.float32, device="cuda")
    say("attn", label, b, lq, nh, d, cap, q_pos, kv, C, in_dt, out_dt)
    rcc.chunk_causal_attn(to_dev(q, in_dt), to_dev(k, in_dt), to_dev(v, in_dt), out,
                          q_pos, kv, C, 1.0 / math.sqrt(d))
    t.cuda.synchronize()
    if in_dt == "f32":
        qf, kf, vf = _bf16_round(q), _bf16_round(k), _bf16_round(v)
    else:
        qf, kf, vf = synth.to_f64(q, "bf16"), Bf16Rows(k), Bf16Rows(v)
    ref = A.chunk_causal_attention(qf, kf, vf, q_pos, kv, C, 1.0 / math.sqrt(d), rows=rows)
    got = to_host_f64(out)
    if rows is not None:
        got = got[:, rows]
    return got, ref, (q, k, v)


@pytest.mark.parametrize("c", [0, 1, 2])
def test_tiny_chunk_by_chunk_fp32(c):
    """Tiny workload: chunk c (32 tokens, frames 2c..2c+1) over cache chunks 0..c."""
    wl = synth.WORKLOADS["tiny"]
    C = wl.chunk_tokens
    got, ref, _ = _attn_case(1, C, 2, 24, 3 * C, c * C, (c + 1) * C, C, "f32", "f32", 101 + c,
                             label=f"tiny c{c}")
    check_attn(got, ref, "tiny")


def test_tiny_one_shot_block_causal():
    """All 96 tiny tokens in one call with the block-causal mask (chunk = 32)."""
    got, ref, (q, k, v) = _attn_case(1, 96, 2, 24, 96, 0, 96, 32, "f32", "f32", 111,
                                     label="tiny one-shot")
    check_attn(got, ref, "tiny one-shot")
    # against the unrounded fp32 inputs too (reported: operands are bf16)
    ref32 = A.chunk_causal_attention(q, k, v, 0, 96, 32, 1 / math.sqrt(24))
    err = np.abs(got - ref32)
    assert err.max() < 5e-2


@pytest.mark.parametrize("b,lq,nh,d,cap,q_pos,kv,C,in_dt,out_dt", [
    (1, 300, 2, 128, 800, 400, 700, 100, "bf16", "bf16"),   # ragged, mid-chunk q_pos
    (2, 257, 3, 128, 600, 343, 600, 257, "bf16", "f32"),    # partial tiles both ways
    (1, 129, 1, 64, 200, 0, 129, 7, "bf16", "bf16"),        # tiny chunks, many masked tiles
    (1, 64, 2, 24, 200, 136, 200, 64, "f32", "f32"),        # D=24, fp32 in
    (1, 100, 2, 40, 150, 50, 150, 1000, "bf16", "bf16"),    # one chunk covers everything
    (1, 1, 4, 128, 70, 69, 70, 70, "bf16", "bf16"),         # single query row
    (1, 200, 2, 128, 1000, 800, 1000, 200, "f32", "bf16"),  # AR step, fp32 in
])
def test_ragged_and_masked_shapes(b, lq, nh, d, cap, q_pos, kv, C, in_dt, out_dt):
    got, ref, _ = _attn_case(b, lq, nh, d, cap, q_pos, kv, C, in_dt, out_dt, 300 + lq,
                             label="shape")
    check_attn(got, ref, f"{(b, lq, nh, d, q_pos, kv, C)}")


def test_cache_over_4gib_per_batch_entry():
    """A bf16 head_dim-128 cache of 2^24 + 32 rows per batch entry (4.3 GB for
    K alone) is past the fast kernel's 32-bit in-entry offsets, so the call
    takes the generic kernel; batch entry 1 then starts 4.3 GB into the
    cache.  Only the first kv rows of each entry are written and read."""
    t = torch()
    b, lq, nh, d, cap, q_pos, kv, C = 2, 100, 1, 128, (1 << 24) + 32, 200, 300, 100
    q = synth.normal((b, lq, nh, d), 501, "bf16")
    k = synth.normal((b, kv, nh, d), 502, "bf16")
    v = synth.normal((b, kv, nh, d), 503, "bf16")
    say("attn cache > 4 GiB per entry", cap)
    kc = t.empty((b, cap, nh, d), dtype=t.bfloat16, device="cuda")
    vc = t.empty((b, cap, nh, d), dtype=t.bfloat16, device="cuda")
    kc[:, :kv] = to_dev(k, "bf16")
    vc[:, :kv] = to_dev(v, "bf16")
    out = t.full((b, lq, nh, d), float("nan"), dtype=t.bfloat16, device="cuda")
    rcc.chunk_causal_attn(to_dev(q, "bf16"), kc, vc, out, q_pos, kv, C, 1.0 / math.sqrt(d))
    t.cuda.synchronize()
    ref = A.chunk_causal_attention(synth.to_f64(q, "bf16"), synth.to_f64(k, "bf16"),
                                   synth.to_f64(v, "bf16"), q_pos, kv, C, 1.0 / math.sqrt(d))
    check_attn(to_host_f64(out), ref, "cache > 4 GiB")
    del kc, vc


def _sample_rows(lq, n, seed):
    r = np.random.default_rng(seed).choice(lq, size=min(n, lq), replace=False)
    edges = [0, 1, 31, 32, 127, 128, lq - 129, lq - 128, lq - 2, lq - 1]
    return np.unique(np.concatenate([r, [e for e in edges if 0 <= e < lq]]))


def test_480p_step_full_size_sampled_rows():
    """Wan-1.3B 480P step: 4680 queries at frames 6..8 over 14040 cached keys."""
    wl = synth.WORKLOADS["480p_step"]
    lq = wl.chunk_tokens
    kv = (6 + 3) * wl.hw
    rows = _sample_rows(lq, 160, 1)
    got, ref, _ = _attn_case(1, lq, wl.n_heads, wl.head_dim, kv, 6 * wl.hw, kv, lq,
                             "bf16", "bf16", 22, rows=rows, label="480p")
    say("480p", check_attn(got, ref, "480p step"))


def test_720p_step_full_size_sampled_rows():
    """Wan-14B 720P step: 40 heads, 10800 queries over 75600 cached keys."""
    wl = synth.WORKLOADS["720p_step"]
    lq = wl.chunk_tokens
    kv = (18 + 3) * wl.hw
    rows = _sample_rows(lq, 48, 2)
    got, ref, _ = _attn_case(1, lq, wl.n_heads, wl.head_dim, kv, 18 * wl.hw, kv, lq,
                             "bf16", "bf16", 60, rows=rows, label="720p")
    say("720p", check_attn(got, ref, "720p step"))


def test_stress_peaked_softmax():
    """Q scaled x8: sharply peaked rows exercise the running-max rescale."""
    got, ref, _ = _attn_case(1, 256, 2, 128, 2048, 1024, 2048, 1024, "bf16", "f32", 500,
                             q_scale=8.0, label="peaked")
    check_attn(got, ref, "peaked", max_abs=5e-2, mean_abs=5e-3, rel_l2=2e-2)


def test_stress_dominant_key_late():
    """One key far above the rest, placed in the last tile: output ~ its value row."""
    t = torch()
    lq, cap, nh, d = 128, 1000, 1, 128
    q = synth.normal((1, lq, nh, d), 600, "bf16")
    k = synth.normal((1, cap, nh, d), 601, "bf16")
    v = synth.normal((1, cap, nh, d), 602, "bf16")
    qf = synth.to_f64(q, "bf16")
    # key 990 = 8 * sqrt(d) * unit mean query direction -> dominates every row's logits
    kd = 8.0 * qf[0].mean(axis=0, keepdims=True) / np.linalg.norm(qf[0].mean(axis=0)) * math.sqrt(d)
    k[0, 990] = synth.f32_to_bf16_bits(kd.astype(np.float32))[0]
    out = t.empty((1, lq, nh, d), dtype=t.float32, device="cuda")
    say("dominant key")
    rcc.chunk_causal_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), out,
                          872, 1000, 1000, 1 / math.sqrt(d))
    t.cuda.synchronize()
    ref = A.chunk_causal_attention(qf, synth.to_f64(k, "bf16"), synth.to_f64(v, "bf16"),
                                   872, 1000, 1000, 1 / math.sqrt(d))
    check_attn(to_host_f64(out), ref, "dominant key")


def test_determinism_and_no_nan():
    t = torch()
    q = to_dev(synth.normal((1, 700, 4, 128), 700, "bf16"), "bf16")
    k = to_dev(synth.normal((1, 3000, 4, 128), 701, "bf16"), "bf16")
    v = to_dev(synth.normal((1, 3000, 4, 128), 702, "bf16"), "bf16")
    outs = []
    for _ in range(2):
        o = t.full((1, 700, 4, 128), float("nan"), dtype=t.bfloat16, device="cuda")
        say("determinism")
        rcc.chunk_causal_attn(q, k, v, o, 2300, 3000, 700, 0.088)
        outs.append(o)
    t.cuda.synchronize()
    assert not bool(t.isnan(outs[0]).any())
    assert t.equal(outs[0].view(t.int16), outs[1].view(t.int16))


def test_errors_reported_without_launch():
    t = torch()
    q = t.zeros((1, 10, 2, 128), dtype=t.bfloat16, device="cuda")
    kc = t.zeros((1, 20, 2, 128), dtype=t.bfloat16, device="cuda")
    out = t.full((1, 10, 2, 128), 7.0, dtype=t.bfloat16, device="cuda")
    cases = [((15, 20, 5), rcc.RCC_ERR_RANGE),   # q_pos + Lq > kv
             ((0, 21, 5), rcc.RCC_ERR_RANGE),    # kv > cache
             ((0, 10, 0), rcc.RCC_ERR_SHAPE)]    # chunk_tokens 0
    for (q_pos, kv, C), st in cases:
        with pytest.raises(rcc.RccError) as e:
            rcc.chunk_causal_attn(q, kc, kc, out, q_pos, kv, C, 0.1)
        assert e.value.status == st
    t.cuda.synchronize()
    assert bool((out == 7.0).all())
