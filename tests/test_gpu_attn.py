"""GPU parity: chunk_causal_attn vs the fp64 oracle.

Element-by-element comparison on seeded inputs: max abs <= 2e-2, mean abs
<= 2e-3 (bf16 operands, fp32 accumulation) plus a relative L2 bound.  These
cases are compared in full; the full-size 480P and 720P steps are in
test_gpu_step.py.  The oracle sees exactly the values the kernel's matrix
cores see: for fp32 inputs, their bf16 rounding.
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


@pytest.mark.parametrize("kv", [1, 20, 32, 33, 64, 65, 96, 100, 128, 129, 160, 192, 200, 224,
                                256, 257, 288])
@pytest.mark.parametrize("C", [0, 16])
def test_fast_path_every_tile_count(kv, C):
    """bf16, head_dim 128 (the fast kernel): key ranges of 1 to 9 tiles of
    32, so the first (checked) tile, the loop over groups of four tiles and
    every remainder of the unchecked sweep are hit.  The queries are the
    last min(kv, 40) keys' positions; C = 0 stands for one chunk over
    everything, 16 makes the visibility block-causal inside the queries."""
    lq = min(kv, 40)
    chunk = lq if C == 0 else C
    got, ref, _ = _attn_case(1, lq, 3, 128, kv, kv - lq, kv, chunk, "bf16", "bf16",
                             700 + kv + C, label="tile count")
    check_attn(got, ref, f"tile count kv={kv} C={chunk}")


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


def _directed_case(seed, q_shift, key_shift):
    """q rows N(0,1) + q_shift * u and keys N(0,1) + key_shift[j] * u for a
    seeded unit vector u: logits (q.k)/sqrt(d) follow key_shift along the keys."""
    lq, kv, d = 128, 2048, 128
    g = np.random.Generator(np.random.PCG64(seed))
    u = g.standard_normal(d)
    u /= np.linalg.norm(u)
    q = synth.bf16_bits_to_f32(synth.normal((1, lq, 1, d), seed + 1, "bf16")) + q_shift * u
    k = synth.bf16_bits_to_f32(synth.normal((1, kv, 1, d), seed + 2, "bf16"))
    k += np.asarray(key_shift, dtype=np.float32)[None, :, None, None] * u
    v = synth.normal((1, kv, 1, d), seed + 3, "bf16")
    qb = synth.f32_to_bf16_bits(q.astype(np.float32))
    kb = synth.f32_to_bf16_bits(k.astype(np.float32))
    t = torch()
    out = t.full((1, lq, 1, d), float("nan"), dtype=t.float32, device="cuda")
    say("directed scores", seed, q_shift)
    rcc.chunk_causal_attn(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(v, "bf16"), out,
                          kv - lq, kv, kv, 1 / math.sqrt(d))
    t.cuda.synchronize()
    ref = A.chunk_causal_attention(synth.to_f64(qb, "bf16"), synth.to_f64(kb, "bf16"),
                                   synth.to_f64(v, "bf16"), kv - lq, kv, kv, 1 / math.sqrt(d))
    return to_host_f64(out), ref


def test_stress_scores_rise_then_jump_past_fp32_range():
    """Logits that climb tile by tile (the softmax reference must move several
    times), then two keys whose base-2 scores sit ~300 above the reference, so
    their exponentials overflow fp32 before the reference catches up, then
    ordinary keys again.  The output mixes the two top keys' values."""
    shift = np.zeros(2048)
    shift[1000:1400] = np.arange(400) * 0.2          # a ramp over 12 key tiles
    shift[1500], shift[1700] = 400.0, 400.5          # far above everything else
    got, ref = _directed_case(910, 6.0, shift)
    assert np.isfinite(got).all()
    say("rise/jump", check_attn(got, ref, "rise then jump"))


@pytest.mark.parametrize("jump", [40.0, 66.0, 120.0])
def test_stress_late_scores_around_the_certificate_bound(jump):
    """Three late keys whose base-2 scores sit about `jump` above the first
    tile's (the per-query spread of the construction is some 15%).  The
    kernel's reference comes from the first tile and later tiles are not
    tested one by one: a row sum up to 2^64 is accepted as is, a larger one
    sends the workgroup through a second, checked sweep.  40 stays below the
    bound, 120 passes it in every row (some sums overflow to inf), 66 lands
    on both sides; every row must match the oracle."""
    shift = np.zeros(2048)
    s = jump * math.sqrt(128) / (math.log2(math.e) * 6.0)
    shift[1800], shift[1801], shift[2000] = s, s - 0.5, s - 1.0
    got, ref = _directed_case(930 + int(jump), 6.0, shift)
    assert np.isfinite(got).all()
    say("late jump", jump, check_attn(got, ref, f"late jump {jump}"))


def test_stress_unnormalised_output_past_fp32_range():
    """Late keys 56-62 (base 2) above the first tile's scores, whose value
    rows are 2^74: the row sums stay below 2^64 but the unnormalised O^T
    (probabilities ~2^60 times 2^74) overflows fp32 in the unchecked sweep.
    The output certificate must send the workgroup through the checked
    sweep, which moves the reference and keeps O^T finite.  Outputs are
    ~2^74, so the comparison is relative."""
    t = torch()
    lq, kv, d = 128, 2048, 128
    g = np.random.Generator(np.random.PCG64(940))
    u = g.standard_normal(d)
    u /= np.linalg.norm(u)
    sh = 60.0 * math.sqrt(d) / (math.log2(math.e) * 6.0)
    shift = np.zeros(kv)
    big = [1800, 1801, 2000]
    shift[big] = [sh, sh - 0.5, sh - 1.0]
    # small query noise, so every row's jump is 60 to within a few units
    q = 0.1 * synth.bf16_bits_to_f32(synth.normal((1, lq, 1, d), 941, "bf16")) + 6.0 * u
    k = synth.bf16_bits_to_f32(synth.normal((1, kv, 1, d), 942, "bf16"))
    k += shift[None, :, None, None] * u
    v = synth.bf16_bits_to_f32(synth.normal((1, kv, 1, d), 943, "bf16"))
    v[0, big] *= 2.0 ** 74
    qb = synth.f32_to_bf16_bits(q.astype(np.float32))
    kb = synth.f32_to_bf16_bits(k.astype(np.float32))
    vb = synth.f32_to_bf16_bits(v.astype(np.float32))
    out = t.full((1, lq, 1, d), float("nan"), dtype=t.float32, device="cuda")
    say("output overflow")
    rcc.chunk_causal_attn(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), out,
                          kv - lq, kv, kv, 1 / math.sqrt(d))
    t.cuda.synchronize()
    got = to_host_f64(out)
    ref = A.chunk_causal_attention(synth.to_f64(qb, "bf16"), synth.to_f64(kb, "bf16"),
                                   synth.to_f64(vb, "bf16"), kv - lq, kv, kv, 1 / math.sqrt(d))
    assert np.isfinite(got).all()
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    rel = np.abs(got - ref) / scale
    say("output overflow rel err", float(rel.max()))
    assert rel.max() < 2e-2


def test_stress_all_scores_far_below_zero():
    """Every logit near -210 (base-2 scores near -300): each probability
    underflows to zero against the initial reference, so the reference must
    be taken from the first tile's max."""
    got, ref = _directed_case(920, -6.0, np.full(2048, 400.0))
    assert np.isfinite(got).all()
    say("all negative", check_attn(got, ref, "all far below zero"))


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
