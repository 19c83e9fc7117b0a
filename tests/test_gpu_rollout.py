"""GPU parity over the full 5 s 480P rollout: 7 chunks x 4 denoising steps.

Each step re-seeds q, k, v, applies Causal-RoPE at global frames 3c..3c+2,
overwrites the chunk's cache rows, and attends to the growing cache (up to
32760 keys).  The oracle keeps its own cache from the same seeded inputs:
rotated k in fp64 stored at the cache's storage precision (bf16, nearest-even),
v as given.  Every step is checked: q' and the written K/V rows on every
token (bf16 RoPE rule; V bit-exact), and the attention output on one seeded
row of every 32-row wave of every head plus the first and last row of every
256-row query tile (max 2e-2 / mean 2e-3), after checking that the whole
NaN-poisoned output is finite.  After the last step of each chunk every
cache row written so far is compared, and the rows past it are still zero.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import (check_attn, check_bf16_rope, half_ulp_bf16, say, to_dev, to_host_f64,
                      torch, wave_rows)
from oracle import attention as A
from oracle import rope3d as R
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu


def _bf16(x64: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x64.astype(np.float32))).astype(np.float64)


def test_480p_rollout_every_step():
    t = torch()
    wl = synth.WORKLOADS["480p_rollout"]
    nh, D, L, hw = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw
    cap = wl.cache_tokens()
    assert cap == 32760
    r = wl.rope
    cfg = rcc.rope_cfg(r.d_t, r.d_h, r.d_w, r.max_t, r.max_h, r.max_w, r.theta)
    tables = rcc.rope3d_tables(cfg)
    otab = R.rope3d_tables(r.d_t, r.d_h, r.d_w, r.theta, r.max_t, r.max_h, r.max_w)
    kc = t.zeros((1, cap, nh, D), dtype=t.bfloat16, device="cuda")
    vc = t.zeros_like(kc)
    okc = np.zeros((1, cap, nh, D))
    ovc = np.zeros((1, cap, nh, D))
    scale = 1.0 / math.sqrt(D)
    for c, s in enumerate(wl.start_frames):
        for step in range(wl.steps):
            seeds = [synth.seed_for("480p_rollout", s, step, x) for x in ("q", "k", "v")]
            host = [synth.normal((1, L, nh, D), sd, "bf16") for sd in seeds]
            dq, dk, dv = (to_dev(x, "bf16") for x in host)
            qo = t.empty_like(dq)
            out = t.full_like(dq, float("nan"))
            kv = (s + wl.frames) * hw
            say("rollout chunk", c, "step", step, "kv", kv)
            rcc.rope3d_apply_append(tables, rcc.grid(wl.frames, wl.height, wl.width, s, 0),
                                    dq, dk, dv, qo, kc, vc)
            rcc.chunk_causal_attn(qo, kc, vc, out, s * hw, kv, L, scale)
            t.cuda.synchronize()

            # oracle: its own cache, from the same seeded inputs
            q, k, v = (synth.to_f64(x, "bf16") for x in host)
            pos = R.positions(wl.frames, wl.height, wl.width, s, 0, L)
            rows = pos[:, 3]
            okc[:, rows] = _bf16(R.rope3d_apply(k, otab, pos))
            ovc[:, rows] = v
            check_bf16_rope(to_host_f64(qo), R.rope3d_apply(q, otab, pos), f"c{c}s{step} q'")
            check_bf16_rope(to_host_f64(kc[:, s * hw:s * hw + L]), R.rope3d_apply(k, otab, pos),
                            f"c{c}s{step} k")
            assert np.array_equal(to_host_f64(vc[:, s * hw:s * hw + L]), v)
            # attention on a row of every wave, with the oracle's own (bf16-stored) q' and cache
            assert bool(t.isfinite(out).all()), f"c{c}s{step}: non-finite attention output"
            arow = wave_rows(L, 100 + 4 * c + step)
            qa = np.zeros((1, L, nh, D))
            qa[:, arow] = _bf16(R.rope3d_apply(q[:, arow], otab, pos[arow]))
            ref = A.chunk_causal_attention(qa, okc, ovc, s * hw, kv, L, scale, rows=arow)
            check_attn(to_host_f64(out[:, arow]), ref, f"c{c}s{step} attn")
        # every cache row written so far
        prefix = (s + wl.frames) * hw
        gk = to_host_f64(kc[:, :prefix])
        # GPU and oracle each round the rotated key to bf16 once: at most one ulp apart
        assert (np.abs(gk - okc[:, :prefix]) <= 2 * half_ulp_bf16(okc[:, :prefix]) + 1e-6).all()
        assert np.array_equal(to_host_f64(vc[:, :prefix]), ovc[:, :prefix])
        # rows past the prefix were never written
        if prefix < cap:
            assert bool((kc[:, prefix:] == 0).all()) and bool((vc[:, prefix:] == 0).all())
