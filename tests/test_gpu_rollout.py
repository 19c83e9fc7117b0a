"""GPU parity over the full 5 s 480P rollout: 7 chunks x 4 denoising steps.

Each step re-seeds q, k, v, applies Causal-RoPE at global frames 3c..3c+2,
overwrites the chunk's cache rows, and attends to the growing cache (up to
32760 keys).  The oracle keeps its own cache from the same seeded inputs:
rotated k in fp64 stored at the cache's storage precision (bf16, nearest-even),
v as given.  Every step is checked: q' and the cache rows on sampled tokens
(bf16 RoPE rule), the attention output on sampled rows of every head
(max 2e-2 / mean 2e-3).  After the last step of each chunk the whole cache
prefix is compared on sampled rows.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import check_attn, check_bf16_rope, say, to_dev, to_host_f64, torch
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
    rng = np.random.default_rng(3)
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
            tok = np.unique(np.concatenate([rng.choice(L, 40, replace=False), [0, L - 1]]))
            rq = R.rope3d_apply(q[:, tok], otab, pos[tok])
            check_bf16_rope(to_host_f64(qo[:, tok]), rq, f"c{c}s{step} q'")
            check_bf16_rope(to_host_f64(kc[:, rows[tok]]),
                            R.rope3d_apply(k[:, tok], otab, pos[tok]), f"c{c}s{step} k")
            # attention on sampled rows, with the oracle's own (bf16-stored) q' and cache
            qa = np.zeros((1, L, nh, D))
            arow = np.unique(np.concatenate([rng.choice(L, 24, replace=False), [0, L - 1]]))
            qa[:, arow] = _bf16(R.rope3d_apply(q[:, arow], otab, pos[arow]))
            ref = A.chunk_causal_attention(qa, okc, ovc, s * hw, kv, L, scale, rows=arow)
            check_attn(to_host_f64(out[:, arow]), ref, f"c{c}s{step} attn")
        # the whole written prefix of the cache, sampled
        prefix = (s + wl.frames) * hw
        sample = np.sort(rng.choice(prefix, 256, replace=False))
        gk = to_host_f64(kc[:, sample])
        assert np.abs(gk - okc[:, sample]).max() <= 2 ** -7 * max(1.0, np.abs(okc[:, sample]).max())
        assert np.array_equal(to_host_f64(vc[:, sample]), ovc[:, sample])
        # rows past the prefix were never written
        if prefix < cap:
            assert bool((kc[:, prefix:] == 0).all()) and bool((vc[:, prefix:] == 0).all())
