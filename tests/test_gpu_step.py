"""GPU parity of whole steps at full size: the 480P step and the 720P step
end to end ([YL] Algorithm 3 steps 5-6).

The cache is built the way the step finds it: every earlier chunk of the
video (frames 0, 3, ...) goes through rope3d_apply_append from its own
seeded q, k, v, then the current chunk does, and its rotated queries attend
to the cache.  The oracle keeps its own cache from the same seeded inputs
(rotated k stored at the cache's bf16 precision, v as given) and its own
bf16-rounded rotated queries.  Checked against it:

* every chunk's written K/V rows, every token (bf16 RoPE rule; V
  bit-exact), the current chunk's q' on every token, and at the end every
  cache row, bit for bit against what its chunk wrote;
* attention: the 480P step on all 4680 rows of all 12 heads; the 720P step
  on one seeded row of every 32-row wave of every head plus the first and
  last row of every 256-row query tile (max 2e-2 / mean 2e-3 / rel L2 1e-2);
* the NaN-poisoned attention output is finite everywhere.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import (check_attn, check_bf16_rope, say, to_dev, to_host_f64, torch,
                      wave_rows)
from oracle import attention as A
from oracle import rope3d as R
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu


def _bf16(x64: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x64.astype(np.float32))).astype(np.float64)


def _bits(x) -> np.ndarray:
    return x.cpu().view(torch().int16).numpy()


def _step_end_to_end(name: str, all_rows: bool):
    t = torch()
    wl = synth.WORKLOADS[name]
    nh, D, F, L, hw = wl.n_heads, wl.head_dim, wl.frames, wl.chunk_tokens, wl.hw
    s_cur = wl.start_frames[0]
    kv = (s_cur + F) * hw
    r = wl.rope
    tables = rcc.rope3d_tables(rcc.rope_cfg(r.d_t, r.d_h, r.d_w, r.max_t, r.max_h, r.max_w,
                                            r.theta))
    otab = R.rope3d_tables(r.d_t, r.d_h, r.d_w, r.theta, r.max_t, r.max_h, r.max_w)
    kc = t.full((1, kv, nh, D), float("nan"), dtype=t.bfloat16, device="cuda")
    vc = t.full_like(kc, float("nan"))
    okc = np.zeros((1, kv, nh, D))
    ovc = np.zeros((1, kv, nh, D))
    snaps = []
    for s in list(range(0, s_cur, F)) + [s_cur]:
        host = [synth.normal((1, L, nh, D), synth.seed_for(name, s, 0, x), "bf16")
                for x in ("q", "k", "v")]
        qo = t.full((1, L, nh, D), float("nan"), dtype=t.bfloat16, device="cuda")
        say(name, "rope + append, start frame", s)
        rcc.rope3d_apply_append(tables, rcc.grid(F, wl.height, wl.width, s, 0),
                                *(to_dev(x, "bf16") for x in host), qo, kc, vc)
        t.cuda.synchronize()
        q, k, v = (synth.to_f64(x, "bf16") for x in host)
        pos = R.positions(F, wl.height, wl.width, s, 0, L)
        rows = pos[:, 3]
        rk = R.rope3d_apply(k, otab, pos)
        check_bf16_rope(to_host_f64(kc[:, s * hw:(s + F) * hw]), rk, f"{name} s{s} k rows")
        assert np.array_equal(to_host_f64(vc[:, s * hw:(s + F) * hw]), v)
        snaps.append((_bits(kc[:, s * hw:(s + F) * hw]), _bits(vc[:, s * hw:(s + F) * hw])))
        okc[:, rows] = _bf16(rk)
        ovc[:, rows] = v
        del rk
    rq = R.rope3d_apply(q, otab, pos)
    check_bf16_rope(to_host_f64(qo), rq, f"{name} q'")
    oq = _bf16(rq)
    del rq
    # every cache row still holds what its chunk wrote (bit for bit)
    assert np.array_equal(_bits(kc), np.concatenate([a for a, _ in snaps], axis=1))
    assert np.array_equal(_bits(vc), np.concatenate([b for _, b in snaps], axis=1))
    del snaps

    out = t.full((1, L, nh, D), float("nan"), dtype=t.bfloat16, device="cuda")
    say(name, "attention", L, "x", kv)
    rcc.chunk_causal_attn(qo, kc, vc, out, s_cur * hw, kv, L, 1.0 / math.sqrt(D))
    t.cuda.synchronize()
    assert bool(t.isfinite(out).all()), f"{name}: non-finite attention output"
    arows = np.arange(L) if all_rows else wave_rows(L, 17)
    ref = A.chunk_causal_attention(oq, okc, ovc, s_cur * hw, kv, L, 1.0 / math.sqrt(D),
                                   rows=arows)
    got = to_host_f64(out)[:, arows]
    return check_attn(got, ref, f"{name} attention ({arows.size} rows x {nh} heads)")


def test_480p_step_end_to_end_every_row():
    """Wan-1.3B 480P: chunks at frames 0 and 3 fill the cache, the chunk at
    frames 6..8 attends all 14040 keys; all 4680 x 12 attention rows."""
    say("480p step", _step_end_to_end("480p_step", all_rows=True))


def test_720p_step_end_to_end_every_wave():
    """Wan-14B 720P: chunks at frames 0, 3, ..., 15 fill the cache, the chunk
    at frames 18..20 attends all 75600 keys; a row of every wave of every head."""
    say("720p step", _step_end_to_end("720p_step", all_rows=False))
