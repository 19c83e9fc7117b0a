"""Run workloads of the hot path a few times each, for rocprofv3 collection.

    python -m rope_chunk_causal_amd.prof_run WORKLOAD [WORKLOAD ...] [--reps N]

WORKLOAD: attn_480p (chunk_causal_attn, 4680 queries over 14040 keys, 12
heads), attn_720p (10800 over 75600, 40 heads), rope_480p (one 4680-token
chunk, 12 heads), rope_sp_b64 (585-token rank slice, 64 chunks batched),
qkv_480p / qkv_sp_b64 (qkv_rope_append, model dim 1536 -> 3 x 12 x 128, on
the same two token sets), ring_1min (one layer of a 1-minute rollout, 80
chunks x 4 steps, RoPE + ring write then attention over a 21-frame rolling
window), sparse_sf512 (block_sparse_attn on the Sparse Forcing-shaped
memory at Top-K 25, 12.5 and 6.25 %, then the dense kernel over the same
memory), sparse_sf344 (the same with [3,4,4] blocks of 48 tokens), copy (a
plain 1 GiB device-to-device copy: the reference for scaling HBM byte
counters), all (copy, attn_480p, attn_720p, rope_480p, rope_sp_b64,
qkv_480p, qkv_sp_b64, sparse_sf512, in that order).  Workloads run in the
order given.  Inputs are seeded N(0,1) bf16 on the device; nothing is
checked here (the tests do that).
"""
from __future__ import annotations

import argparse
import math

import torch

import rope_chunk_causal_amd as rcc
from rope_chunk_causal_amd import synth

COPY_BYTES = 1 << 30


def _randn(gen, *shape):
    return torch.randn(*shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def attn(name: str, reps: int, gen) -> None:
    wl = synth.WORKLOADS["480p_step" if name == "attn_480p" else "720p_step"]
    s = wl.start_frames[0]
    kv = (s + wl.frames) * wl.hw
    q = _randn(gen, 1, wl.chunk_tokens, wl.n_heads, wl.head_dim)
    k = _randn(gen, 1, kv, wl.n_heads, wl.head_dim)
    v = _randn(gen, 1, kv, wl.n_heads, wl.head_dim)
    o = torch.empty_like(q)
    for _ in range(reps):
        rcc.chunk_causal_attn(q, k, v, o, s * wl.hw, kv, wl.chunk_tokens, 1 / math.sqrt(wl.head_dim))


def rope(name: str, reps: int, gen) -> None:
    wl = synth.WORKLOADS["480p_step" if name == "rope_480p" else "480p_sp_shard"]
    s = wl.start_frames[0]
    if name == "rope_480p":
        batch, n, off = 1, wl.chunk_tokens, 0
    else:
        batch, n, off = 64, wl.chunk_tokens // synth.SP_DEGREE, 2 * (wl.chunk_tokens // synth.SP_DEGREE)
    r = wl.rope
    cfg = rcc.rope_cfg(r.d_t, r.d_h, r.d_w, r.max_t, r.max_h, r.max_w, r.theta)
    tables = rcc.rope3d_tables(cfg)
    cap = (s + wl.frames) * wl.hw
    q, k, v = (_randn(gen, batch, n, wl.n_heads, wl.head_dim) for _ in range(3))
    qo = torch.empty_like(q)
    kc = torch.empty(batch, cap, wl.n_heads, wl.head_dim, device="cuda", dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    g = rcc.grid(wl.frames, wl.height, wl.width, s, off)
    for _ in range(reps):
        rcc.rope3d_apply_append(tables, g, q, k, v, qo, kc, vc)


def qkv(name: str, reps: int, gen) -> None:
    wl = synth.WORKLOADS["480p_step"]
    nh, D = wl.n_heads, wl.head_dim
    K = nh * D
    if name == "qkv_480p":
        batch, n, s, off = 1, wl.chunk_tokens, wl.start_frames[0], 0
    else:
        n = wl.chunk_tokens // synth.SP_DEGREE
        batch, s, off = 64, 9, 2 * n
    r = wl.rope
    cfg = rcc.rope_cfg(r.d_t, r.d_h, r.d_w, r.max_t, r.max_h, r.max_w, r.theta)
    tables = rcc.rope3d_tables(cfg)
    cap = (s + wl.frames) * wl.hw
    x = _randn(gen, batch, n, K)
    w = (torch.randn(3 * nh * D, K, generator=gen, device="cuda") / math.sqrt(K)).to(torch.bfloat16)
    qo = torch.empty(batch, n, nh, D, device="cuda", dtype=torch.bfloat16)
    kc = torch.empty(batch, cap, nh, D, device="cuda", dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    g = rcc.grid(wl.frames, wl.height, wl.width, s, off)
    for _ in range(reps):
        rcc.qkv_rope_append(tables, g, x, w, None, qo, kc, vc)


def ring_1min(reps: int, gen) -> None:
    wl = synth.WORKLOADS["480p_rolling_1min"]
    nh, D, L, F = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.frames
    r = wl.rope
    cfg = rcc.rope_cfg(r.d_t, r.d_h, r.d_w, r.max_t, r.max_h, r.max_w, r.theta)
    tables = rcc.rope3d_tables(cfg)
    ring = rcc.ring(wl.sink_frames, wl.window_frames)
    kc = torch.zeros(1, wl.cache_tokens(), nh, D, device="cuda", dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    sets = [[_randn(gen, 1, L, nh, D) for _ in range(3)] for _ in range(4)]
    qo = torch.empty(1, L, nh, D, device="cuda", dtype=torch.bfloat16)
    out = torch.empty_like(qo)
    i = 0
    for _ in range(reps):
        for s in wl.start_frames:
            g = rcc.grid(F, wl.height, wl.width, s, 0)
            for _ in range(wl.steps):
                q, k, v = sets[i % 4]
                i += 1
                rcc.rope3d_apply_append_ring(tables, g, ring, q, k, v, qo, kc, vc)
                rcc.chunk_causal_attn_ring(g, ring, qo, kc, vc, out, 1 / math.sqrt(D))


def sparse_sf512(reps: int, gen, workloads=None) -> None:
    w0 = next(iter(synth.SPARSE_WORKLOADS.values()))
    q = _randn(gen, 1, w0.q_tokens, w0.n_heads, w0.head_dim)
    k = _randn(gen, 1, w0.kv_tokens, w0.n_heads, w0.head_dim)
    v = _randn(gen, 1, w0.kv_tokens, w0.n_heads, w0.head_dim)
    o = torch.empty_like(q)
    scale = 1 / math.sqrt(w0.head_dim)
    for w in (workloads or synth.SPARSE_WORKLOADS).values():
        p, l = synth.block_lists(w, 7)
        dp, dl = torch.from_numpy(p).cuda(), torch.from_numpy(l).cuda()
        for _ in range(reps):
            rcc.block_sparse_attn(q, k, v, o, w.kv_tokens, w.block, dp, dl, scale)
    for _ in range(reps):
        rcc.chunk_causal_attn(q, k, v, o, w0.kv_tokens - w0.q_tokens, w0.kv_tokens, w0.q_tokens,
                              scale)


def copy(reps: int) -> None:
    a = torch.ones(COPY_BYTES // 2, device="cuda", dtype=torch.bfloat16)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)


def main() -> None:
    p = argparse.ArgumentParser()
    p.add_argument("workload", nargs="+", choices=["attn_480p", "attn_720p", "rope_480p", "rope_sp_b64",
                                        "qkv_480p", "qkv_sp_b64", "ring_1min", "sparse_sf512",
                                        "sparse_sf344",
                                        "copy", "all"])
    p.add_argument("--reps", type=int, default=3)
    a = p.parse_args()
    rcc.lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    names = []
    for n in a.workload:
        names += ["copy", "attn_480p", "attn_720p", "rope_480p", "rope_sp_b64", "qkv_480p",
                  "qkv_sp_b64", "sparse_sf512"] if n == "all" else [n]
    for n in names:
        if n == "copy":
            copy(a.reps)
        elif n.startswith("attn"):
            attn(n, a.reps, gen)
        elif n.startswith("qkv"):
            qkv(n, a.reps, gen)
        elif n == "ring_1min":
            ring_1min(a.reps, gen)
        elif n == "sparse_sf512":
            sparse_sf512(a.reps, gen)
        elif n == "sparse_sf344":
            sparse_sf512(a.reps, gen, synth.SPARSE_WORKLOADS_344)
        else:
            rope(n, a.reps, gen)
        torch.cuda.synchronize()
        print(f"{n}: {a.reps} reps done", flush=True)


if __name__ == "__main__":
    main()
