#!/usr/bin/env python3
"""Benchmark of the Causal-RoPE + chunk-causal attention hot path on one MI355X.

One step = one pass of the path over the Wan-1.3B-shaped 480P workload:
rope3d_apply_append on the 4680-token chunk at global frames 6..8 (12 heads,
head_dim 128, bf16) writing rotated K and V into the cache, then
chunk_causal_attn of the chunk's 4680 queries over the 14040 cached keys
(frames 0..8).  The cos/sin tables are built once per process before timing,
as the method prescribes (precomputed, not per call).  Before the W warm-up
steps the step runs untimed for PREWARM_S seconds: the board's power
management takes tens of milliseconds to settle its clocks after idle, and a
timed region that starts earlier measures that ramp rather than the kernels
(the first 20 steps after idle run ~20% slower than the steady state).

Prints ONE JSON line.  `value` is the step's attention TFLOP/s over the whole
step time (RoPE included); the roofline object is for the dominant kernel
(attention), timed with HIP events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk-causal attn TFLOP/s + ms/chunk (Wan-1.3B 480P); RoPE kernel GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
N_SETS = 6  # rotating input sets: > 256 MB of traffic between reuses of one set
PREWARM_S = 0.25  # untimed steps before the warm-up, so the clocks have settled


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=4680,
                   help="query rows per head in the oracle's timed sample")
    return p.parse_args()


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed: what the
    compiler sees, so that editing a comment keeps the hash."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of what the attention kernels are compiled from (comments and
    whitespace ignored): their sources, and from the shared internal header
    the vector typedefs, the buffer-resource flags and the attention argument
    struct (the rest of that header serves other kernels)."""
    import re
    csrc = os.path.join(ROOT, "rope_chunk_causal_amd", "csrc")
    h = hashlib.sha256()
    for f in ("attn.hip", "attn_d128.hip", "attn_tile.h"):
        with open(os.path.join(csrc, f)) as fh:
            h.update(_code_only(fh.read()).encode())
    text = open(os.path.join(csrc, "rcc_internal.h")).read()
    for m in re.finditer(r"^typedef [^\n]*;$|^constexpr int kRawBufferFlags[^\n]*;$|"
                         r"^struct AttnArgs \{.*?^\};", text, re.M | re.S):
        h.update(_code_only(m.group(0)).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (the library has no multi-GPU path); "
              f"got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    import rope_chunk_causal_amd as rcc
    from rope_chunk_causal_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rcc.lib()

    wl = synth.WORKLOADS["480p_step"]
    s = wl.start_frames[0]
    nh, D, L, hw = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw
    kv = (s + wl.frames) * hw
    cap = kv
    q_pos = s * hw
    scale = 1.0 / math.sqrt(D)
    r = wl.rope
    cfg = rcc.rope_cfg(r.d_t, r.d_h, r.d_w, r.max_t, r.max_h, r.max_w, r.theta)

    t0 = time.perf_counter()
    tables = rcc.rope3d_tables(cfg)
    torch.cuda.synchronize()
    tables_ms = (time.perf_counter() - t0) * 1e3

    gen = torch.Generator(device=dev)
    gen.manual_seed(20)
    bf = torch.bfloat16

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(bf)

    sets = []
    for _ in range(N_SETS):
        sets.append(dict(
            q=randn(1, L, nh, D), k=randn(1, L, nh, D), v=randn(1, L, nh, D),
            q_out=torch.empty(1, L, nh, D, device=dev, dtype=bf),
            kc=randn(1, cap, nh, D), vc=randn(1, cap, nh, D),   # frames 0..5 already cached
            out=torch.empty(1, L, nh, D, device=dev, dtype=bf)))
    grid = rcc.grid(wl.frames, wl.height, wl.width, s, 0)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        s = stream
        st = sets[i % N_SETS]
        if ev is not None:
            ev[0].record(s)
        rcc.rope3d_apply_append(tables, grid, st["q"], st["k"], st["v"], st["q_out"],
                                st["kc"], st["vc"], stream=s)
        if ev is not None:
            ev[1].record(s)
        rcc.chunk_causal_attn(st["q_out"], st["kc"], st["vc"], st["out"], q_pos, kv, L, scale,
                              stream=s)
        if ev is not None:
            ev[2].record(s)

    prewarm = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PREWARM_S:
        for _ in range(10):
            step(prewarm)
            prewarm += 1
        torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-kernel durations with HIP events on the launch stream (separate pass)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    rope_all = sorted(e[0].elapsed_time(e[1]) for e in evs)
    attn_all = sorted(e[1].elapsed_time(e[2]) for e in evs)
    rope_ms = sum(rope_all) / args.steps
    attn_ms = sum(attn_all) / args.steps

    attn_flops = 4.0 * L * kv * D * nh
    rope_bytes = 6.0 * L * nh * D * 2
    step_tflops = attn_flops / (ms_per_step * 1e-3) / 1e12
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    rope_gbps = rope_bytes / (rope_ms * 1e-3) / 1e9

    # RoPE bandwidth configuration: one SP rank's 585-token slice, 64 chunks batched
    sp = synth.WORKLOADS["480p_sp_shard"]
    n_sp, B_sp, s_sp = sp.chunk_tokens // synth.SP_DEGREE, 64, sp.start_frames[0]
    cap_sp = (s_sp + sp.frames) * sp.hw
    sp_sets = []
    for _ in range(2):
        sp_sets.append([randn(B_sp, n_sp, nh, D) for _ in range(3)] +
                       [torch.empty(B_sp, n_sp, nh, D, device=dev, dtype=bf),
                        torch.empty(B_sp, cap_sp, nh, D, device=dev, dtype=bf),
                        torch.empty(B_sp, cap_sp, nh, D, device=dev, dtype=bf)])
    g_sp = rcc.grid(sp.frames, sp.height, sp.width, s_sp, 2 * n_sp)
    for i in range(3):
        rcc.rope3d_apply_append(tables, g_sp, *sp_sets[i % 2], stream=stream)
    reps = 20
    sp_ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    sp_ev[0].record(stream)
    for i in range(reps):
        rcc.rope3d_apply_append(tables, g_sp, *sp_sets[i % 2], stream=stream)
        sp_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    sp_ms = sum(sp_ev[i].elapsed_time(sp_ev[i + 1]) for i in range(reps)) / reps
    sp_bytes = 6.0 * B_sp * n_sp * nh * D * 2
    sp_gbps = sp_bytes / (sp_ms * 1e-3) / 1e9
    del sp_sets
    cp_gbps = _plain_copy_gbps(sp_bytes, reps, dev)
    cp480_gbps = _plain_copy_gbps(rope_bytes, reps, dev)

    rollout = rollout_480p(rcc, synth, cfg, tables, randn, stream, dev)
    qkv = qkv_rope_fused(rcc, synth, cfg, tables, randn, stream, dev)
    rolling = rolling_rollout(rcc, synth, cfg, tables, randn, stream, dev)
    sparse = block_sparse(rcc, synth, randn, stream, dev)
    attn720 = attn_720p(rcc, synth, randn, stream, dev)
    attn720_long = attn_720p_long_cache(rcc, synth, randn, stream, dev)
    occupancy = attn_occupancy(rcc, synth, randn, stream, dev)

    traffic = read_traffic("chunk_causal_attn_480p_step")
    result = {
        "metric": METRIC,
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, Wan-1.3B 480P shapes)",
        "config": {"workload": "480p_step", "heads": nh, "head_dim": D,
                   "rope_bands": [r.d_t, r.d_h, r.d_w], "grid": [wl.frames, wl.height, wl.width],
                   "start_frame": s, "q_tokens": L, "kv_tokens": kv, "batch": 1},
        "ms_per_chunk": round(ms_per_step, 4),
        "prewarm_steps": prewarm,
        "attn_ms": round(attn_ms, 4),
        "attn_ms_median": round(attn_all[len(attn_all) // 2], 4),
        "attn_ms_min": round(attn_all[0], 4),
        "attn_tflops": round(attn_tflops, 2),
        "rope_ms": round(rope_ms, 4),
        "rope_gbps": round(rope_gbps, 1),
        "rope_frac_hbm": round(rope_gbps / PEAK_HBM_GBPS, 4),
        "rope_plain_copy_gbps": round(cp480_gbps, 1),
        "rope_frac_of_plain_copy": round(rope_gbps / cp480_gbps, 4),
        "rope_sp_shard_b64": {"ms": round(sp_ms, 4), "gbps": round(sp_gbps, 1),
                              "bytes": sp_bytes, "frac_hbm": round(sp_gbps / PEAK_HBM_GBPS, 4),
                              "plain_copy_gbps": round(cp_gbps, 1),
                              "frac_of_plain_copy": round(sp_gbps / cp_gbps, 4)},
        "tables_once_ms": round(tables_ms, 3),
        "rollout_480p": rollout,
        "qkv_rope_append": qkv,
        "rolling_1min": rolling,
        "block_sparse": sparse,
        "attn_720p": attn720,
        "attn_720p_cache_past_4gib": attn720_long,
        "attn_occupancy": occupancy,
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": None,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows, wl, s, kv, scale)
        result["cpu_oracle_other_workloads"] = cpu_oracle_workloads()
    print(json.dumps(result), flush=True)


def _plain_copy_gbps(nbytes, reps, dev):
    """A plain device-to-device copy (torch copy_) moving the same bytes (half
    read, half written), two rotating buffer pairs, HIP events per copy: the
    rate a bandwidth-bound kernel of this size can be held against."""
    import torch
    n_el = int(nbytes // 4)
    bf = torch.bfloat16
    cp = [(torch.empty(n_el, device=dev, dtype=bf), torch.empty(n_el, device=dev, dtype=bf))
          for _ in range(2)]
    for i in range(3):
        cp[i % 2][1].copy_(cp[i % 2][0])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        cp[i % 2][1].copy_(cp[i % 2][0])
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(reps)) / reps
    return 4.0 * n_el / (ms * 1e-3) / 1e9


def _time_events(fn, stream, reps):
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return sum(ev[i].elapsed_time(ev[i + 1]) for i in range(reps)) / reps


def qkv_rope_fused(rcc, synth, cfg, tables, randn, stream, dev):
    """The fused QKV projection + Causal-RoPE + cache write on the 480P chunk
    (4680 tokens) and on the 64-chunk SP-rank batch (64 x 585 tokens), model
    dim 1536 -> 3 x 12 x 128, with the unfused path beside it: three torch
    (hipBLASLt) projections into contiguous q, k, v, then rope3d_apply_append.
    Two input sets alternate; HIP events on the launch stream."""
    import torch
    wl = synth.WORKLOADS["480p_step"]
    nh, D = wl.n_heads, wl.head_dim
    K = nh * D
    out = {}
    for name, B, n, s, off in (("480p_chunk", 1, wl.chunk_tokens, wl.start_frames[0], 0),
                               ("sp_shard_b64", 64, wl.chunk_tokens // synth.SP_DEGREE, 9,
                                2 * (wl.chunk_tokens // synth.SP_DEGREE))):
        g = rcc.grid(wl.frames, wl.height, wl.width, s, off)
        cap = (s + wl.frames) * wl.hw
        sets = []
        for _ in range(2):
            x = randn(B, n, K)
            w = (randn(3 * nh * D, K).float() / math.sqrt(K)).to(torch.bfloat16)
            sets.append(dict(x=x, w=w, q=torch.empty(B, n, nh, D, device=dev, dtype=torch.bfloat16),
                             kc=torch.empty(B, cap, nh, D, device=dev, dtype=torch.bfloat16),
                             vc=torch.empty(B, cap, nh, D, device=dev, dtype=torch.bfloat16),
                             yq=torch.empty(B, n, K, device=dev, dtype=torch.bfloat16),
                             yk=torch.empty(B, n, K, device=dev, dtype=torch.bfloat16),
                             yv=torch.empty(B, n, K, device=dev, dtype=torch.bfloat16)))

        def fused(i):
            st = sets[i % 2]
            rcc.qkv_rope_append(tables, g, st["x"], st["w"], None, st["q"], st["kc"], st["vc"],
                                stream=stream)

        def unfused(i):
            st = sets[i % 2]
            w = st["w"]
            torch.matmul(st["x"], w[:K].t(), out=st["yq"])
            torch.matmul(st["x"], w[K:2 * K].t(), out=st["yk"])
            torch.matmul(st["x"], w[2 * K:].t(), out=st["yv"])
            rcc.rope3d_apply_append(tables, g, st["yq"].view(B, n, nh, D),
                                    st["yk"].view(B, n, nh, D), st["yv"].view(B, n, nh, D),
                                    st["q"], st["kc"], st["vc"], stream=stream)

        for i in range(4):
            fused(i)
            unfused(i)
        torch.cuda.synchronize()
        reps = 20
        f_ms = _time_events(fused, stream, reps)
        u_ms = _time_events(unfused, stream, reps)
        flop = 2.0 * B * n * K * 3 * nh * D
        out[name] = {"tokens": B * n, "ms": round(f_ms, 4), "tflops": round(flop / f_ms / 1e9, 1),
                     "unfused_ms": round(u_ms, 4), "flop": flop}
    return out


def rollout_480p(rcc, synth, cfg, tables, randn, stream, dev):
    """The full 5 s 480P rollout on one layer: 7 chunks x 4 denoising steps,
    each RoPE+append then attention over the growing cache (timed once after
    one untimed pass; inputs pre-generated in HBM)."""
    import torch
    wl = synth.WORKLOADS["480p_rollout"]
    nh, D, L, hw = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw
    cap = wl.cache_tokens()
    kc = torch.zeros(1, cap, nh, D, device=dev, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    steps = [(s, [randn(1, L, nh, D) for _ in range(3)])
             for s in wl.start_frames for _ in range(wl.steps)]
    qo = torch.empty(1, L, nh, D, device=dev, dtype=torch.bfloat16)
    out = torch.empty_like(qo)
    scale = 1.0 / math.sqrt(D)

    def run(ev=None):
        for i, (s, (q, k, v)) in enumerate(steps):
            if ev is not None:
                ev[i][0].record(stream)
            rcc.rope3d_apply_append(tables, rcc.grid(wl.frames, wl.height, wl.width, s, 0),
                                    q, k, v, qo, kc, vc, stream=stream)
            if ev is not None:
                ev[i][1].record(stream)
            rcc.chunk_causal_attn(qo, kc, vc, out, s * hw, (s + wl.frames) * hw, L, scale,
                                  stream=stream)
            if ev is not None:
                ev[i][2].record(stream)

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    total_ms = (time.perf_counter() - t0) * 1e3
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in steps]
    run(ev)
    torch.cuda.synchronize()
    rope_ms = sum(e[0].elapsed_time(e[1]) for e in ev)
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in ev)
    flops = sum(4.0 * L * (s + wl.frames) * hw * D * nh for s, _ in steps)
    rope_bytes = len(steps) * 6.0 * L * nh * D * 2
    return {"chunks": len(wl.start_frames), "steps_per_chunk": wl.steps,
            "ms_total": round(total_ms, 3), "ms_per_chunk": round(total_ms / len(wl.start_frames), 4),
            "attn_ms": round(attn_ms, 3), "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 1),
            "rope_ms": round(rope_ms, 3), "rope_gbps": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
            "attn_flop": flops}


def rolling_rollout(rcc, synth, cfg, tables, randn, stream, dev):
    """One layer of a 1-minute 480P rollout (80 chunks x 4 denoising steps,
    frames 0..239) through the rolling-window ring of 21 frames, beside the
    same rollout over a cache that keeps every frame.  Each step is
    RoPE + append then attention over what the cache holds.  Eight input sets
    rotate (their content does not change the work); the ring rollout is
    timed once after an untimed pass, the full-cache one once after a short
    warm-up; HIP events on the launch stream give the per-kernel sums.
    Also times the ring write alone on the 64-chunk SP-rank batch."""
    import torch
    wl = synth.WORKLOADS["480p_rolling_1min"]
    nh, D, L, hw, F = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw, wl.frames
    bf = torch.bfloat16
    sets = [[randn(1, L, nh, D) for _ in range(3)] for _ in range(8)]
    qo = torch.empty(1, L, nh, D, device=dev, dtype=bf)
    out = torch.empty_like(qo)
    scale = 1.0 / math.sqrt(D)
    steps = [s for s in wl.start_frames for _ in range(wl.steps)]
    ring = rcc.ring(wl.sink_frames, wl.window_frames)

    def run(kc, vc, use_ring, steps, ev=None):
        for i, s in enumerate(steps):
            q, k, v = sets[i % len(sets)]
            g = rcc.grid(F, wl.height, wl.width, s, 0)
            if ev is not None:
                ev[i][0].record(stream)
            if use_ring:
                rcc.rope3d_apply_append_ring(tables, g, ring, q, k, v, qo, kc, vc,
                                             stream=stream)
            else:
                rcc.rope3d_apply_append(tables, g, q, k, v, qo, kc, vc, stream=stream)
            if ev is not None:
                ev[i][1].record(stream)
            if use_ring:
                rcc.chunk_causal_attn_ring(g, ring, qo, kc, vc, out, scale, stream=stream)
            else:
                rcc.chunk_causal_attn(qo, kc, vc, out, s * hw, (s + F) * hw, L, scale,
                                      stream=stream)
            if ev is not None:
                ev[i][2].record(stream)

    def timed(cap, use_ring, warm_steps):
        kc = torch.zeros(1, cap, nh, D, device=dev, dtype=bf)
        vc = torch.zeros_like(kc)
        run(kc, vc, use_ring, warm_steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(kc, vc, use_ring, steps)
        torch.cuda.synchronize()
        total = (time.perf_counter() - t0) * 1e3
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in steps]
        run(kc, vc, use_ring, steps, ev)
        torch.cuda.synchronize()
        rope = [e[0].elapsed_time(e[1]) for e in ev]
        attn = [e[1].elapsed_time(e[2]) for e in ev]
        del kc, vc
        return total, rope, attn

    ring_rows = wl.cache_tokens()
    r_total, r_rope, r_attn = timed(ring_rows, True, steps)
    full_rows = (wl.start_frames[-1] + F) * hw
    f_total, f_rope, f_attn = timed(full_rows, False, steps[:8])
    torch.cuda.empty_cache()

    def flops(s, ring_kv):
        lk = min(s + F, wl.sink_frames + wl.window_frames) if ring_kv else s + F
        return 4.0 * L * lk * hw * D * nh
    r_flop = sum(flops(s, True) for s in steps)
    f_flop = sum(flops(s, False) for s in steps)
    full_from = next(i for i, s in enumerate(steps) if s + F >= wl.sink_frames + wl.window_frames)
    steady_attn = sum(r_attn[full_from:]) / (len(steps) - full_from)
    steady_rope = sum(r_rope[full_from:]) / (len(steps) - full_from)
    rope_bytes = 6.0 * L * nh * D * 2

    # the ring write alone on the SP-rank batch (64 x 585 tokens at frames 237..239)
    n_sp, B_sp = L // synth.SP_DEGREE, 64
    g_sp = rcc.grid(F, wl.height, wl.width, 237, 2 * n_sp)
    sp_sets = [[randn(B_sp, n_sp, nh, D) for _ in range(3)] +
               [torch.empty(B_sp, n_sp, nh, D, device=dev, dtype=bf),
                torch.empty(B_sp, ring_rows, nh, D, device=dev, dtype=bf),
                torch.empty(B_sp, ring_rows, nh, D, device=dev, dtype=bf)] for _ in range(2)]

    def sp_ring(i):
        rcc.rope3d_apply_append_ring(tables, g_sp, ring, *sp_sets[i % 2], stream=stream)
    for i in range(3):
        sp_ring(i)
    sp_ms = _time_events(sp_ring, stream, 20)
    sp_bytes = 6.0 * B_sp * n_sp * nh * D * 2
    del sp_sets
    torch.cuda.empty_cache()
    kv_bytes = 2 * nh * D * 2
    return {"window_frames": wl.window_frames, "sink_frames": wl.sink_frames,
            "chunks": len(wl.start_frames), "steps_per_chunk": wl.steps,
            "ms_total": round(r_total, 2), "ms_per_chunk": round(r_total / len(wl.start_frames), 4),
            "attn_ms": round(sum(r_attn), 2),
            "attn_tflops": round(r_flop / (sum(r_attn) * 1e-3) / 1e12, 1),
            "steady_attn_ms_per_step": round(steady_attn, 4),
            "steady_rope_ms_per_step": round(steady_rope, 4),
            "steady_rope_gbps": round(rope_bytes / (steady_rope * 1e-3) / 1e9, 1),
            "ring_rows": ring_rows, "ring_kv_bytes": ring_rows * kv_bytes,
            "rope_ring_sp_b64": {"ms": round(sp_ms, 4),
                                 "gbps": round(sp_bytes / (sp_ms * 1e-3) / 1e9, 1)},
            "full_cache": {"ms_total": round(f_total, 2), "attn_ms": round(sum(f_attn), 2),
                           "attn_tflops": round(f_flop / (sum(f_attn) * 1e-3) / 1e12, 1),
                           "last_attn_ms_per_step": round(f_attn[-1], 4),
                           "cache_rows": full_rows, "kv_bytes": full_rows * kv_bytes}}


def attn_720p(rcc, synth, randn, stream, dev):
    """chunk_causal_attn on the Wan-14B-shaped 720P step: 10800 queries (frames
    18..20) over 75600 keys, 40 heads; 2 untimed launches, then 10 timed with
    HIP events on the launch stream."""
    import torch
    wl = synth.WORKLOADS["720p_step"]
    s = wl.start_frames[0]
    nh, D, L, hw = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw
    kv = (s + wl.frames) * hw
    q = randn(1, L, nh, D)
    k = randn(1, kv, nh, D)
    v = randn(1, kv, nh, D)
    o = torch.empty_like(q)
    scale = 1.0 / math.sqrt(D)

    def run(i):
        rcc.chunk_causal_attn(q, k, v, o, s * hw, kv, L, scale, stream=stream)
    for i in range(2):
        run(i)
    ms = _time_events(run, stream, 10)
    flop = wl.attn_flops(s)
    del q, k, v, o
    torch.cuda.empty_cache()
    return {"ms": round(ms, 3), "tflops": round(flop / (ms * 1e-3) / 1e12, 1), "q_tokens": L,
            "kv_tokens": kv, "heads": nh, "frac_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def attn_720p_long_cache(rcc, synth, randn, stream, dev):
    """chunk_causal_attn at 720P late in a long video: the chunk at frames
    117..119 over a cache that keeps all 120 frames (432000 keys x 40 heads,
    4.4 GB each for K and V, past 4 GiB per batch entry), on the same
    bf16 head_dim-128 kernel as every other step; 1 untimed launch, then 3
    timed with HIP events on the launch stream."""
    import torch
    wl = synth.WORKLOADS["720p_step"]
    nh, D, L, hw = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw
    s = 117
    kv = (s + wl.frames) * hw
    q = randn(1, L, nh, D)
    k = torch.empty(1, kv, nh, D, device=dev, dtype=torch.bfloat16)
    v = torch.empty_like(k)
    for t in (k, v):       # fill frame by frame (bounded temporaries)
        for f0 in range(0, kv, 12 * hw):
            n = min(12 * hw, kv - f0)
            t[:, f0:f0 + n] = randn(1, n, nh, D)
    o = torch.empty_like(q)
    scale = 1.0 / math.sqrt(D)

    def run(i):
        rcc.chunk_causal_attn(q, k, v, o, s * hw, kv, L, scale, stream=stream)
    run(0)
    ms = _time_events(run, stream, 3)
    flop = 4.0 * L * kv * D * nh
    entry_bytes = kv * nh * D * 2
    del q, k, v, o
    torch.cuda.empty_cache()
    return {"ms": round(ms, 3), "tflops": round(flop / (ms * 1e-3) / 1e12, 1), "q_tokens": L,
            "kv_tokens": kv, "heads": nh, "k_cache_bytes_per_entry": entry_bytes,
            "past_4gib": entry_bytes > (1 << 32),
            "frac_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def attn_occupancy(rcc, synth, randn, stream, dev):
    """The 480P attention shape with 1, 4, 8, 10 and 12 heads (19 query tiles
    per head, one round of workgroups): the same work per workgroup at every
    size.  A launch that takes longer with more busy CUs is held by the
    chip's power limit, not by the grid.  10 timed launches each."""
    wl = synth.WORKLOADS["480p_step"]
    s = wl.start_frames[0]
    L, D, hw = wl.chunk_tokens, wl.head_dim, wl.hw
    kv = (s + wl.frames) * hw
    out = {}
    for nh in (1, 4, 8, 10, 12):
        q = randn(1, L, nh, D)
        k = randn(1, kv, nh, D)
        v = randn(1, kv, nh, D)
        o = q.clone()

        def run(i):
            rcc.chunk_causal_attn(q, k, v, o, s * hw, kv, L, 1.0 / math.sqrt(D), stream=stream)
        for i in range(3):
            run(i)
        ms = _time_events(run, stream, 10)
        out[f"heads_{nh}"] = {"busy_cus": 19 * nh, "ms": round(ms, 4),
                              "tflops": round(4.0 * L * kv * D * nh / (ms * 1e-3) / 1e12, 1)}
    return out


def block_sparse(rcc, synth, randn, stream, dev):
    """Block-sparse attention on the Sparse Forcing-shaped memory (query
    chunk of 84 blocks of 64 tokens, 168 persistent + 336 local-window blocks,
    12 heads; and the same token counts in [3,4,4] blocks of 48: 112 query,
    224 persistent and 448 window blocks) at Top-K 25 / 12.5 / 6.25 % of the
    window, beside the dense kernel over the whole memory (every key
    visible).  TFLOP/s counts the selected query-key pairs only.  HIP events
    on the launch stream."""
    import numpy as np
    import torch
    out = {}
    w0 = next(iter(synth.SPARSE_WORKLOADS.values()))
    q = randn(1, w0.q_tokens, w0.n_heads, w0.head_dim)
    k = randn(1, w0.kv_tokens, w0.n_heads, w0.head_dim)
    v = randn(1, w0.kv_tokens, w0.n_heads, w0.head_dim)
    o = torch.empty_like(q)
    scale = 1.0 / math.sqrt(w0.head_dim)

    def dense(i):
        rcc.chunk_causal_attn(q, k, v, o, w0.kv_tokens - w0.q_tokens, w0.kv_tokens, w0.q_tokens,
                              scale, stream=stream)
    for i in range(3):
        dense(i)
    d_ms = _time_events(dense, stream, 20)
    d_flop = 4.0 * w0.q_tokens * w0.kv_tokens * w0.head_dim * w0.n_heads
    for name, w in list(synth.SPARSE_WORKLOADS.items()) + list(synth.SPARSE_WORKLOADS_344.items()):
        p, l = synth.block_lists(w, 7)
        dp = torch.from_numpy(p).to(dev)
        dl = torch.from_numpy(np.ascontiguousarray(l)).to(dev)

        def run(i):
            rcc.block_sparse_attn(q, k, v, o, w.kv_tokens, w.block, dp, dl, scale, stream=stream)
        for i in range(3):
            run(i)
        ms = _time_events(run, stream, 20)
        out[name] = {"top_k_blocks": w.top_k, "ms": round(ms, 4),
                     "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 1),
                     "speedup_vs_dense": round(d_ms / ms, 3), "flop": w.flops()}
    out["dense_full_memory"] = {"ms": round(d_ms, 4),
                                "tflops": round(d_flop / (d_ms * 1e-3) / 1e12, 1),
                                "q_tokens": w0.q_tokens, "kv_tokens": w0.kv_tokens}
    return out


def _host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS threads numpy uses."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count()
    return model, threads


def _oracle_chunks(wl, name, starts, tabs, cache_tokens, n_heads=None):
    """The oracle's cache after RoPE + append of the chunks at `starts` (seeded
    q, k, v per chunk, as the tests draw them); returns (cache k, cache v,
    rotated q of the last chunk, its positions)."""
    import numpy as np
    from oracle import rope3d as R
    from rope_chunk_causal_amd import synth
    nh = wl.n_heads if n_heads is None else n_heads
    L, D = wl.chunk_tokens, wl.head_dim
    kc = np.zeros((1, cache_tokens, nh, D))
    vc = np.zeros((1, cache_tokens, nh, D))
    q = pos = None
    for s in starts:
        q, k, v = (synth.to_f64(synth.normal((1, L, nh, D), synth.seed_for(name, s, 0, x),
                                             "bf16"), "bf16") for x in ("q", "k", "v"))
        pos = R.positions(wl.frames, wl.height, wl.width, s, 0, L)
        q = R.rope3d_apply_append(q, k, v, kc, vc, tabs, wl.frames, wl.height, wl.width, s, 0)
    return kc, vc, q, pos


def cpu_baseline(rows_per_head, wl, s, kv, scale):
    """The oracle (as it stands) timed on the host on the 480P step: RoPE +
    append of the current chunk, then attention for `rows_per_head` query
    rows of every head over the 14040 cached keys.  The cache is built the
    way the step finds it (chunks at frames 0 and 3 appended first, untimed).
    Reported in the metric's unit (TFLOP/s of attention)."""
    import numpy as np
    from oracle import attention as A
    from oracle import rope3d as R
    from rope_chunk_causal_amd import synth

    nh, D, L, hw = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw
    r = wl.rope
    tabs = R.rope3d_tables(r.d_t, r.d_h, r.d_w, r.theta, r.max_t, r.max_h, r.max_w)
    kc, vc, _, _ = _oracle_chunks(wl, "480p_step", range(0, s, wl.frames), tabs, kv)
    q, k, v = (synth.to_f64(synth.normal((1, L, nh, D), synth.seed_for("480p_step", s, 0, x),
                                         "bf16"), "bf16") for x in ("q", "k", "v"))
    t0 = time.perf_counter()
    qr = R.rope3d_apply_append(q, k, v, kc, vc, tabs, wl.frames, wl.height, wl.width, s, 0)
    t_rope = time.perf_counter() - t0
    rows = np.sort(np.random.default_rng(0).choice(L, size=rows_per_head, replace=False))
    t0 = time.perf_counter()
    A.chunk_causal_attention(qr, kc, vc, s * hw, kv, L, scale, rows=rows)
    t_attn = time.perf_counter() - t0
    flops = 4.0 * rows_per_head * kv * D * nh
    model, threads = _host_info()
    return {"value": round(flops / t_attn / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows_per_head} of {L} query rows per head x {nh} heads, Lk {kv}, fp64 "
                      f"numpy: attention {t_attn:.2f} s; RoPE+append of the whole chunk "
                      f"{t_rope:.2f} s",
            "attn_s": round(t_attn, 3), "rope_s": round(t_rope, 3),
            "rope_gbps": round(6.0 * L * nh * D * 2 / t_rope / 1e9, 3), "cpu": model}


def cpu_oracle_workloads():
    """The oracle timed on the host beside the other workloads' GPU figures,
    each on a stated sample: the SP-rank shard x 64 RoPE + append (whole
    batch, GB/s of the same algorithmic bytes as the kernel), the 5 s 480P
    rollout (the last denoising step of each of the 7 chunks, 468 query rows
    per head, TFLOP/s of attention; the full rollout's time extrapolated from
    it), and the 720P step (216 query rows per head, TFLOP/s)."""
    import numpy as np
    from oracle import attention as A
    from oracle import rope3d as R
    from rope_chunk_causal_amd import synth
    model, threads = _host_info()
    out = {"cpu": model, "cores": threads, "kind": "oracle"}

    sp = synth.WORKLOADS["480p_sp_shard"]
    n, B, s_sp = sp.chunk_tokens // synth.SP_DEGREE, 64, sp.start_frames[0]
    r = sp.rope
    tabs = R.rope3d_tables(r.d_t, r.d_h, r.d_w, r.theta, r.max_t, r.max_h, r.max_w)
    cap = (s_sp + sp.frames) * sp.hw
    q, k, v = (synth.to_f64(synth.normal((B, n, sp.n_heads, sp.head_dim), 40 + i, "bf16"), "bf16")
               for i in range(3))
    kc = np.zeros((B, cap, sp.n_heads, sp.head_dim))
    vc = np.zeros_like(kc)
    t0 = time.perf_counter()
    R.rope3d_apply_append(q, k, v, kc, vc, tabs, sp.frames, sp.height, sp.width, s_sp, 2 * n)
    t = time.perf_counter() - t0
    nbytes = 6.0 * B * n * sp.n_heads * sp.head_dim * 2
    out["rope_sp_shard_b64"] = {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s",
                                "s": round(t, 3), "sample": f"whole batch ({B} x {n} tokens)"}
    del q, k, v, kc, vc

    wl = synth.WORKLOADS["480p_rollout"]
    nh, D, L, hw = wl.n_heads, wl.head_dim, wl.chunk_tokens, wl.hw
    rows_per_head = 468
    rows = np.sort(np.random.default_rng(1).choice(L, size=rows_per_head, replace=False))
    kc = np.zeros((1, wl.cache_tokens(), nh, D))
    vc = np.zeros_like(kc)
    t_rope = t_attn = flop = 0.0
    for s in wl.start_frames:
        q, k, v = (synth.to_f64(synth.normal((1, L, nh, D),
                                             synth.seed_for("480p_rollout", s, wl.steps - 1, x),
                                             "bf16"), "bf16") for x in ("q", "k", "v"))
        t0 = time.perf_counter()
        qr = R.rope3d_apply_append(q, k, v, kc, vc, tabs, wl.frames, wl.height, wl.width, s, 0)
        t_rope += time.perf_counter() - t0
        kv = (s + wl.frames) * hw
        t0 = time.perf_counter()
        A.chunk_causal_attention(qr, kc, vc, s * hw, kv, L, 1.0 / math.sqrt(D), rows=rows)
        t_attn += time.perf_counter() - t0
        flop += 4.0 * rows_per_head * kv * D * nh
    full_flop = sum(4.0 * L * (s + wl.frames) * hw * D * nh for s in wl.start_frames) * wl.steps
    tf = flop / t_attn / 1e12
    out["rollout_480p"] = {"value": round(tf, 6), "unit": "TFLOP/s",
                           "attn_s": round(t_attn, 3), "rope_s": round(t_rope, 3),
                           "sample": f"last denoising step of each of the {len(wl.start_frames)} "
                                     f"chunks, {rows_per_head} of {L} query rows per head x "
                                     f"{nh} heads (RoPE + append of whole chunks)",
                           "full_rollout_attn_s_extrapolated": round(full_flop / (tf * 1e12), 1)}
    del kc, vc

    wl = synth.WORKLOADS["720p_step"]
    D, L, hw = wl.head_dim, wl.chunk_tokens, wl.hw
    nh = 5          # one GPU's share of the 40 heads split over 8
    s = wl.start_frames[0]
    kv = (s + wl.frames) * hw
    rows_per_head = 1728
    rows = np.sort(np.random.default_rng(2).choice(L, size=rows_per_head, replace=False))
    r = wl.rope
    tabs = R.rope3d_tables(r.d_t, r.d_h, r.d_w, r.theta, r.max_t, r.max_h, r.max_w)
    kc, vc, qr, _ = _oracle_chunks(wl, "720p_step", list(range(0, s + 1, wl.frames)), tabs, kv,
                                   n_heads=nh)
    t0 = time.perf_counter()
    A.chunk_causal_attention(qr, kc, vc, s * hw, kv, L, 1.0 / math.sqrt(D), rows=rows)
    t_attn = time.perf_counter() - t0
    flop = 4.0 * rows_per_head * kv * D * nh
    out["attn_720p"] = {"value": round(flop / t_attn / 1e12, 6), "unit": "TFLOP/s",
                        "attn_s": round(t_attn, 3),
                        "sample": f"{rows_per_head} of {L} query rows per head x {nh} of "
                                  f"{wl.n_heads} heads, Lk {kv} (cache from the oracle's RoPE + "
                                  f"append of the 7 chunks, untimed)",
                        "full_step_s_extrapolated": round(wl.attn_flops(s) / (flop / t_attn), 1)}
    return out


if __name__ == "__main__":
    main()
