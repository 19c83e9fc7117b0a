"""Seeded synthetic inputs and workload shapes.

This module is shared by the GPU path's tests/benchmark and by the CPU
oracle's callers.  It holds no arithmetic of the method itself: it only
draws i.i.d. N(0,1) numbers from numpy's PCG64 generator, rounds them to
the storage dtype (fp32, or bf16 by round-to-nearest-even on the bit
pattern), and describes the workload shapes.

bf16 arrays are carried as ``uint16`` bit patterns, since numpy has no
bfloat16 type; ``bf16_bits_to_f32`` widens them exactly.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np


# --------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as uint16 bits.

    NaN is kept quiet; the inputs drawn here are always finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(shape, seed: int, dtype: str, scale: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, scale^2) drawn from PCG64(seed) in float32.

    dtype "f32" returns float32; "bf16" returns the RNE-rounded uint16 bits.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """The exact float64 value of a stored array (fp32 or bf16 bits)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class RopeShape:
    """Per-axis RoPE band dims (each even) plus theta and table lengths."""
    d_t: int
    d_h: int
    d_w: int
    theta: float = 10000.0
    max_t: int = 1024
    max_h: int = 1024
    max_w: int = 1024

    @property
    def head_dim(self) -> int:
        return self.d_t + self.d_h + self.d_w


def wan_band_split(head_dim: int):
    """Band dims (t, h, w) used by the Wan-shaped workloads.

    head_dim 128 gives 44/42/42 and head_dim 24 gives 8/8/8: the two
    spatial bands get 2*floor(head_dim/6) dims each, time takes the rest.
    """
    s = 2 * (head_dim // 6)
    return head_dim - 2 * s, s, s


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    frames/height/width: the chunk grid (frames = latent frames per chunk).
    start_frames: the start frame s of every chunk in the rollout; the
    attention step for chunk s sees cache frames [0, s + frames).
    steps: denoising steps per chunk (each re-runs RoPE+append+attention).
    window_frames > 0: the cache is a rolling-window ring that keeps the
    first sink_frames frames and the window_frames most recent ones; the
    step for chunk s then sees min(s + frames, sink + window) frames.
    """
    name: str
    n_heads: int
    head_dim: int
    frames: int
    height: int
    width: int
    start_frames: List[int]
    steps: int
    dtype: str
    batch: int = 1
    max_t: int = 1024
    window_frames: int = 0
    sink_frames: int = 0

    @property
    def hw(self) -> int:
        return self.height * self.width

    @property
    def chunk_tokens(self) -> int:
        return self.frames * self.hw

    @property
    def rope(self) -> RopeShape:
        d_t, d_h, d_w = wan_band_split(self.head_dim)
        return RopeShape(d_t, d_h, d_w, 10000.0, self.max_t,
                         max(self.height, 1), max(self.width, 1))

    def cache_frames(self, start_frame: int) -> int:
        """Frames the step for chunk start_frame attends."""
        end = start_frame + self.frames
        if self.window_frames > 0:
            return min(end, self.sink_frames + self.window_frames)
        return end

    def cache_tokens(self) -> int:
        if self.window_frames > 0:
            return (self.sink_frames + self.window_frames) * self.hw
        return (max(self.start_frames) + self.frames) * self.hw

    def attn_flops(self, start_frame: int) -> float:
        """4*Lq*Lk*D*heads over visible pairs (all keys visible in the AR step)."""
        lq = self.chunk_tokens
        lk = self.cache_frames(start_frame) * self.hw
        return 4.0 * lq * lk * self.head_dim * self.n_heads * self.batch

    def rope_bytes(self, n_tokens: Optional[int] = None, elem: int = 2) -> float:
        """Read q,k,v + write q', k-cache, v-cache."""
        n = self.chunk_tokens if n_tokens is None else n_tokens
        return 6.0 * n * self.n_heads * self.head_dim * elem * self.batch


WORKLOADS: Dict[str, Workload] = {
    # 2 heads, head_dim 24 (8/8/8), 3 chunks of 2 frames of 4x4 patches.
    "tiny": Workload("tiny", 2, 24, 2, 4, 4, [0, 2, 4], 1, "f32", max_t=16),
    # Wan-1.3B-shaped 480P single step: chunk at frames 6..8, cache 0..8.
    "480p_step": Workload("480p_step", 12, 128, 3, 30, 52, [6], 1, "bf16"),
    # Full 5 s 480P rollout: 7 chunks x 4 denoising steps.
    "480p_rollout": Workload("480p_rollout", 12, 128, 3, 30, 52,
                             [0, 3, 6, 9, 12, 15, 18], 4, "bf16"),
    # One sequence-parallel rank's 1/8 slice of a chunk at frames 9..11.
    "480p_sp_shard": Workload("480p_sp_shard", 12, 128, 3, 30, 52, [9], 1, "bf16"),
    # Wan-14B-shaped 720P step: 40 heads, chunk at frames 18..20.
    "720p_step": Workload("720p_step", 40, 128, 3, 45, 80, [18], 1, "bf16"),
    # Long rollouts through a rolling window of 21 latent frames (the 5 s
    # horizon): 20 s = 81 latent frames in 27 chunks, 1 min = 240 frames in
    # 80 chunks, 4 denoising steps each.
    "480p_rolling_20s": Workload("480p_rolling_20s", 12, 128, 3, 30, 52,
                                 list(range(0, 81, 3)), 4, "bf16", window_frames=21),
    "480p_rolling_1min": Workload("480p_rolling_1min", 12, 128, 3, 30, 52,
                                  list(range(0, 240, 3)), 4, "bf16", window_frames=21),
}

SP_DEGREE = 8  # ranks the 480p_sp_shard workload is split over


@dataclasses.dataclass(frozen=True)
class SparseWorkload:
    """Block-sparse attention over a persistent + local block memory.

    The memory holds n_persist blocks, then the local window of n_window
    blocks whose last q_blocks blocks are the query chunk's own (the chunk
    was just written).  Each query block's local list holds its own block
    (the diagonal) and top_k - 1 other window blocks drawn without
    replacement; every query block also attends all persistent blocks.
    """
    name: str
    n_heads: int
    head_dim: int
    block: int          # tokens per block, B_t * B_h * B_w
    q_blocks: int       # query chunk
    n_persist: int      # persistent blocks (sinks + kept history)
    n_window: int       # local window blocks (includes the chunk)
    top_k: int          # local blocks per query block
    batch: int = 1

    @property
    def q_tokens(self) -> int:
        return self.q_blocks * self.block

    @property
    def kv_tokens(self) -> int:
        return (self.n_persist + self.n_window) * self.block

    def flops(self) -> float:
        keys = (self.n_persist + self.top_k) * self.block
        return 4.0 * self.q_tokens * keys * self.head_dim * self.n_heads * self.batch


def block_lists(w: SparseWorkload, seed: int):
    """Seeded persistent and local block lists (int32) for workload w.

    persist [batch, heads, n_persist] = blocks 0 .. n_persist-1 in a seeded
    order; local [batch, heads, q_blocks, top_k] = the query block's own
    block first, then distinct random window blocks.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    persist = np.empty((w.batch, w.n_heads, w.n_persist), dtype=np.int32)
    local = np.empty((w.batch, w.n_heads, w.q_blocks, w.top_k), dtype=np.int32)
    lo = w.n_persist
    own0 = w.n_persist + w.n_window - w.q_blocks
    for b in range(w.batch):
        for h in range(w.n_heads):
            persist[b, h] = g.permutation(w.n_persist)
            for i in range(w.q_blocks):
                others = np.delete(np.arange(lo, lo + w.n_window), own0 + i - lo)
                local[b, h, i, 0] = own0 + i
                local[b, h, i, 1:] = g.choice(others, w.top_k - 1, replace=False)
    return persist, local


# Sparse Forcing's setting ([1,8,8] blocks of 64 tokens at 896x512: 32 x 56
# patches, 28 blocks per latent frame): the query chunk is 3 frames (84
# blocks), the local window 12 frames (336 blocks), the persistent memory
# 6 frames' worth (168 blocks: 3 sink frames + 84 kept blocks); Top-K of
# 25%, 12.5% and 6.25% of the local window.
SPARSE_WORKLOADS: Dict[str, SparseWorkload] = {
    name: SparseWorkload(name, 12, 128, 64, 84, 168, 336, k)
    for name, k in (("sf512_top25", 84), ("sf512_top12.5", 42), ("sf512_top6.25", 21))
}


def seed_for(workload: str, start_frame: int, step: int, tensor: str) -> int:
    """Deterministic seed per (workload, chunk, step, tensor)."""
    base = {"tiny": 1, "480p_step": 20, "480p_rollout": 300,
            "480p_sp_shard": 40, "720p_step": 50, "480p_rolling_20s": 600,
            "480p_rolling_1min": 900}[workload]
    t = {"q": 0, "k": 100000, "v": 200000, "kc": 300000, "vc": 400000}[tensor]
    return base + 10 * start_frame + step + t

# The same memory with Sparse Forcing's [3,4,4] blocks (48 tokens: three
# latent frames of 4 x 4 patches, 112 blocks per 3-frame chunk at 896x512):
# query chunk 112 blocks, local window 12 frames (448 blocks), persistent
# memory 6 frames' worth (224 blocks); Top-K of 25%, 12.5% and 6.25% of the
# window.  The keys and queries are the [1,8,8] workloads' counts (5376 and
# 32256 tokens).
SPARSE_WORKLOADS_344: Dict[str, SparseWorkload] = {
    name: SparseWorkload(name, 12, 128, 48, 112, 224, 448, k)
    for name, k in (("sf344_top25", 112), ("sf344_top12.5", 56), ("sf344_top6.25", 28))
}
