"""fp64 oracle: 3D RoPE with a global time index, plus the KV-cache write.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy, float64 and
complex128 throughout.  [YL] is Yuan & Li, "Accelerating Video Generation
Inference with Sequential-Parallel 3D Positional Encoding Using a Global
Time Index" (arXiv 2603.06664).

Readings taken where the pages leave a step open:

* The per-band frequency schedule is not printed.  Each axis b with d_b
  dims gets the RoFormer schedule of its own band:
  theta_{b,j} = theta ** (-2 j / d_b), j = 0 .. d_b/2 - 1.
* Bands are concatenated t, then h, then w along head_dim, and pair j uses
  the angle of exactly one axis (the ``cat`` of Algorithm 2).  The sum in
  the §3.3.2 item 2 equation is read as that block-diagonal product.
* Pairs are adjacent elements (2j, 2j+1): Algorithm 2 reshapes the last
  dim to (-1, 2) before viewing it as complex.
* The rotation multiplies by e^{+i phi} (§3.3.1 equation).
* h and w come from the flat token index by row-major (F, H, W) order, the
  order in which Algorithm 2 broadcasts its tables over the grid.
* The output takes the caller's storage type; the oracle returns float64.
"""
from __future__ import annotations

import numpy as np


def band_angles(d_b: int, theta: float) -> np.ndarray:
    """theta_{b,j} = theta^(-2j/d_b) for j = 0 .. d_b/2-1 (float64).

    [YL] §3.3.1: frequencies are split into temporal, height and width
    parts; within a part the rotary schedule follows RoFormer.
    """
    if d_b % 2:
        raise ValueError("band dims must be even")
    j = np.arange(d_b // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / d_b)


def freq_table(max_pos: int, d_b: int, theta: float) -> np.ndarray:
    """freqs_b[p, j] = exp(i * p * theta_{b,j}), p = 0 .. max_pos-1 (complex128).

    [YL] §3.4.1 item 2 (tables precomputed once into contiguous memory) and
    Algorithm 2, whose ``freqs[0]``, ``freqs[1]``, ``freqs[2]`` are these
    per-axis tables indexed by frame, row and column.
    """
    p = np.arange(max_pos, dtype=np.float64)[:, None]
    ang = p * band_angles(d_b, theta)[None, :]
    return np.cos(ang) + 1j * np.sin(ang)


def rope3d_tables(d_t: int, d_h: int, d_w: int, theta: float,
                  max_t: int, max_h: int, max_w: int):
    """The three per-axis tables (t, h, w) of Algorithm 2 ([YL] §3.3.2)."""
    return (freq_table(max_t, d_t, theta),
            freq_table(max_h, d_h, theta),
            freq_table(max_w, d_w, theta))


def positions(frames: int, height: int, width: int, start_frame: int,
              token_offset: int, n_tokens: int) -> np.ndarray:
    """(t_global, h, w, cache_row) of tokens token_offset .. +n_tokens-1.

    [YL] §3.3.3 and Algorithm 3 steps 2-3: a rank owning the slice that
    starts at global index Delta (= r * L_local) gives its local token i the
    chunk-global index i_global = Delta + i; the frame inside the chunk is
    floor(i_global / (H*W)) and the global time index adds the start frame
    s (§3.3.2 item 1: s = k * tau for block k).  h and w follow row-major
    (F, H, W) order.  The cache row is the token's index in a cache that
    holds every frame from global frame 0 in order: s*H*W + i_global.
    Returns int64 [n_tokens, 4].
    """
    hw = height * width
    i_global = np.arange(token_offset, token_offset + n_tokens, dtype=np.int64)
    t_local = i_global // hw
    rem = i_global % hw
    out = np.empty((n_tokens, 4), dtype=np.int64)
    out[:, 0] = start_frame + t_local
    out[:, 1] = rem // width
    out[:, 2] = rem % width
    out[:, 3] = start_frame * hw + i_global
    return out


def token_freqs(tables, pos: np.ndarray) -> np.ndarray:
    """Per-token complex factors: cat(T[t], H[h], W[w]) along the pair axis.

    Algorithm 2 ([YL] §3.3.2): the time table is read at the global frame,
    the height and width tables at h and w, and the three are concatenated
    in that order.  Returns complex128 [n, D/2].
    """
    ft, fh, fw = tables
    return np.concatenate([ft[pos[:, 0]], fh[pos[:, 1]], fw[pos[:, 2]]], axis=1)


def rope3d_apply(x: np.ndarray, tables, pos: np.ndarray) -> np.ndarray:
    """Rotate x [B, n, heads, D] at positions pos [n, 4]; returns float64.

    Algorithm 2 ([YL] §3.3.2): view the last dim as complex numbers made of
    adjacent pairs in float64, multiply by the per-token factor (the same
    for every head), and view the product back as interleaved real pairs.
    """
    x = np.asarray(x, dtype=np.float64)
    b, n, nh, d = x.shape
    f = token_freqs(tables, pos)                       # [n, D/2]
    if f.shape[1] * 2 != d:
        raise ValueError("head_dim != d_t + d_h + d_w")
    xc = x.reshape(b, n, nh, d // 2, 2)
    xc = xc[..., 0] + 1j * xc[..., 1]                  # [B, n, heads, D/2]
    y = xc * f[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = y.real
    out[..., 1::2] = y.imag
    return out


def rope3d_apply_append(q, k, v, k_cache, v_cache, tables,
                        frames, height, width, start_frame, token_offset):
    """Causal-RoPE on a token slice, then the KV-cache write.

    [YL] Algorithm 3 steps 2, 3 and 5: positions from (Delta, s, H, W)
    with no other rank's data; q and k are rotated, v is not; the rotated k
    and the unrotated v overwrite the cache rows of these tokens.
    q, k, v: [B, n, heads, D]; k_cache, v_cache: [B, cache_tokens, heads, D]
    float64 arrays updated in place.  Returns the rotated q (float64).
    """
    n = q.shape[1]
    pos = positions(frames, height, width, start_frame, token_offset, n)
    q_rot = rope3d_apply(q, tables, pos)
    k_rot = rope3d_apply(k, tables, pos)
    rows = pos[:, 3]
    if n and rows[-1] >= k_cache.shape[1]:
        raise ValueError("cache too small")
    k_cache[:, rows] = k_rot
    v_cache[:, rows] = np.asarray(v, dtype=np.float64)
    return q_rot
