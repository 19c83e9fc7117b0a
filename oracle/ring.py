"""fp64 oracle: a rolling-window KV cache indexed by global time.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy float64.

[YL] §2.1 credits Self-Forcing's KV caching with a rolling window for
rollouts of any length.  [SF] (Sparse Forcing: Native Trainable Sparse
Attention for Real-time Autoregressive Diffusion Video Generation) §3.2
shows why a full cache cannot scale (tens of GB for a minute of video) and
§3.3 keeps a bounded memory made of sink blocks that persist plus a local
window of the most recent blocks; §4.3 compares a plain sliding window with
sink frames under the same KV budget.  Neither page fixes the storage, so
the readings taken here are:

* The cache holds ``sink`` frames that never leave (global frames
  0 .. sink-1, the sink frames of [SF] §4.3) and the ``window`` most recent
  frames after them.  ``sink = 0`` is the plain rolling window.  Every
  frame's K rows keep the rotation of their global time index: frames are
  never re-rotated when older ones leave ([YL] §3.3.2 item 1 fixes the time
  index of a block by its global position, and the rotary factors make
  q.k depend on the difference of the two global indices only).
* After the chunk of frames [s, s+F) is written, the cache holds the sink
  frames below s+F and the last ``window`` frames that end at s+F-1; the
  chunk attends to all of them (it is the newest block, so block-causal
  visibility removes nothing else).  window >= F: a chunk never evicts
  its own frames.
* Storage is a ring: frame t lives in frame slot t if t < sink, else in
  slot sink + (t - sink) mod window; token (h, w) of the frame is row
  slot * H*W + h*W + w of a cache of (sink + window) * H*W rows.
* Optionally the tokens of a frame are stored block-contiguously ([SF]
  §3.3 blockify, with blocks of (1, B_h, B_w): one frame deep): the
  frame's (H/B_h) x (W/B_w) blocks in row-major order, each block's B_h x B_w
  tokens in row-major order, so block j of a frame is rows
  [j B_h B_w, (j+1) B_h B_w) of its slot.  B_h and B_w divide H and W.
"""
from __future__ import annotations

import numpy as np

from . import rope3d


def _check(frames: int, sink: int, window: int):
    if sink < 0 or window < 1:
        raise ValueError("need sink >= 0 and window >= 1")
    if window < frames:
        raise ValueError("the window must hold a whole chunk (window >= frames)")


def frame_slot(t, sink: int, window: int):
    """Ring slot of global frame t (reading in the module header)."""
    t = np.asarray(t, dtype=np.int64)
    return np.where(t < sink, t, sink + np.mod(t - sink, window))


def held_frames(frames: int, start_frame: int, sink: int, window: int) -> np.ndarray:
    """Global frames in the cache once chunk [s, s+F) is written, ascending.

    The sink frames below s+F, then the most recent ``window`` frames
    ending at s+F-1 ([SF] §3.3: persistent sink blocks plus a local window
    of the newest blocks).
    """
    _check(frames, sink, window)
    end = start_frame + frames
    lo = max(sink, end - window)
    return np.concatenate([np.arange(min(sink, end), dtype=np.int64),
                           np.arange(lo, end, dtype=np.int64)])


def frame_row(h, w, height: int, width: int, block_h: int = 0, block_w: int = 0):
    """Row of token (h, w) inside its frame slot: h*W + w, or, blockified,
    (block index, row-major over the frame's blocks) * B_h B_w + (row-major
    index inside the block)."""
    h = np.asarray(h, dtype=np.int64)
    w = np.asarray(w, dtype=np.int64)
    if not block_h and not block_w:
        return h * width + w
    if block_h <= 0 or block_w <= 0 or height % block_h or width % block_w:
        raise ValueError("block dims must be positive and divide the frame")
    block = (h // block_h) * (width // block_w) + w // block_w
    return block * (block_h * block_w) + (h % block_h) * block_w + w % block_w


def positions(frames: int, height: int, width: int, start_frame: int, token_offset: int,
              n_tokens: int, sink: int, window: int, block_h: int = 0,
              block_w: int = 0) -> np.ndarray:
    """(t_global, h, w, ring_row) of tokens token_offset .. +n_tokens-1.

    t, h, w are those of ``rope3d.positions`` ([YL] §3.3.3: global time index
    from the start frame and the slice offset); the row is the token's row in
    the ring: frame_slot(t) * H*W + frame_row(h, w).
    """
    _check(frames, sink, window)
    pos = rope3d.positions(frames, height, width, start_frame, token_offset, n_tokens).copy()
    pos[:, 3] = (frame_slot(pos[:, 0], sink, window) * (height * width)
                 + frame_row(pos[:, 1], pos[:, 2], height, width, block_h, block_w))
    return pos


def rope3d_apply_append(q, k, v, k_ring, v_ring, tables, frames, height, width,
                        start_frame, token_offset, sink, window, block_h=0, block_w=0):
    """Causal-RoPE on a token slice, then the write into the ring.

    [YL] Algorithm 3 steps 2, 3 and 5 with the cache row replaced by the
    ring row: q and k are rotated at their global (t, h, w), v is not; the
    rotated k and the unrotated v overwrite the ring rows of these tokens
    (evicting whatever frame held those slots).  k_ring, v_ring:
    [B, (sink + window) * H*W, heads, D] float64, updated in place.
    Returns the rotated q.
    """
    n = q.shape[1]
    pos = positions(frames, height, width, start_frame, token_offset, n, sink, window,
                    block_h, block_w)
    if k_ring.shape[1] < (sink + window) * height * width:
        raise ValueError("ring smaller than (sink + window) frames")
    k_ring[:, pos[:, 3]] = rope3d.rope3d_apply(k, tables, pos)
    v_ring[:, pos[:, 3]] = np.asarray(v, dtype=np.float64)
    return rope3d.rope3d_apply(q, tables, pos)


def held_rows(frames: int, height: int, width: int, start_frame: int,
              sink: int, window: int) -> np.ndarray:
    """Ring rows of every held frame, frames in ascending global order."""
    hw = height * width
    f = held_frames(frames, start_frame, sink, window)
    return (frame_slot(f, sink, window)[:, None] * hw + np.arange(hw)[None, :]).reshape(-1)


def ring_attention(q, k_ring, v_ring, frames, height, width, start_frame, sink, window,
                   scale, rows=None, block=256):
    """softmax(scale * q K_M^T) V_M over the held memory M, float64.

    [YL] Algorithm 3 step 6 with the cache replaced by the memory the ring
    holds after the chunk's write ([SF] §3.3: K and V are the stacked rows
    of the held blocks).  Every query of the chunk sees every held row.
    q: [B, Lq, heads, D]; returns [B, len(rows), heads, D].
    """
    q = np.asarray(q, dtype=np.float64)
    b, lq, nh, d = q.shape
    rows = np.arange(lq) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = held_rows(frames, height, width, start_frame, sink, window)
    out = np.empty((b, len(rows), nh, d))
    for bi in range(b):
        for h in range(nh):
            kh = np.asarray(k_ring[bi, keys, h, :], dtype=np.float64)
            vh = np.asarray(v_ring[bi, keys, h, :], dtype=np.float64)
            for r0 in range(0, len(rows), block):
                rb = rows[r0:r0 + block]
                s = scale * (q[bi, rb, h, :] @ kh.T)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                out[bi, r0:r0 + len(rb), h, :] = p @ vh
    return out
