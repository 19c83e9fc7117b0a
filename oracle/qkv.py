"""fp64 oracle: the local QKV projection fused with Causal-RoPE and the cache write.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy float64.

[YL] Algorithm 3 step 1 projects the rank's token slice x to q, k, v before
the positions and the rotation of steps 2-3, and §3.4.1 item 3 fuses that
projection with Causal-RoPE into one kernel.  The pages do not define QKV
further; the reading taken here:

* QKV is one linear map applied per token: y = x W^T (+ b), with W the
  rows of the q, k and v projections stacked in that order, each
  [heads * head_dim, model_dim] with rows head-major then head_dim (the
  usual fused projection layout).  The bias is optional.
* q, k, v are the three row groups of y viewed as [B, n, heads, head_dim];
  everything after that is ``rope3d.rope3d_apply_append``.
"""
from __future__ import annotations

import numpy as np

from . import rope3d


def qkv_project(x, w_qkv, bias, n_heads: int, head_dim: int):
    """q, k, v = split(x W^T + b); returns three float64 [B, n, heads, D].

    x: [B, n, model_dim]; w_qkv: [3 * heads * D, model_dim]; bias: None or
    [3 * heads * D].  [YL] Algorithm 3 step 1 (reading in the module header).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_qkv, dtype=np.float64)
    hd = n_heads * head_dim
    if w.shape != (3 * hd, x.shape[-1]):
        raise ValueError("w_qkv must be [3 * heads * head_dim, model_dim]")
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    b, n = x.shape[:2]
    return tuple(y[..., i * hd:(i + 1) * hd].reshape(b, n, n_heads, head_dim) for i in range(3))


def qkv_rope_append(x, w_qkv, bias, n_heads: int, head_dim: int, k_cache, v_cache, tables,
                    frames, height, width, start_frame, token_offset):
    """Projection, then Causal-RoPE and the KV-cache write of the slice.

    [YL] Algorithm 3 steps 1-3 and 5 for the slice that starts at chunk index
    token_offset (= r * L_local): q, k, v from ``qkv_project``, positions
    from (Delta, s, H, W), q and k rotated, the rotated k and the unrotated v
    written to the cache rows of these tokens.  Returns the rotated q.
    """
    q, k, v = qkv_project(x, w_qkv, bias, n_heads, head_dim)
    return rope3d.rope3d_apply_append(q, k, v, k_cache, v_cache, tables,
                                      frames, height, width, start_frame, token_offset)
