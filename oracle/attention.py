"""fp64 oracle: chunk-causal attention of a query chunk over the KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  [YL] is Yuan & Li,
"Accelerating Video Generation Inference with Sequential-Parallel 3D
Positional Encoding Using a Global Time Index" (arXiv 2603.06664).

Readings taken where the pages leave a step open:

* Visibility is block (chunk) causal: a query sees every key of its own
  chunk and of every earlier chunk, and no later one.  §3.2 requires that
  a token attend only to earlier context, and §3.3 generates block-wise,
  one chunk of tau latent frames at a time.  The chunk of cache row j is
  floor(j / C) with C = F*H*W tokens.
* The softmax scale is given by the caller (1/sqrt(head_dim) in every
  workload).
"""
from __future__ import annotations

import numpy as np


def visible(q_rows: np.ndarray, q_pos: int, kv_len: int,
            chunk_tokens: int) -> np.ndarray:
    """Boolean [len(q_rows), kv_len]: may query q_rows[i] read key j?

    Query row i sits at cache position q_pos + i.  Key j is visible iff
    j < kv_len and chunk(j) <= chunk(q_pos + i).
    """
    qc = (q_pos + np.asarray(q_rows, dtype=np.int64)) // chunk_tokens
    kc = np.arange(kv_len, dtype=np.int64) // chunk_tokens
    return kc[None, :] <= qc[:, None]


def chunk_causal_attention(q, k_cache, v_cache, q_pos: int, kv_len: int,
                           chunk_tokens: int, scale: float,
                           rows=None, block: int = 256) -> np.ndarray:
    """O = softmax(scale * Q K^T + mask) V per batch and head, float64.

    [YL] Algorithm 3 step 6: the queries attend to the keys and values read
    back from the cache.  q: [B, Lq, heads, D]; k_cache, v_cache:
    [B, >=kv_len, heads, D].  ``rows`` optionally restricts the output to a
    subset of query rows (returned in that order); rows are processed in
    blocks of ``block`` so memory stays bounded.  Returns [B, len(rows),
    heads, D].
    """
    q = np.asarray(q, dtype=np.float64)
    b, lq, nh, d = q.shape
    if rows is None:
        rows = np.arange(lq, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((b, len(rows), nh, d), dtype=np.float64)
    for bi in range(b):
        for h in range(nh):
            kh = np.asarray(k_cache[bi, :kv_len, h, :], dtype=np.float64)
            vh = np.asarray(v_cache[bi, :kv_len, h, :], dtype=np.float64)
            for r0 in range(0, len(rows), block):
                rb = rows[r0:r0 + block]
                s = scale * (q[bi, rb, h, :] @ kh.T)          # [rb, kv_len]
                s = np.where(visible(rb, q_pos, kv_len, chunk_tokens), s, -np.inf)
                s = s - s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                out[bi, r0:r0 + len(rb), h, :] = p @ vh
    return out
