"""fp64 oracle: block-sparse attention over a persistent + local block memory.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy float64.

[SF] (Sparse Forcing: Native Trainable Sparse Attention for Real-time
Autoregressive Diffusion Video Generation) §3.3 keeps a KV memory of whole
spatiotemporal blocks stored block-contiguously (blockify: B tokens per
block, each block's tokens adjacent).  The memory seen at a step is the
persistent set P (sink blocks plus blocks chosen from history) together
with the local window L, K = [K_P; K_L]; inside the local window each
query block q keeps only its Top-K blocks Omega(q).  §3.4 wants one kernel
that attends each query block to P and to its own Omega(q).  How P and
Omega are chosen (block scores, Top-C, Top-K) needs trained weights and is
not part of this computation: the block lists are inputs.  Readings:

* Query block i is query rows [i*B, (i+1)*B) (the last one may be short);
  key block j is cache rows [j*B, (j+1)*B), and only whole blocks inside
  the first kv_tokens rows exist (j < kv_tokens // B).
* The persistent list is per (batch, head), shared by every query block;
  the local lists are per (batch, head, query block).
* Query block i attends the union of the two lists: an index listed twice
  counts once, and entries outside [0, kv_tokens // B) (-1 pads a list)
  are ignored.  Every query of the block sees every key of the union
  (the selection is the mask; no other causal rule applies inside it).
* softmax(scale * q k^T) v over those keys; a query block whose union is
  empty gets zeros.
"""
from __future__ import annotations

import numpy as np


def key_blocks(persist, local, n_kblocks: int) -> np.ndarray:
    """Sorted union of the valid block indices of the two lists."""
    ids = np.concatenate([np.asarray(persist, dtype=np.int64).reshape(-1),
                          np.asarray(local, dtype=np.int64).reshape(-1)])
    ids = ids[(ids >= 0) & (ids < n_kblocks)]
    return np.unique(ids)


def block_sparse_attention(q, k_cache, v_cache, kv_tokens: int, block: int, persist, local,
                           scale: float) -> np.ndarray:
    """Attention of every query block over its persistent + local key blocks.

    q: [B, n_q, heads, D]; caches [B, >= kv_tokens, heads, D];
    persist: int [B, heads, n_p]; local: int [B, heads, ceil(n_q / block), n_l].
    Returns float64 [B, n_q, heads, D] ([SF] §3.3 memory M = P u L with the
    local Top-K selection Omega(q); reading in the module header).
    """
    q = np.asarray(q, dtype=np.float64)
    b, n_q, nh, d = q.shape
    n_qb = -(-n_q // block)
    n_kb = kv_tokens // block
    persist = np.asarray(persist)
    local = np.asarray(local)
    if persist.shape[:2] != (b, nh) or local.shape[:3] != (b, nh, n_qb):
        raise ValueError("persist must be [B, heads, n_p] and local [B, heads, n_qblocks, n_l]")
    out = np.zeros((b, n_q, nh, d))
    for bi in range(b):
        for h in range(nh):
            for i in range(n_qb):
                blocks = key_blocks(persist[bi, h], local[bi, h, i], n_kb)
                if blocks.size == 0:
                    continue
                rows = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
                kh = np.asarray(k_cache[bi, rows, h, :], dtype=np.float64)
                vh = np.asarray(v_cache[bi, rows, h, :], dtype=np.float64)
                qr = slice(i * block, min((i + 1) * block, n_q))
                s = scale * (q[bi, qr, h, :] @ kh.T)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                out[bi, qr, h, :] = p @ vh
    return out
