"""CPU fp64 oracle for the Causal-RoPE SP hot path — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and
it shares no code with the GPU library: it imports numpy only.

It is the plain definition of what the path computes, written from

  [YL] C. Yuan, P. Li, "Accelerating Video Generation Inference with
       Sequential-Parallel 3D Positional Encoding Using a Global Time
       Index" (arXiv 2603.06664),

section by section:

* ``rope3d``    — per-axis frequency tables (§3.3.1, Algorithm 2 ``freqs``),
                  global time index and local index derivation (§3.3.2
                  item 1, §3.3.3, Algorithm 3 step 3), the complex-multiply
                  rotation (§3.3.1 equation, §3.3.2 item 2, Algorithm 2) and
                  the KV-cache write (Algorithm 3 step 5).
* ``attention`` — attention of a query chunk over the cache (Algorithm 3
                  step 6) with the block-causal visibility rule (§3.2,
                  §3.3 block-wise autoregression).
* ``qkv``       — the local QKV projection (Algorithm 3 step 1) followed by
                  Causal-RoPE and the cache write: the fusion of §3.4.1
                  item 3.
* ``ring``      — a rolling-window KV cache (sink frames plus the most
                  recent window of frames, stored as a ring) indexed by the
                  global time index, and attention over what it holds
                  ([YL] §2.1; [SF] §3.2-3.3, §4.3, where [SF] is "Sparse
                  Forcing: Native Trainable Sparse Attention for Real-time
                  Autoregressive Diffusion Video Generation").
* ``block_sparse`` — attention of each query block over the union of a
                  persistent block list and its own local block list
                  ([SF] §3.3-3.4; the selection is an input).

Every function here is pinned by the ``-m "not gpu"`` tests against facts
fixed by the pages or by mathematics (closed forms, invariants, brute force
on tiny inputs, library special cases); none is "parity unpinned".
"""
from . import rope3d, attention, qkv, ring, block_sparse  # noqa: F401
