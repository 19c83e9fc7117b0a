"""Host logic of bench.py and of the seeded block lists (CPU only).

* ``--gpus`` above 1 is refused before anything touches a GPU.
* The attention source hash that keys the committed traffic profile ignores
  comments and whitespace, and ``read_traffic`` reports bytes only while the
  profile's hash matches.
* ``synth.block_lists`` draws lists that follow the workloads' recipe: the
  persistent list a permutation of the persistent blocks, each query block's
  local list its own (diagonal) block first, then distinct window blocks.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rope_chunk_causal_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_code_only_drops_comments_and_whitespace():
    a = "int a = 1;  // note\n/* block\n comment */\nint b;\n"
    b = "int a = 1;\n\n   int b;"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")


def test_traffic_needs_the_profile_hash(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    prof = tmp_path / "profiles" / "k_hbm_traffic.txt"
    prof.write_text("# comment = ignored\nsource_hash = abc\nbytes_per_launch = 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.read_traffic("k") == 1234.0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abd")
    assert bench.read_traffic("k") is None
    assert bench.read_traffic("missing") is None


def test_committed_traffic_profile_matches_the_sources():
    assert bench.read_traffic("chunk_causal_attn_480p_step") is not None


@pytest.mark.parametrize("name", sorted(synth.SPARSE_WORKLOADS) + sorted(synth.SPARSE_WORKLOADS_344))
def test_block_lists_follow_the_recipe(name):
    w = {**synth.SPARSE_WORKLOADS, **synth.SPARSE_WORKLOADS_344}[name]
    persist, local = synth.block_lists(w, 7)
    assert persist.shape == (w.batch, w.n_heads, w.n_persist) and persist.dtype == np.int32
    assert local.shape == (w.batch, w.n_heads, w.q_blocks, w.top_k) and local.dtype == np.int32
    own0 = w.n_persist + w.n_window - w.q_blocks
    for b in range(w.batch):
        for h in range(w.n_heads):
            assert sorted(persist[b, h]) == list(range(w.n_persist))
            for i in range(w.q_blocks):
                lst = local[b, h, i]
                assert lst[0] == own0 + i
                assert len(set(lst.tolist())) == w.top_k
                assert lst.min() >= w.n_persist and lst.max() < w.n_persist + w.n_window
    # the memory the lists index is whole blocks of the workload's cache
    assert w.kv_tokens == (w.n_persist + w.n_window) * w.block
    assert w.q_tokens == w.q_blocks * w.block
