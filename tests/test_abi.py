"""The C-ABI library loads, exports every entry point include/rcc.h declares,
and rejects bad arguments on the host (no GPU needed: these calls return
before anything is launched)."""
import ctypes
import os
import re

import pytest

import rope_chunk_causal_amd as rcc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rcc.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"RCC_API\s+[\w\s\*]+?\b(rcc_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert set(_declared()) == set(rcc.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    if not os.path.exists(rcc.LIB_PATH):
        pytest.skip("librcc.so not built")
    lib = ctypes.CDLL(rcc.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert rcc.lib().rcc_status_string(rcc.RCC_ERR_RANGE) == b"RCC_ERR_RANGE"


def test_tables_size_is_host_only():
    cfg = rcc.rope_cfg(44, 42, 42, 1024, 64, 128)
    assert rcc.rope3d_tables_floats(cfg) == 1024 * 44 + 64 * 42 + 128 * 42
    with pytest.raises(rcc.RccError):
        rcc.rope3d_tables_floats(rcc.rope_cfg(43, 42, 42, 1024, 64, 128))


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Fake, aligned device addresses: every case below must fail a host check
# first, so nothing is ever launched with them.  Skipped where a GPU exists.
FAKE = 1 << 40


def _sealed(cfg, buf=FAKE, floats=None):
    """A tables descriptor from rcc_rope3d_tables_init (host only) over a fake
    buffer of exactly the cfg's size; zeroed if init rejects the cfg."""
    desc = rcc.rcc_rope3d_tables()
    n = rcc.lib().rcc_rope3d_tables_floats(ctypes.byref(cfg)) if floats is None else floats
    rcc.lib().rcc_rope3d_tables_init(ctypes.byref(cfg), buf, n, ctypes.byref(desc))
    return desc


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
@pytest.mark.parametrize("kw,status", [
    (dict(in_dtype=7), rcc.RCC_ERR_DTYPE),
    (dict(head_dim=24 + 4), rcc.RCC_ERR_SHAPE),
    (dict(head_dim=136), rcc.RCC_ERR_SHAPE),
    (dict(chunk_tokens=0), rcc.RCC_ERR_SHAPE),
    (dict(q_pos=70), rcc.RCC_ERR_RANGE),
    (dict(kv_tokens=97), rcc.RCC_ERR_RANGE),
    (dict(q=0), rcc.RCC_ERR_NULL),
    (dict(out=FAKE + 8), rcc.RCC_ERR_ALIGN),
    (dict(q_tokens=-1), rcc.RCC_ERR_SHAPE),
    (dict(scale=0.0), rcc.RCC_ERR_SHAPE),
    (dict(scale=-0.1), rcc.RCC_ERR_SHAPE),
    # valid sizes whose bf16 / head_dim-128 launch would exceed 2^32 work-items
    (dict(in_dtype=rcc.RCC_BF16, out_dtype=rcc.RCC_BF16, head_dim=128, batch=65535,
          n_heads=65535, q_tokens=512, q_pos=0, kv_tokens=512, chunk_tokens=512, cache=512),
     rcc.RCC_ERR_SHAPE),
])
def test_attn_host_checks(kw, status):
    a = dict(in_dtype=rcc.RCC_F32, out_dtype=rcc.RCC_F32, batch=1, n_heads=2, head_dim=24,
             q_tokens=32, q_pos=64, kv_tokens=96, chunk_tokens=32, scale=0.2, q=FAKE,
             k=FAKE, v=FAKE, cache=96, out=FAKE)
    a.update(kw)
    st = rcc.lib().rcc_chunk_causal_attn(
        a["in_dtype"], a["out_dtype"], a["batch"], a["n_heads"], a["head_dim"], a["q_tokens"],
        a["q_pos"], a["kv_tokens"], a["chunk_tokens"], a["scale"], a["q"], a["k"], a["v"],
        a["cache"], a["out"], None)
    assert st == status, rcc.lib().rcc_last_error()


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
@pytest.mark.parametrize("kw,status", [
    (dict(cfg=rcc.rope_cfg(8, 8, 7, 16, 4, 4)), rcc.RCC_ERR_SHAPE),     # odd band
    (dict(cfg=rcc.rope_cfg(8, 8, 4, 16, 4, 4)), rcc.RCC_ERR_SHAPE),     # D = 20, not 8k
    (dict(grid=rcc.grid(2, 4, 4, 15, 0)), rcc.RCC_ERR_RANGE),            # s + F > max_t
    (dict(grid=rcc.grid(2, 5, 4, 0, 0)), rcc.RCC_ERR_RANGE),             # H > max_h
    (dict(grid=rcc.grid(2, 4, 4, 0, 1)), rcc.RCC_ERR_RANGE),             # Delta + n > FHW
    (dict(grid=rcc.grid(2, 4, 4, -1, 0)), rcc.RCC_ERR_RANGE),            # s < 0
    (dict(grid=rcc.grid(0, 4, 4, 0, 0)), rcc.RCC_ERR_SHAPE),             # empty grid
    (dict(cache=95), rcc.RCC_ERR_RANGE),                                 # cache too small
    (dict(in_dtype=3), rcc.RCC_ERR_DTYPE),
    (dict(batch=0), rcc.RCC_ERR_SHAPE),
    (dict(v=0), rcc.RCC_ERR_NULL),
    (dict(k=FAKE + 4), rcc.RCC_ERR_ALIGN),
    (dict(q_out=FAKE, out_dtype=rcc.RCC_BF16), rcc.RCC_ERR_DTYPE),     # in-place, mixed dtype
])
def test_apply_host_checks(kw, status):
    a = dict(cfg=rcc.rope_cfg(8, 8, 8, 16, 4, 4), grid=rcc.grid(2, 4, 4, 4, 0),
             in_dtype=rcc.RCC_F32, out_dtype=rcc.RCC_F32, batch=1, n=32, nh=2,
             q=FAKE, k=FAKE, v=FAKE, q_out=FAKE + 4096, kc=FAKE, vc=FAKE, cache=96)
    a.update(kw)
    st = rcc.lib().rcc_rope3d_apply_append(
        ctypes.byref(_sealed(a["cfg"])), ctypes.byref(a["grid"]), a["in_dtype"], a["out_dtype"],
        a["batch"], a["n"], a["nh"], a["q"], a["k"], a["v"], a["q_out"], a["kc"], a["vc"],
        a["cache"], None)
    assert st == status, rcc.lib().rcc_last_error()


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
def test_positions_and_tables_host_checks():
    L = rcc.lib()
    g = rcc.grid(2, 4, 4, 0, 30)
    assert L.rcc_rope3d_positions(ctypes.byref(g), 3, FAKE, None) == rcc.RCC_ERR_RANGE
    assert L.rcc_rope3d_positions(ctypes.byref(g), 2, 0, None) == rcc.RCC_ERR_NULL
    assert L.rcc_rope3d_positions(ctypes.byref(g), 0, 0, None) == rcc.RCC_OK
    desc = rcc.rcc_rope3d_tables()
    bad = rcc.rope_cfg(8, 8, 8, 16, 4, 0)
    assert L.rcc_rope3d_tables_init(ctypes.byref(bad), FAKE, 1 << 20, ctypes.byref(desc)) == \
        rcc.RCC_ERR_SHAPE
    good = rcc.rope_cfg(8, 8, 8, 16, 4, 4)
    assert L.rcc_rope3d_tables_init(ctypes.byref(good), FAKE + 4, 1 << 20, ctypes.byref(desc)) == \
        rcc.RCC_ERR_ALIGN
    assert L.rcc_rope3d_tables_init(ctypes.byref(good), 0, 1 << 20, ctypes.byref(desc)) == \
        rcc.RCC_ERR_NULL
    assert L.rcc_rope3d_tables_init(ctypes.byref(good), FAKE, 1 << 20, None) == rcc.RCC_ERR_NULL
    assert L.rcc_rope3d_tables_build(None, None) == rcc.RCC_ERR_NULL
    # tables of more than 2^30 floats (kernels address them with 32-bit byte offsets)
    huge = rcc.rope_cfg(44, 42, 42, 1 << 26, 64, 128)
    assert L.rcc_rope3d_tables_floats(ctypes.byref(huge)) == -1
    assert L.rcc_rope3d_tables_init(ctypes.byref(huge), FAKE, 1 << 40, ctypes.byref(desc)) == \
        rcc.RCC_ERR_SHAPE
    edge = rcc.rope_cfg(2, 2, 2, (1 << 29) - 2, 1, 1)             # 2^30 floats: allowed
    assert L.rcc_rope3d_tables_floats(ctypes.byref(edge)) == 1 << 30
    over = rcc.rope_cfg(2, 2, 2, (1 << 29) - 1, 1, 1)             # 2^30 + 2 floats: refused
    assert L.rcc_rope3d_tables_floats(ctypes.byref(over)) == -1


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
def test_tables_descriptor_binds_its_cfg_to_its_buffer():
    """A descriptor is made only by init, for a buffer of at least the cfg's
    size; a call given a descriptor whose cfg, buffer or length changed
    afterwards, or one init never sealed, fails its host check and launches
    nothing (no GPU here: any launch would fail with RCC_ERR_HIP instead)."""
    L = rcc.lib()
    cfg = rcc.rope_cfg(8, 8, 8, 16, 4, 4)
    n = L.rcc_rope3d_tables_floats(ctypes.byref(cfg))
    assert n == 16 * 8 + 4 * 8 + 4 * 8
    desc = rcc.rcc_rope3d_tables()
    # a buffer one float short is refused, and the descriptor left unsealed
    assert L.rcc_rope3d_tables_init(ctypes.byref(cfg), FAKE, n - 1, ctypes.byref(desc)) == \
        rcc.RCC_ERR_SHAPE
    assert desc.seal == 0 and desc.data is None

    def apply(d, grid=rcc.grid(2, 4, 4, 4, 0), cache=96):
        return L.rcc_rope3d_apply_append(ctypes.byref(d), ctypes.byref(grid), rcc.RCC_F32,
                                         rcc.RCC_F32, 1, 32, 2, FAKE, FAKE, FAKE, FAKE + 4096,
                                         FAKE, FAKE, cache, None)

    def qkv(d):
        return L.rcc_qkv_rope_append(ctypes.byref(d), ctypes.byref(rcc.grid(2, 4, 4, 4, 0)), 1,
                                     32, 2, 64, FAKE, FAKE, None, FAKE, FAKE, FAKE, 96, None)

    assert apply(desc) == rcc.RCC_ERR_SHAPE            # never sealed
    assert L.rcc_rope3d_tables_build(ctypes.byref(desc), None) == rcc.RCC_ERR_SHAPE
    assert L.rcc_rope3d_tables_init(ctypes.byref(cfg), FAKE, n, ctypes.byref(desc)) == rcc.RCC_OK
    assert desc.floats == n and desc.data == FAKE and desc.cfg.max_t == 16
    # the sealed descriptor passes: these fail later, on the grid and cache checks
    assert apply(desc, grid=rcc.grid(2, 4, 4, 15, 0)) == rcc.RCC_ERR_RANGE   # s + F > max_t
    assert apply(desc, cache=95) == rcc.RCC_ERR_RANGE
    for field, value in (("max_t", 1024), ("max_h", 64), ("d_t", 16), ("theta", 500.0)):
        changed = rcc.rcc_rope3d_tables.from_buffer_copy(desc)
        setattr(changed.cfg, field, value)
        assert apply(changed) == rcc.RCC_ERR_SHAPE, field
        assert qkv(changed) == rcc.RCC_ERR_SHAPE, field
        assert L.rcc_rope3d_tables_build(ctypes.byref(changed), None) == rcc.RCC_ERR_SHAPE
    for field, value in (("floats", n - 1), ("floats", 1 << 30), ("data", FAKE + 4096)):
        changed = rcc.rcc_rope3d_tables.from_buffer_copy(desc)
        setattr(changed, field, value)
        assert apply(changed) == rcc.RCC_ERR_SHAPE, field
    # a larger buffer than needed is fine
    assert L.rcc_rope3d_tables_init(ctypes.byref(cfg), FAKE, n + 100, ctypes.byref(desc)) == \
        rcc.RCC_OK
    assert apply(desc, cache=95) == rcc.RCC_ERR_RANGE


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
@pytest.mark.parametrize("kw,status", [
    (dict(cfg=rcc.rope_cfg(8, 8, 8, 16, 4, 4)), rcc.RCC_ERR_SHAPE),     # D = 24, not 32k
    (dict(model_dim=40), rcc.RCC_ERR_SHAPE),                            # not 32k
    (dict(model_dim=48), rcc.RCC_ERR_SHAPE),
    (dict(model_dim=0), rcc.RCC_ERR_SHAPE),
    (dict(batch=0), rcc.RCC_ERR_SHAPE),
    (dict(nh=0), rcc.RCC_ERR_SHAPE),
    (dict(n=1 << 20, model_dim=4096), rcc.RCC_ERR_SHAPE),                # x >= 4 GiB
    (dict(grid=rcc.grid(2, 4, 4, 15, 0)), rcc.RCC_ERR_RANGE),            # s + F > max_t
    (dict(grid=rcc.grid(2, 4, 4, 0, 1)), rcc.RCC_ERR_RANGE),             # Delta + n > FHW
    (dict(cache=95), rcc.RCC_ERR_RANGE),
    (dict(x=0), rcc.RCC_ERR_NULL),
    (dict(w=FAKE + 8), rcc.RCC_ERR_ALIGN),
    (dict(bias=FAKE + 2), rcc.RCC_ERR_ALIGN),
])
def test_qkv_host_checks(kw, status):
    a = dict(cfg=rcc.rope_cfg(16, 8, 8, 16, 4, 4), grid=rcc.grid(2, 4, 4, 4, 0), batch=1, n=32,
             nh=2, model_dim=64, x=FAKE, w=FAKE, bias=None, q_out=FAKE, kc=FAKE, vc=FAKE,
             cache=96)
    a.update(kw)
    if "n" in kw:  # a long slice needs a grid and cache that hold it
        a["grid"] = rcc.grid(1, 1024, 1024, 0, 0)
        a["cfg"] = rcc.rope_cfg(16, 8, 8, 16, 1024, 1024)
        a["cache"] = a["n"]
    st = rcc.lib().rcc_qkv_rope_append(
        ctypes.byref(_sealed(a["cfg"])), ctypes.byref(a["grid"]), a["batch"], a["n"], a["nh"],
        a["model_dim"], a["x"], a["w"], a["bias"], a["q_out"], a["kc"], a["vc"], a["cache"],
        None)
    assert st == status, rcc.lib().rcc_last_error()


@pytest.mark.parametrize("F,H,W,s,sink,window,held", [
    (3, 2, 2, 0, 0, 21, 3 * 4),        # first chunk
    (3, 2, 2, 15, 0, 21, 18 * 4),      # still filling
    (3, 2, 2, 18, 0, 21, 21 * 4),      # exactly full
    (3, 2, 2, 99, 0, 21, 21 * 4),      # long after the ring wrapped
    (2, 3, 5, 0, 1, 4, 2 * 15),
    (2, 3, 5, 6, 1, 4, 5 * 15),
])
def test_ring_held_tokens(F, H, W, s, sink, window, held):
    assert rcc.ring_held_tokens(rcc.grid(F, H, W, s), rcc.ring(sink, window)) == held
    if H % 2 == 0:    # blockifying frames does not change what is held
        assert rcc.ring_held_tokens(rcc.grid(F, H, W, s), rcc.ring(sink, window, 2, 1)) == held


def test_ring_held_tokens_rejects_bad_rings():
    L = rcc.lib()
    g = rcc.grid(3, 2, 2, 0)
    for r in (rcc.ring(0, 2), rcc.ring(-1, 5), rcc.ring(1 << 30, 1 << 30), rcc.ring(0, 3, 2, 0),
              rcc.ring(0, 3, 0, 2), rcc.ring(0, 3, -2, 2), rcc.ring(0, 3, 2, 3)):
        assert L.rcc_ring_held_tokens(ctypes.byref(g), ctypes.byref(r)) == -1
    assert L.rcc_ring_held_tokens(ctypes.byref(g), None) == -1


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
@pytest.mark.parametrize("kw,status", [
    (dict(ring=None), rcc.RCC_ERR_NULL),
    (dict(ring=rcc.ring(0, 1)), rcc.RCC_ERR_SHAPE),                     # window < F
    (dict(ring=rcc.ring(-1, 4)), rcc.RCC_ERR_SHAPE),
    (dict(ring=rcc.ring(1, 3, 3, 4)), rcc.RCC_ERR_SHAPE),                # 3 does not divide 4
    (dict(cache=4 * 16 - 1), rcc.RCC_ERR_RANGE),                        # smaller than the ring
    (dict(grid=rcc.grid(2, 4, 4, 15, 0)), rcc.RCC_ERR_RANGE),            # s + F > max_t
    (dict(grid=rcc.grid(2, 4, 4, 0, 1)), rcc.RCC_ERR_RANGE),             # Delta + n > FHW
    (dict(k=0), rcc.RCC_ERR_NULL),
    (dict(q=FAKE + 4), rcc.RCC_ERR_ALIGN),
])
def test_apply_ring_host_checks(kw, status):
    # A chunk at frames 12..13 far past a 1-sink 3-window ring: its plain
    # cache rows would end at 14*16, but the ring needs only 4*16 rows.
    a = dict(cfg=rcc.rope_cfg(8, 8, 8, 16, 4, 4), grid=rcc.grid(2, 4, 4, 12, 0),
             ring=rcc.ring(1, 3), q=FAKE, k=FAKE, v=FAKE, cache=4 * 16)
    a.update(kw)
    L = rcc.lib()
    ring = ctypes.byref(a["ring"]) if a["ring"] is not None else None
    st = L.rcc_rope3d_apply_append_ring(
        ctypes.byref(_sealed(a["cfg"])), ctypes.byref(a["grid"]), ring, rcc.RCC_F32,
        rcc.RCC_F32, 1, 32, 2, a["q"], a["k"], a["v"], FAKE + 4096, FAKE, FAKE, a["cache"],
        None)
    assert st == status, L.rcc_last_error()
    if "q" not in kw and "k" not in kw:
        # the fused projection applies the same ring rules (D = 32 here)
        cfg = rcc.rope_cfg(16, 8, 8, 16, 4, 4)
        st = L.rcc_qkv_rope_append_ring(
            ctypes.byref(_sealed(cfg)), ctypes.byref(a["grid"]), ring, 1, 32, 2, 64, FAKE, FAKE,
            None, FAKE, FAKE, FAKE, a["cache"], None)
        assert st == status, L.rcc_last_error()


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
def test_ring_positions_and_attention_host_checks():
    L = rcc.lib()
    g, r = rcc.grid(2, 4, 4, 12, 0), rcc.ring(1, 3)
    assert L.rcc_ring_positions(ctypes.byref(g), ctypes.byref(r), 33, FAKE, None) == \
        rcc.RCC_ERR_RANGE
    assert L.rcc_ring_positions(ctypes.byref(g), None, 8, FAKE, None) == rcc.RCC_ERR_NULL
    assert L.rcc_ring_positions(ctypes.byref(g), ctypes.byref(r), 0, 0, None) == rcc.RCC_OK

    def attn(grid, ring, q_tokens=32, cache=64, head_dim=24, out=FAKE):
        return L.rcc_chunk_causal_attn_ring(
            ctypes.byref(grid), ring and ctypes.byref(ring), rcc.RCC_F32, rcc.RCC_F32, 1, 2,
            head_dim, q_tokens, 0.2, FAKE, FAKE, FAKE, cache, out, None)
    assert attn(g, None) == rcc.RCC_ERR_NULL
    assert attn(g, rcc.ring(0, 1)) == rcc.RCC_ERR_SHAPE
    assert attn(g, r, q_tokens=33) == rcc.RCC_ERR_RANGE               # more than the chunk
    assert attn(g, r, cache=63) == rcc.RCC_ERR_RANGE                  # ring holds 64 rows
    assert attn(g, r, head_dim=20) == rcc.RCC_ERR_SHAPE
    assert attn(g, r, out=FAKE + 8) == rcc.RCC_ERR_ALIGN
    assert attn(g, r, q_tokens=0) == rcc.RCC_OK


@pytest.mark.skipif(_gpu_present(), reason="host-check cases use fake pointers; CPU only")
@pytest.mark.parametrize("kw,status", [
    (dict(in_dtype=rcc.RCC_F32), rcc.RCC_ERR_DTYPE),
    (dict(out_dtype=5), rcc.RCC_ERR_DTYPE),
    (dict(head_dim=64), rcc.RCC_ERR_SHAPE),
    (dict(block=40), rcc.RCC_ERR_SHAPE),
    (dict(block=96), rcc.RCC_ERR_SHAPE),
    (dict(block=512), rcc.RCC_ERR_SHAPE),
    (dict(n_p=600, n_l=425), rcc.RCC_ERR_SHAPE),             # more than 1024 entries
    (dict(kv=32768 * 32 + 32, cache=1 << 21, block=32), rcc.RCC_ERR_SHAPE),  # > 32768 blocks
    (dict(kv=1025), rcc.RCC_ERR_RANGE),                      # beyond the cache
    (dict(scale=0.0), rcc.RCC_ERR_SHAPE),
    (dict(n_l=-1), rcc.RCC_ERR_SHAPE),
    (dict(persist=0), rcc.RCC_ERR_NULL),
    (dict(local=FAKE + 2), rcc.RCC_ERR_ALIGN),
    (dict(out=FAKE + 8), rcc.RCC_ERR_ALIGN),
    (dict(q_tokens=0, q=0), rcc.RCC_OK),                     # nothing to do
    # valid sizes whose launch grid would exceed 2^32 work-items
    (dict(batch=1024, nh=1024, q_tokens=1024 * 256, block=256, n_p=0, n_l=0), rcc.RCC_ERR_SHAPE),
    (dict(batch=1024, nh=1024, q_tokens=1024 * 48, kv=960, block=48, n_p=0, n_l=0),
     rcc.RCC_ERR_SHAPE),
])
def test_block_sparse_host_checks(kw, status):
    a = dict(in_dtype=rcc.RCC_BF16, out_dtype=rcc.RCC_BF16, batch=1, nh=2, head_dim=128,
             q_tokens=128, kv=1024, block=64, scale=0.1, q=FAKE, cache=1024, persist=FAKE,
             n_p=3, local=FAKE, n_l=4, out=FAKE)
    a.update(kw)
    st = rcc.lib().rcc_block_sparse_attn(
        a["in_dtype"], a["out_dtype"], a["batch"], a["nh"], a["head_dim"], a["q_tokens"], a["kv"],
        a["block"], a["scale"], a["q"], FAKE, FAKE, a["cache"], a["persist"], a["n_p"],
        a["local"], a["n_l"], a["out"], None)
    assert st == status, rcc.lib().rcc_last_error()


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "rcc.h"

int main(void) {
  rcc_rope3d_cfg cfg = {44, 42, 42, 10000.0, 1024, 64, 128};
  rcc_grid g = {3, 30, 52, 6, 0};
  rcc_ring ring = {0, 21, 0, 0};
  rcc_rope3d_tables tab;
  long long floats = (long long)rcc_rope3d_tables_floats(&cfg);
  long long held = (long long)rcc_ring_held_tokens(&g, &ring);
  rcc_status st = rcc_chunk_causal_attn(RCC_BF16, RCC_BF16, 1, 12, 128, 4680, 9360, 14040,
                                        4680, 0.0883883f, NULL, NULL, NULL, 14040, NULL, NULL);
  /* a descriptor over a fake (never touched) device address, then changed */
  rcc_status init = rcc_rope3d_tables_init(&cfg, (float*)(size_t)0x10000000000ull, floats, &tab);
  tab.cfg.max_t = 4096;
  rcc_status changed = rcc_rope3d_apply_append(&tab, &g, RCC_BF16, RCC_BF16, 1, 4680, 12,
                                               NULL, NULL, NULL, NULL, NULL, NULL, 14040, NULL);
  printf("%lld %lld %s %d %s %s\n", floats, held, rcc_status_string(st),
         (int)(strlen(rcc_last_error()) > 0), rcc_status_string(init),
         rcc_status_string(changed));
  return 0;
}
"""


def test_header_compiles_as_c99_and_links():
    """A plain C99 program includes rcc.h, links librcc.so and makes host-only
    calls (sizes, ring rows, an argument error, a tables descriptor rejected
    after its cfg changed): the boundary needs no C++."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(rcc.LIB_PATH):
        pytest.skip("gcc or librcc.so missing")
    work = os.path.join(ROOT, "rope_chunk_causal_amd", "_build", "ctest")
    os.makedirs(work, exist_ok=True)
    src, exe = os.path.join(work, "abi.c"), os.path.join(work, "abi")
    with open(src, "w") as f:
        f.write(C_PROGRAM)
    libdir = os.path.dirname(rcc.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", src,
                        "-L", libdir, "-lrcc", "-Wl,-rpath," + libdir, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "rcc.h" not in r.stderr, r.stderr       # no warnings from our header
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    floats, held, status, has_detail, init, changed = out.stdout.split()
    assert int(floats) == 2 * (1024 * 22 + 64 * 21 + 128 * 21)
    assert int(held) == 9 * 1560
    assert status == "RCC_ERR_NULL" and has_detail == "1"
    assert init == "RCC_OK" and changed == "RCC_ERR_SHAPE"
