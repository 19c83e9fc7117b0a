"""GPU parity: block_sparse_attn vs ``oracle.block_sparse``.

Seeded bf16 N(0,1) q, k, v; block lists drawn with padding (-1), repeats and
out-of-range entries mixed in, so the kernel's union has to drop them.
Every case is compared in full: the small ones (ragged last query block,
every block size) and the Sparse Forcing-shaped workloads (every row of
every head).  Attention bar: max 2e-2 / mean 2e-3 (rel L2 1e-2).  Also: every block
selected equals the dense kernel; empty unions give exact zeros; list order
and padding leave the output bit-identical.
"""
import math

import numpy as np
import pytest

import rope_chunk_causal_amd as rcc
from gpu_util import check_attn, say, to_dev, to_host_f64, torch
from oracle import block_sparse as S
from rope_chunk_causal_amd import synth

pytestmark = pytest.mark.gpu


def _messy_lists(seed, B, nh, n_qb, n_kb, n_p, n_l):
    g = np.random.Generator(np.random.PCG64(seed))
    persist = g.integers(-1, n_kb + 3, size=(B, nh, n_p)).astype(np.int32)
    local = g.integers(-2, n_kb + 3, size=(B, nh, n_qb, n_l)).astype(np.int32)
    if n_l > 1:
        local[..., -1] = local[..., 0]                   # a repeat in every list
    return persist, local


def _run(B, nh, n_q, kv, cap, blk, n_p, n_l, seed, out_dtype="bf16", lists=None):
    t = torch()
    D = 128
    qb = synth.normal((B, n_q, nh, D), seed, "bf16")
    kb = synth.normal((B, cap, nh, D), seed + 1, "bf16")
    vb = synth.normal((B, cap, nh, D), seed + 2, "bf16")
    n_qb = -(-n_q // blk)
    persist, local = lists if lists is not None else _messy_lists(seed + 3, B, nh, n_qb, kv // blk,
                                                                  n_p, n_l)
    dq, dk, dv = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    odt = t.bfloat16 if out_dtype == "bf16" else t.float32
    out = t.full((B, n_q, nh, D), float("nan"), dtype=odt, device="cuda")
    dp = t.from_numpy(persist).cuda() if persist.shape[-1] else None
    dl = t.from_numpy(local).cuda() if local.shape[-1] else None
    say("block_sparse", B, nh, n_q, kv, cap, blk, persist.shape, local.shape, out_dtype)
    rcc.block_sparse_attn(dq, dk, dv, out, kv, blk, dp, dl, 1.0 / math.sqrt(D))
    t.cuda.synchronize()
    return out, (qb, kb, vb), (persist, local)


@pytest.mark.parametrize("B,nh,n_q,kv,cap,blk,n_p,n_l,out_dtype", [
    (1, 2, 150, 640, 700, 64, 2, 3, "bf16"),     # ragged last query block, spare cache rows
    (2, 3, 64, 1024, 1024, 32, 4, 6, "bf16"),
    (1, 2, 300, 1280, 1300, 128, 1, 4, "f32"),
    (1, 1, 512, 2560, 2560, 256, 3, 2, "bf16"),
    (1, 2, 128, 4096, 4096, 64, 0, 9, "bf16"),   # local lists only
    (1, 2, 128, 4096, 4096, 64, 7, 0, "bf16"),   # persistent list only
    (1, 2, 150, 960, 1000, 48, 2, 3, "bf16"),    # [3,4,4] blocks of 48; ragged last query block
    (2, 3, 96, 1440, 1440, 48, 4, 6, "f32"),     # 48-row blocks, two batch entries
    (1, 2, 480, 4800, 4800, 48, 0, 9, "bf16"),   # 48-row blocks, local lists only, 10 blocks
])
def test_small_shapes_every_row(B, nh, n_q, kv, cap, blk, n_p, n_l, out_dtype):
    out, (qb, kb, vb), (persist, local) = _run(B, nh, n_q, kv, cap, blk, n_p, n_l, 31, out_dtype)
    ref = S.block_sparse_attention(synth.to_f64(qb, "bf16"), synth.to_f64(kb, "bf16"),
                                   synth.to_f64(vb, "bf16"), kv, blk, persist, local,
                                   1.0 / math.sqrt(128))
    got = to_host_f64(out)
    empty = ~np.abs(ref).any(axis=-1)
    assert np.array_equal(got[empty], ref[empty])       # empty unions: exact zeros
    check_attn(got, ref, f"sparse B{B} q{n_q} kv{kv} blk{blk}")


@pytest.mark.parametrize("blk", [64, 48])
def test_every_block_selected_matches_the_dense_kernel(blk):
    t = torch()
    nh, n_q, kv = 2, 4 * blk, 32 * blk
    n_kb = kv // blk
    persist = np.tile(np.arange(0, n_kb, 2, dtype=np.int32), (1, nh, 1))
    local = np.tile(np.arange(1, n_kb, 2, dtype=np.int32), (1, nh, n_q // blk, 1))
    out, (qb, kb, vb), _ = _run(1, nh, n_q, kv, kv, blk, 0, 0, 41, lists=(persist, local))
    dq, dk, dv = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    dense = t.empty_like(out)
    rcc.chunk_causal_attn(dq, dk, dv, dense, kv - n_q, kv, n_q, 1.0 / math.sqrt(128))
    t.cuda.synchronize()
    # The dense kernel rounds q * scale * log2(e) to bf16 where the block-sparse
    # kernel rounds q, so the two differ by about the bf16 rounding of the
    # scores (each meets the oracle bar on its own in the tests above).
    check_attn(to_host_f64(out), to_host_f64(dense), "sparse vs dense kernel",
               max_abs=4e-3, mean_abs=4e-4, rel_l2=1e-2)


@pytest.mark.parametrize("blk", [64, 48])
def test_empty_selection_gives_zeros(blk):
    t = torch()
    persist = np.full((1, 2, 3), -1, dtype=np.int32)
    local = np.array([[[[99, -1]], [[4, 5]]]], dtype=np.int32).reshape(1, 2, 1, 2)
    out, _, _ = _run(1, 2, blk, 5 * blk, 5 * blk, blk, 0, 0, 51, lists=(persist, local))
    assert bool((out[:, :, 0] == 0).all())              # head 0: nothing valid
    assert bool(t.isfinite(out).all())


@pytest.mark.parametrize("blk", [64, 48])
def test_list_order_and_padding_do_not_change_bits(blk):
    t = torch()
    B, nh, n_q, kv = 1, 2, 3 * blk, 24 * blk
    g = np.random.Generator(np.random.PCG64(61))
    persist = g.choice(24, size=(B, nh, 4), replace=False).astype(np.int32)
    local = np.stack([np.stack([g.choice(24, 5, replace=False) for _ in range(3)])
                      for _ in range(nh)])[None].astype(np.int32)
    a, _, _ = _run(B, nh, n_q, kv, kv, blk, 0, 0, 62, lists=(persist, local))
    messy_p = np.concatenate([persist[..., ::-1], np.full((B, nh, 2), -1, np.int32)], axis=-1)
    messy_l = np.concatenate([local[..., ::-1], persist[:, :, None, :2].repeat(3, axis=2),
                              np.full((B, nh, 3, 1), 77, np.int32)], axis=-1)
    b, _, _ = _run(B, nh, n_q, kv, kv, blk, 0, 0, 62, lists=(np.ascontiguousarray(messy_p),
                                                              np.ascontiguousarray(messy_l)))
    assert bool((a.view(t.int16) == b.view(t.int16)).all())


@pytest.mark.parametrize("name", sorted(synth.SPARSE_WORKLOADS) + sorted(synth.SPARSE_WORKLOADS_344))
def test_sparse_forcing_shapes_every_row(name):
    """Sparse Forcing-shaped memory, 12 heads: [1,8,8] blocks (84 query blocks
    of 64 tokens, 168 persistent + 336 window blocks) and [3,4,4] blocks (112
    query blocks of 48 tokens, 224 persistent + 448 window blocks).  Every
    query row of every head, and the whole NaN-poisoned output finite."""
    w = {**synth.SPARSE_WORKLOADS, **synth.SPARSE_WORKLOADS_344}[name]
    persist, local = synth.block_lists(w, 7)
    out, (qb, kb, vb), _ = _run(w.batch, w.n_heads, w.q_tokens, w.kv_tokens, w.kv_tokens, w.block,
                                0, 0, 71, lists=(persist, local))
    assert bool(torch().isfinite(out).all()), f"{name}: non-finite output"
    ref = S.block_sparse_attention(synth.to_f64(qb, "bf16"), synth.to_f64(kb, "bf16"),
                                   synth.to_f64(vb, "bf16"), w.kv_tokens, w.block, persist,
                                   local, 1.0 / math.sqrt(w.head_dim))
    say(name, check_attn(to_host_f64(out), ref, name))


@pytest.mark.parametrize("blk,jump", [(64, 40.0), (64, 120.0), (48, 40.0), (48, 120.0)])
def test_late_scores_around_the_certificate_bound(blk, jump):
    """Keys of one late local block (last in the visit order) whose base-2
    scores sit about `jump` above the rest, along a seeded direction u
    (q = N(0,1) + 6 u, those keys N(0,1) + s u).  The kernel takes each row's
    reference from its first tile and tests no later tile: a row sum up to
    2^64 is accepted (40), a larger or infinite one (120) sends the
    workgroup through a second, checked sweep.  Every row against the oracle."""
    D, nh, n_q, kv = 128, 1, 2 * blk, 16 * blk
    g = np.random.Generator(np.random.PCG64(81 + int(jump) + blk))
    u = g.standard_normal(D)
    u /= np.linalg.norm(u)
    s = jump * math.sqrt(D) / (math.log2(math.e) * 6.0)
    shift = np.zeros(kv)
    shift[13 * blk + 3], shift[13 * blk + 5], shift[13 * blk + 9] = s, s - 0.5, s - 1.0
    q = synth.bf16_bits_to_f32(synth.normal((1, n_q, nh, D), 82, "bf16")) + 6.0 * u
    k = synth.bf16_bits_to_f32(synth.normal((1, kv, nh, D), 83, "bf16"))
    k += shift[None, :, None, None] * u
    qb = synth.f32_to_bf16_bits(q.astype(np.float32))
    kb = synth.f32_to_bf16_bits(k.astype(np.float32))
    vb = synth.normal((1, kv, nh, D), 84, "bf16")
    persist = np.array([[[0, 2, 4]]], dtype=np.int32)
    local = np.array([[[[13, 7, 10], [10, 13, 7]]]], dtype=np.int32)
    t = torch()
    out = t.full((1, n_q, nh, D), float("nan"), dtype=t.float32, device="cuda")
    say("sparse late jump", blk, jump)
    rcc.block_sparse_attn(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), out, kv, blk,
                          t.from_numpy(persist).cuda(), t.from_numpy(local).cuda(),
                          1.0 / math.sqrt(D))
    t.cuda.synchronize()
    got = to_host_f64(out)
    assert np.isfinite(got).all()
    ref = S.block_sparse_attention(synth.to_f64(qb, "bf16"), synth.to_f64(kb, "bf16"),
                                   synth.to_f64(vb, "bf16"), kv, blk, persist, local,
                                   1.0 / math.sqrt(D))
    say("sparse late jump", blk, jump, check_attn(got, ref, f"sparse late jump {blk} {jump}"))


@pytest.mark.parametrize("blk", [64, 48])
def test_unnormalised_output_past_fp32_range(blk):
    """A late local block whose keys sit ~60 (base 2) above the rest and
    whose value rows are 2^74: row sums stay below 2^64 but the unnormalised
    O^T overflows fp32 in the unchecked sweep, so the output certificate
    must send the workgroup through the checked sweep.  Outputs are ~2^74,
    so the comparison is relative."""
    D, nh, n_q, kv = 128, 1, 2 * blk, 16 * blk
    g = np.random.Generator(np.random.PCG64(91 + blk))
    u = g.standard_normal(D)
    u /= np.linalg.norm(u)
    sh = 60.0 * math.sqrt(D) / (math.log2(math.e) * 6.0)
    big = [13 * blk + 3, 13 * blk + 5, 13 * blk + 9]
    shift = np.zeros(kv)
    shift[big] = [sh, sh - 0.5, sh - 1.0]
    q = 0.1 * synth.bf16_bits_to_f32(synth.normal((1, n_q, nh, D), 92, "bf16")) + 6.0 * u
    k = synth.bf16_bits_to_f32(synth.normal((1, kv, nh, D), 93, "bf16"))
    k += shift[None, :, None, None] * u
    v = synth.bf16_bits_to_f32(synth.normal((1, kv, nh, D), 94, "bf16"))
    v[0, big] *= 2.0 ** 74
    qb, kb, vb = (synth.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    persist = np.array([[[0, 2, 4]]], dtype=np.int32)
    local = np.array([[[[13, 7, 10], [10, 13, 7]]]], dtype=np.int32)
    t = torch()
    out = t.full((1, n_q, nh, D), float("nan"), dtype=t.float32, device="cuda")
    say("sparse output overflow", blk)
    rcc.block_sparse_attn(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), out, kv, blk,
                          t.from_numpy(persist).cuda(), t.from_numpy(local).cuda(),
                          1.0 / math.sqrt(D))
    t.cuda.synchronize()
    got = to_host_f64(out)
    assert np.isfinite(got).all()
    ref = S.block_sparse_attention(synth.to_f64(qb, "bf16"), synth.to_f64(kb, "bf16"),
                                   synth.to_f64(vb, "bf16"), kv, blk, persist, local,
                                   1.0 / math.sqrt(D))
    rel = np.abs(got - ref) / np.abs(ref).max(axis=-1, keepdims=True)
    say("sparse output overflow", blk, "rel err", float(rel.max()))
    assert rel.max() < 2e-2


@pytest.mark.parametrize("blk", [64, 48])
@pytest.mark.parametrize("n_sel", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("where", ["persist", "local"])
def test_stream_lengths(blk, n_sel, where):
    """Streams of 1 to 5 key blocks (2 to 10 tiles of 32 keys at 64-row
    blocks, 2 to 8 at 48-row blocks, the last one partial for odd counts),
    all in the persistent list or all in the local lists: the wave's first
    (checked) tile, the unrolled tile loops and their remainders.  Every row
    against the oracle."""
    nh, n_q, kv = 2, 2 * blk + 7, 12 * blk
    g = np.random.Generator(np.random.PCG64(500 + 10 * n_sel + blk))
    n_qb, n_kb = -(-n_q // blk), kv // blk
    if where == "persist":
        persist = np.stack([g.choice(n_kb, n_sel, replace=False) for _ in range(nh)])[None]
        local = np.zeros((1, nh, n_qb, 0), dtype=np.int32)
    else:
        persist = np.zeros((1, nh, 0), dtype=np.int32)
        local = np.stack([np.stack([g.choice(n_kb, n_sel, replace=False) for _ in range(n_qb)])
                          for _ in range(nh)])[None]
    persist, local = persist.astype(np.int32), local.astype(np.int32)
    out, (qb, kb, vb), _ = _run(1, nh, n_q, kv, kv, blk, 0, 0, 520 + n_sel, lists=(persist, local))
    ref = S.block_sparse_attention(synth.to_f64(qb, "bf16"), synth.to_f64(kb, "bf16"),
                                   synth.to_f64(vb, "bf16"), kv, blk, persist, local,
                                   1.0 / math.sqrt(128))
    check_attn(to_host_f64(out), ref, f"stream {where} {n_sel} x {blk}")


def test_errors_reported_without_launch():
    t = torch()
    q = t.zeros((1, 64, 2, 128), dtype=t.bfloat16, device="cuda")
    kc = t.zeros((1, 256, 2, 128), dtype=t.bfloat16, device="cuda")
    out = t.full_like(q, 3.0)
    lists = t.zeros((1, 2, 1, 2), dtype=t.int32, device="cuda")
    for kw, status in ((dict(block_tokens=40), rcc.RCC_ERR_SHAPE),
                       (dict(kv_tokens=257), rcc.RCC_ERR_RANGE)):
        a = dict(kv_tokens=256, block_tokens=64)
        a.update(kw)
        with pytest.raises(rcc.RccError) as e:
            rcc.block_sparse_attn(q, kc, kc, out, a["kv_tokens"], a["block_tokens"], None, None,
                                  0.1)
        assert e.value.status == status
    with pytest.raises(rcc.RccError) as e:
        rcc.block_sparse_attn(q.float(), kc.float(), kc.float(), out.float(), 256, 64, None,
                              lists, 0.1)
    assert e.value.status == rcc.RCC_ERR_DTYPE
    assert bool((out == 3.0).all())


@pytest.mark.parametrize("bh,bw", [(0, 0), (8, 8), (4, 16)])
def test_block_sparse_over_a_rolling_ring(bh, bw):
    """The pieces together: RoPE + ring write for a rollout (1 sink frame, 4
    window frames), then block-sparse attention of the last chunk over the
    ring, its sink blocks persistent and a random local subset of the window
    (always its own blocks).  Frames of 8 x 16 patches are two 64-token
    blocks each, so the held ring is 10 blocks: runs of 64 row-major tokens,
    or spatial 8 x 8 / 4 x 16 tiles when the ring write blockifies frames."""
    t = torch()
    from oracle import ring as G
    from oracle import rope3d as R
    d, nh, F, H, W, sink, window, blk = (44, 42, 42), 2, 2, 8, 16, 1, 4, 64
    D, hw = 128, 128
    cfg = rcc.rope_cfg(*d, 32, 8, 16)
    tables = rcc.rope3d_tables(cfg)
    otab = R.rope3d_tables(*d, 10000.0, 32, 8, 16)
    cap = (sink + window) * hw
    kr = t.zeros((1, cap, nh, D), dtype=t.bfloat16, device="cuda")
    vr = t.zeros_like(kr)
    okr, ovr = np.zeros((1, cap, nh, D)), np.zeros((1, cap, nh, D))
    r = rcc.ring(sink, window, bh, bw)
    for c in range(6):                                   # frames 0..11: the window wraps
        s = c * F
        host = [synth.normal((1, F * hw, nh, D), 700 + 10 * c + i, "bf16") for i in range(3)]
        dq, dk, dv = (to_dev(x, "bf16") for x in host)
        qo = t.empty_like(dq)
        say("ring + sparse: write chunk", c)
        rcc.rope3d_apply_append_ring(tables, rcc.grid(F, H, W, s, 0), r, dq, dk, dv, qo,
                                     kr, vr)
        q, k, v = (synth.to_f64(x, "bf16") for x in host)
        oq = G.rope3d_apply_append(q, k, v, okr, ovr, otab, F, H, W, s, 0, sink, window, bh, bw)
    held = rcc.ring_held_tokens(rcc.grid(F, H, W, 10), r)
    assert held == cap
    n_kb, n_qb = held // blk, F * hw // blk
    own = G.frame_slot(np.arange(10, 12), sink, window)          # slots of the chunk's frames
    own_blocks = (own[:, None] * (hw // blk) + np.arange(hw // blk)[None, :]).reshape(-1)
    # query block i of the chunk: its 64 tokens in the ring's row order
    qrows = G.positions(F, H, W, 10, 0, F * hw, sink, window, bh, bw)[:, 3]
    perm = np.argsort(qrows)                     # chunk token of each ring-ordered row
    qo = qo[:, t.from_numpy(perm).cuda()].contiguous()
    oq = oq[:, perm]
    g = np.random.Generator(np.random.PCG64(5))
    persist = np.tile(np.arange(sink * hw // blk, dtype=np.int32), (1, nh, 1))
    local = np.empty((1, nh, n_qb, 3), dtype=np.int32)
    for h in range(nh):
        for i in range(n_qb):
            local[0, h, i] = [own_blocks[i], *g.choice(np.arange(sink * hw // blk, n_kb), 2)]
    out = t.full_like(qo, float("nan"))
    say("ring + sparse: attention")
    rcc.block_sparse_attn(qo, kr, vr, out, held, blk, t.from_numpy(persist).cuda(),
                          t.from_numpy(local).cuda(), 1.0 / math.sqrt(D))
    t.cuda.synchronize()
    bf = lambda x: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)
    ref = S.block_sparse_attention(bf(oq), bf(okr), ovr, held, blk, persist, local,
                                   1.0 / math.sqrt(D))
    check_attn(to_host_f64(out), ref, "ring + block-sparse")
