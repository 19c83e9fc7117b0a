"""Thin ctypes binding over librcc.so (include/rcc.h), same names as the C ABI.

Argument marshalling only: every step of the path runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  The
binding checks that each tensor is contiguous, on the GPU, of a supported
dtype and large enough for the sizes passed, so the kernels never address
memory outside the caller's tensors; everything else is checked in C.

If librcc.so is missing or does not load, ``lib()`` raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "librcc.so")

RCC_OK, RCC_ERR_NULL, RCC_ERR_SHAPE, RCC_ERR_RANGE, RCC_ERR_DTYPE, RCC_ERR_ALIGN, RCC_ERR_HIP = range(7)
RCC_F32, RCC_BF16 = 0, 1

EXPORTS = ("rcc_rope3d_tables_floats", "rcc_rope3d_tables_init", "rcc_rope3d_tables_build",
           "rcc_rope3d_positions",
           "rcc_rope3d_apply_append", "rcc_qkv_rope_append", "rcc_chunk_causal_attn",
           "rcc_ring_held_tokens", "rcc_ring_positions", "rcc_rope3d_apply_append_ring",
           "rcc_qkv_rope_append_ring", "rcc_chunk_causal_attn_ring", "rcc_block_sparse_attn",
           "rcc_status_string", "rcc_last_error")


class RccError(RuntimeError):
    def __init__(self, status: int, call: str, detail: str):
        self.status = status
        super().__init__(f"{call}: {_status_name(status)}: {detail}")


class rcc_rope3d_cfg(ctypes.Structure):
    _fields_ = [("d_t", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_w", ctypes.c_int32),
                ("theta", ctypes.c_double),
                ("max_t", ctypes.c_int32), ("max_h", ctypes.c_int32), ("max_w", ctypes.c_int32)]


class rcc_rope3d_tables(ctypes.Structure):
    _fields_ = [("cfg", rcc_rope3d_cfg), ("data", ctypes.c_void_p), ("floats", ctypes.c_int64),
                ("seal", ctypes.c_uint64)]


class rcc_grid(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("height", ctypes.c_int32),
                ("width", ctypes.c_int32), ("start_frame", ctypes.c_int32),
                ("token_offset", ctypes.c_int64)]


class rcc_ring(ctypes.Structure):
    _fields_ = [("sink_frames", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("block_h", ctypes.c_int32), ("block_w", ctypes.c_int32)]


def rope_cfg(d_t, d_h, d_w, max_t, max_h, max_w, theta=10000.0) -> rcc_rope3d_cfg:
    return rcc_rope3d_cfg(d_t=d_t, d_h=d_h, d_w=d_w, theta=float(theta), max_t=max_t,
                          max_h=max_h, max_w=max_w)


class RopeTables:
    """A sealed tables descriptor (``desc``) and the device buffer it binds
    (``buf``, a float32 tensor kept alive here)."""

    def __init__(self, desc: rcc_rope3d_tables, buf):
        self.desc = desc
        self.buf = buf

    @property
    def cfg(self) -> rcc_rope3d_cfg:
        return self.desc.cfg

    @property
    def head_dim(self) -> int:
        c = self.desc.cfg
        return c.d_t + c.d_h + c.d_w


def grid(frames, height, width, start_frame, token_offset=0) -> rcc_grid:
    return rcc_grid(frames, height, width, start_frame, token_offset)


def ring(sink_frames, window_frames, block_h=0, block_w=0) -> rcc_ring:
    return rcc_ring(sink_frames, window_frames, block_h, block_w)


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load librcc.so once; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m rope_chunk_causal_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    cfgp, gridp = ctypes.POINTER(rcc_rope3d_cfg), ctypes.POINTER(rcc_grid)
    ringp = ctypes.POINTER(rcc_ring)
    L.rcc_rope3d_tables_floats.argtypes = [cfgp]
    L.rcc_rope3d_tables_floats.restype = I64
    tabp = ctypes.POINTER(rcc_rope3d_tables)
    L.rcc_rope3d_tables_init.argtypes = [cfgp, P, I64, tabp]
    L.rcc_rope3d_tables_init.restype = ctypes.c_int
    L.rcc_rope3d_tables_build.argtypes = [tabp, P]
    L.rcc_rope3d_tables_build.restype = ctypes.c_int
    L.rcc_rope3d_positions.argtypes = [gridp, I64, P, P]
    L.rcc_rope3d_positions.restype = ctypes.c_int
    L.rcc_rope3d_apply_append.argtypes = [tabp, gridp, ctypes.c_int, ctypes.c_int,
                                          I32, I64, I32, P, P, P, P, P, P, I64, P]
    L.rcc_rope3d_apply_append.restype = ctypes.c_int
    L.rcc_qkv_rope_append.argtypes = [tabp, gridp, I32, I64, I32, I32, P, P, P, P, P, P, I64, P]
    L.rcc_qkv_rope_append.restype = ctypes.c_int
    L.rcc_chunk_causal_attn.argtypes = [ctypes.c_int, ctypes.c_int, I32, I32, I32,
                                        I64, I64, I64, I64, F, P, P, P, I64, P, P]
    L.rcc_chunk_causal_attn.restype = ctypes.c_int
    L.rcc_ring_held_tokens.argtypes = [gridp, ringp]
    L.rcc_ring_held_tokens.restype = I64
    L.rcc_ring_positions.argtypes = [gridp, ringp, I64, P, P]
    L.rcc_ring_positions.restype = ctypes.c_int
    L.rcc_rope3d_apply_append_ring.argtypes = [tabp, gridp, ringp, ctypes.c_int, ctypes.c_int,
                                               I32, I64, I32, P, P, P, P, P, P, I64, P]
    L.rcc_rope3d_apply_append_ring.restype = ctypes.c_int
    L.rcc_qkv_rope_append_ring.argtypes = [tabp, gridp, ringp, I32, I64, I32, I32,
                                           P, P, P, P, P, P, I64, P]
    L.rcc_qkv_rope_append_ring.restype = ctypes.c_int
    L.rcc_chunk_causal_attn_ring.argtypes = [gridp, ringp, ctypes.c_int, ctypes.c_int, I32, I32,
                                             I32, I64, F, P, P, P, I64, P, P]
    L.rcc_chunk_causal_attn_ring.restype = ctypes.c_int
    L.rcc_block_sparse_attn.argtypes = [ctypes.c_int, ctypes.c_int, I32, I32, I32, I64, I64, I32,
                                        F, P, P, P, I64, P, I32, P, I32, P, P]
    L.rcc_block_sparse_attn.restype = ctypes.c_int
    L.rcc_status_string.argtypes = [ctypes.c_int]
    L.rcc_status_string.restype = ctypes.c_char_p
    L.rcc_last_error.argtypes = []
    L.rcc_last_error.restype = ctypes.c_char_p
    _ = D
    _lib = L
    return L


def _status_name(st: int) -> str:
    try:
        return lib().rcc_status_string(st).decode()
    except Exception:  # pragma: no cover
        return str(st)


def _check(st: int, call: str) -> None:
    if st != RCC_OK:
        raise RccError(st, call, lib().rcc_last_error().decode())


# ---------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RCC_F32
    if t.dtype == torch.bfloat16:
        return RCC_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t, name: str, numel: int, dtype=None) -> int:
    """data_ptr of a contiguous GPU tensor holding at least `numel` elements."""
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ----------------------------------------------------------- entry points

def rope3d_tables_floats(cfg: rcc_rope3d_cfg) -> int:
    n = lib().rcc_rope3d_tables_floats(ctypes.byref(cfg))
    if n < 0:
        raise RccError(RCC_ERR_SHAPE, "rope3d_tables_floats", "invalid cfg")
    return n


def rope3d_tables_init(cfg: rcc_rope3d_cfg, buf) -> RopeTables:
    """Seal a descriptor binding `cfg` to the float32 GPU buffer `buf` (host
    only; the buffer is not filled)."""
    torch = _torch()
    desc = rcc_rope3d_tables()
    if buf is None or not buf.is_cuda or not buf.is_contiguous() or buf.dtype != torch.float32:
        raise ValueError("buf must be a contiguous float32 GPU tensor")
    _check(lib().rcc_rope3d_tables_init(ctypes.byref(cfg), buf.data_ptr(), buf.numel(),
                                        ctypes.byref(desc)), "rope3d_tables_init")
    return RopeTables(desc, buf)


def rope3d_tables_build(tables: RopeTables, stream=None) -> RopeTables:
    """Fill the tables' device buffer with cos/sin (once)."""
    _check(lib().rcc_rope3d_tables_build(ctypes.byref(_desc(tables)), _stream(stream)),
           "rope3d_tables_build")
    return tables


def rope3d_tables(cfg: rcc_rope3d_cfg, buf=None, stream=None) -> RopeTables:
    """Allocate (unless `buf` is given), seal and fill the cos/sin tables of `cfg`."""
    torch = _torch()
    if buf is None:
        buf = torch.empty(rope3d_tables_floats(cfg), dtype=torch.float32, device="cuda")
    return rope3d_tables_build(rope3d_tables_init(cfg, buf), stream)


def _desc(tables) -> rcc_rope3d_tables:
    if not isinstance(tables, RopeTables):
        raise TypeError("tables must come from rope3d_tables / rope3d_tables_init")
    return tables.desc


def rope3d_positions(g: rcc_grid, n_tokens: int, thw=None, stream=None):
    """int32 [n_tokens, 4] = (t_global, h, w, cache_row) from the device function."""
    torch = _torch()
    if thw is None:
        thw = torch.empty((max(n_tokens, 0), 4), dtype=torch.int32, device="cuda")
    p = _ptr(thw, "thw", 4 * max(n_tokens, 0), torch.int32) if n_tokens > 0 else 0
    _check(lib().rcc_rope3d_positions(ctypes.byref(g), n_tokens, p, _stream(stream)),
           "rope3d_positions")
    return thw


def _rope_append_args(tables, q, k, v, q_out, k_cache, v_cache):
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or q_out.shape != q.shape:
        raise ValueError("q, k, v, q_out must share one [B, n, heads, D] shape")
    B, n, nh, D = q.shape
    if D != tables.head_dim:
        raise ValueError(f"head_dim {D} is not the tables' d_t + d_h + d_w = {tables.head_dim}")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or \
            k_cache.shape[0] != B or tuple(k_cache.shape[2:]) != (nh, D):
        raise ValueError("caches must be [B, cache_tokens, heads, D]")
    if k.dtype != q.dtype or v.dtype != q.dtype or k_cache.dtype != q_out.dtype or \
            v_cache.dtype != q_out.dtype:
        raise TypeError("q/k/v share in_dtype; q_out/k_cache/v_cache share out_dtype")
    cap = k_cache.shape[1]
    numel = B * n * nh * D
    return (_dtype_code(q), _dtype_code(q_out), B, n, nh,
            _ptr(q, "q", numel), _ptr(k, "k", numel), _ptr(v, "v", numel),
            _ptr(q_out, "q_out", numel), _ptr(k_cache, "k_cache", B * cap * nh * D),
            _ptr(v_cache, "v_cache", B * cap * nh * D), cap)


def rope3d_apply_append(tables: RopeTables, g: rcc_grid, q, k, v, q_out,
                        k_cache, v_cache, stream=None) -> None:
    """q, k, v [B, n, heads, D]; q_out same shape; caches [B, cache_tokens, heads, D]."""
    desc = _desc(tables)
    args = _rope_append_args(tables, q, k, v, q_out, k_cache, v_cache)
    _check(lib().rcc_rope3d_apply_append(ctypes.byref(desc), ctypes.byref(g), *args,
                                         _stream(stream)), "rope3d_apply_append")


def rope3d_apply_append_ring(tables: RopeTables, g: rcc_grid, r: rcc_ring, q, k, v,
                             q_out, k_cache, v_cache, stream=None) -> None:
    """As rope3d_apply_append, writing the rolling-window ring rows of the slice."""
    desc = _desc(tables)
    args = _rope_append_args(tables, q, k, v, q_out, k_cache, v_cache)
    _check(lib().rcc_rope3d_apply_append_ring(ctypes.byref(desc), ctypes.byref(g),
                                              ctypes.byref(r), *args, _stream(stream)),
           "rope3d_apply_append_ring")


def _qkv_args(tables, x, w_qkv, bias, q_out, k_cache, v_cache):
    torch = _torch()
    if x.dim() != 3 or q_out.dim() != 4 or tuple(q_out.shape[:2]) != tuple(x.shape[:2]):
        raise ValueError("x must be [B, n, model_dim] and q_out [B, n, heads, D]")
    B, n, K = x.shape
    nh, D = q_out.shape[2], q_out.shape[3]
    if D != tables.head_dim:
        raise ValueError(f"head_dim {D} is not the tables' d_t + d_h + d_w = {tables.head_dim}")
    if tuple(w_qkv.shape) != (3 * nh * D, K):
        raise ValueError("w_qkv must be [3 * heads * D, model_dim]")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or \
            k_cache.shape[0] != B or tuple(k_cache.shape[2:]) != (nh, D):
        raise ValueError("caches must be [B, cache_tokens, heads, D]")
    for name, t in (("x", x), ("w_qkv", w_qkv), ("q_out", q_out), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != 3 * nh * D):
        raise TypeError("bias must be float32 [3 * heads * D] or None")
    cap = k_cache.shape[1]
    return (B, n, nh, K, _ptr(x, "x", B * n * K), _ptr(w_qkv, "w_qkv", 3 * nh * D * K),
            _ptr(bias, "bias", 3 * nh * D), _ptr(q_out, "q_out", B * n * nh * D),
            _ptr(k_cache, "k_cache", B * cap * nh * D),
            _ptr(v_cache, "v_cache", B * cap * nh * D), cap)


def qkv_rope_append(tables: RopeTables, g: rcc_grid, x, w_qkv, bias, q_out,
                    k_cache, v_cache, stream=None) -> None:
    """x [B, n, model_dim] bf16; w_qkv [3*heads*D, model_dim] bf16; bias fp32
    [3*heads*D] or None; q_out [B, n, heads, D] bf16; caches [B, cache_tokens,
    heads, D] bf16."""
    desc = _desc(tables)
    args = _qkv_args(tables, x, w_qkv, bias, q_out, k_cache, v_cache)
    _check(lib().rcc_qkv_rope_append(ctypes.byref(desc), ctypes.byref(g), *args,
                                     _stream(stream)), "qkv_rope_append")


def qkv_rope_append_ring(tables: RopeTables, g: rcc_grid, r: rcc_ring, x, w_qkv, bias,
                         q_out, k_cache, v_cache, stream=None) -> None:
    """As qkv_rope_append, writing the rolling-window ring rows of the slice."""
    desc = _desc(tables)
    args = _qkv_args(tables, x, w_qkv, bias, q_out, k_cache, v_cache)
    _check(lib().rcc_qkv_rope_append_ring(ctypes.byref(desc), ctypes.byref(g),
                                          ctypes.byref(r), *args, _stream(stream)),
           "qkv_rope_append_ring")


def _attn_shapes(q, k_cache, v_cache, out):
    if q.dim() != 4 or out.shape != q.shape:
        raise ValueError("q and out must share one [B, Lq, heads, D] shape")
    B, lq, nh, D = q.shape
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or \
            k_cache.shape[0] != B or tuple(k_cache.shape[2:]) != (nh, D):
        raise ValueError("caches must be [B, cache_tokens, heads, D]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches share in_dtype")
    return B, lq, nh, D, k_cache.shape[1]


def chunk_causal_attn(q, k_cache, v_cache, out, q_pos: int, kv_tokens: int,
                      chunk_tokens: int, scale: float, stream=None) -> None:
    """q [B, Lq, heads, D], caches [B, cache_tokens, heads, D], out like q."""
    B, lq, nh, D, cap = _attn_shapes(q, k_cache, v_cache, out)
    _check(lib().rcc_chunk_causal_attn(
        _dtype_code(q), _dtype_code(out), B, nh, D, lq, q_pos, kv_tokens, chunk_tokens,
        float(scale), _ptr(q, "q", B * lq * nh * D), _ptr(k_cache, "k_cache", B * cap * nh * D),
        _ptr(v_cache, "v_cache", B * cap * nh * D), cap, _ptr(out, "out", B * lq * nh * D),
        _stream(stream)), "chunk_causal_attn")


def ring_held_tokens(g: rcc_grid, r: rcc_ring) -> int:
    """Ring rows the chunk of `g` attends once written (host only)."""
    n = lib().rcc_ring_held_tokens(ctypes.byref(g), ctypes.byref(r))
    if n < 0:
        raise RccError(RCC_ERR_SHAPE, "ring_held_tokens", "invalid grid or ring")
    return n


def ring_positions(g: rcc_grid, r: rcc_ring, n_tokens: int, thw=None, stream=None):
    """int32 [n_tokens, 4] = (t_global, h, w, ring_row) from the device function."""
    torch = _torch()
    if thw is None:
        thw = torch.empty((max(n_tokens, 0), 4), dtype=torch.int32, device="cuda")
    p = _ptr(thw, "thw", 4 * max(n_tokens, 0), torch.int32) if n_tokens > 0 else 0
    _check(lib().rcc_ring_positions(ctypes.byref(g), ctypes.byref(r), n_tokens, p,
                                    _stream(stream)), "ring_positions")
    return thw


def chunk_causal_attn_ring(g: rcc_grid, r: rcc_ring, q, k_cache, v_cache, out, scale: float,
                           stream=None) -> None:
    """Attention of q (the chunk of `g`, or a slice of it) over every row the
    ring holds once that chunk is written."""
    B, lq, nh, D, cap = _attn_shapes(q, k_cache, v_cache, out)
    _check(lib().rcc_chunk_causal_attn_ring(
        ctypes.byref(g), ctypes.byref(r), _dtype_code(q), _dtype_code(out), B, nh, D, lq,
        float(scale), _ptr(q, "q", B * lq * nh * D), _ptr(k_cache, "k_cache", B * cap * nh * D),
        _ptr(v_cache, "v_cache", B * cap * nh * D), cap, _ptr(out, "out", B * lq * nh * D),
        _stream(stream)), "chunk_causal_attn_ring")


def block_sparse_attn(q, k_cache, v_cache, out, kv_tokens: int, block_tokens: int, persist,
                      local, scale: float, stream=None) -> None:
    """q [B, Lq, heads, 128] bf16 (block-contiguous), caches [B, cache_tokens,
    heads, 128] bf16, out like q (bf16 or fp32); persist int32 [B, heads, n_p]
    or None; local int32 [B, heads, ceil(Lq / block_tokens), n_l] or None."""
    torch = _torch()
    B, lq, nh, D, cap = _attn_shapes(q, k_cache, v_cache, out)
    n_qb = -(-lq // block_tokens)
    n_p = 0 if persist is None else persist.shape[-1]
    n_l = 0 if local is None else local.shape[-1]
    if persist is not None and tuple(persist.shape) != (B, nh, n_p):
        raise ValueError("persist must be [B, heads, n_persist]")
    if local is not None and tuple(local.shape) != (B, nh, n_qb, n_l):
        raise ValueError("local must be [B, heads, ceil(Lq / block_tokens), n_local]")
    _check(lib().rcc_block_sparse_attn(
        _dtype_code(q), _dtype_code(out), B, nh, D, lq, kv_tokens, block_tokens, float(scale),
        _ptr(q, "q", B * lq * nh * D), _ptr(k_cache, "k_cache", B * cap * nh * D),
        _ptr(v_cache, "v_cache", B * cap * nh * D), cap,
        _ptr(persist, "persist", B * nh * n_p, torch.int32) if n_p else 0, n_p,
        _ptr(local, "local", B * nh * n_qb * n_l, torch.int32) if n_l else 0, n_l,
        _ptr(out, "out", B * lq * nh * D), _stream(stream)), "block_sparse_attn")
