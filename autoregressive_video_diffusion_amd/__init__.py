"""Chunk-causal Causal-RoPE attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libcrattn.so`` (C ABI declared in
``include/crattn.h``).  Each function has the name of the C entry point it
wraps and only marshals arguments: torch tensors become device pointers and
sizes, the current torch stream becomes the HIP stream.  All computation runs
in the library's HIP kernels; there is no fallback.  If the library has not
been built, importing the binding's functions raises immediately.

Entry points (see include/crattn.h for the full contracts):

* ``rope_table_bytes`` / ``rope_precompute`` -- cos/sin tables of the 3D
  rotary code, built once on the device.
* ``rope_apply_append`` -- rotate Q and K from a global time index, write Q',
  append K' and V to the KV cache, in one pass.
* ``qkv_rope_append`` -- the QKV projection of the chunk's hidden states with
  the same rotation and append fused into its epilogue.
* ``chunk_causal_attn_workspace_bytes`` / ``chunk_causal_attn`` -- flash
  attention of a chunk's queries against the cache, bidirectional inside a
  chunk and causal across chunks.
* ``chunk_causal_attn_rope`` -- the same attention on un-rotated queries,
  rotated on load.
* ``hsa_pool_bytes`` / ``hsa_pool_keys`` / ``hsa_select`` / ``hsa_attn`` --
  hierarchical block-sparse attention: pooled frame and block keys, two-level
  block selection per query block, attention over the own chunk plus the
  selected blocks.
* ``svg2_kmeans_workspace_bytes`` / ``svg2_kmeans`` / ``svg2_kmeans2`` / ``svg2_n_slots`` /
  ``svg2_plan`` / ``svg2_attn_workspace_bytes`` / ``svg2_attn`` --
  semantic-permutation sparse attention: k-means of queries and keys with the
  reordering by cluster, centroid top-p selection with the key lists and
  query tiles, attention of the query tiles over their key lists.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "CrattnError", "lib_path", "load", "rope_table_bytes", "rope_precompute",
    "rope_apply_append", "qkv_rope_append", "chunk_causal_attn_workspace_bytes",
    "chunk_causal_attn", "chunk_causal_attn_noalloc", "chunk_causal_attn_rope", "hsa_pool_bytes",
    "hsa_pool_keys", "hsa_select", "hsa_attn", "svg2_kmeans_workspace_bytes", "svg2_kmeans", "svg2_kmeans2",
    "svg2_n_slots", "svg2_plan", "svg2_attn_workspace_bytes", "svg2_attn", "crattn_last_error", "EXPORTS",
    "HSA_QBLOCK", "HSA_KBLOCK", "SVG2_QTILE",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libcrattn.so")

CRATTN_OK, CRATTN_EINVAL, CRATTN_ENOTSUP, CRATTN_EHIP = 0, 1, 2, 3
CRATTN_F32, CRATTN_BF16 = 0, 1

# Every symbol include/crattn.h declares.
EXPORTS = ("rope_table_bytes", "rope_precompute", "rope_apply_append", "qkv_rope_append",
           "chunk_causal_attn_workspace_bytes", "chunk_causal_attn", "chunk_causal_attn_noalloc",
           "chunk_causal_attn_rope",
           "hsa_pool_bytes", "hsa_pool_keys", "hsa_select", "hsa_attn",
           "svg2_kmeans_workspace_bytes", "svg2_kmeans", "svg2_kmeans2", "svg2_n_slots",
           "svg2_plan",
           "svg2_attn_workspace_bytes", "svg2_attn", "crattn_last_error")
HSA_QBLOCK, HSA_KBLOCK = 256, 64
SVG2_QTILE = 256

_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int


class _KmProblem(ctypes.Structure):
    """svg2_kmeans_problem of include/crattn.h."""
    _fields_ = [("x", _vp), ("stride_b", _i64), ("stride_h", _i64), ("stride_row", _i64),
                ("B", _i32), ("H", _i32), ("n", _i32), ("C", _i32),
                ("centroids", _vp), ("cent_stride", _i64), ("perm", _vp), ("perm_stride", _i64),
                ("offsets", _vp), ("off_stride", _i64), ("workspace", _vp),
                ("ws_bytes", ctypes.c_size_t)]


class CrattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def load():
    """Load libcrattn.so (built by ``python -m autoregressive_video_diffusion_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with "
                          "`python -m autoregressive_video_diffusion_amd.build`")
    lib = ctypes.CDLL(lib_path)
    lib.rope_table_bytes.argtypes = [_i32, _i32, _i32, _i32]
    lib.rope_table_bytes.restype = ctypes.c_size_t
    lib.rope_precompute.argtypes = [_vp, _i32, _i32, _i32, _i32, ctypes.c_double, _vp]
    lib.rope_precompute.restype = _i32
    lib.rope_apply_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32,
                                      _i32, _i32, _i32, _i32, _i64, _i64, _i64, _i32, _i32, _i32,
                                      _vp]
    lib.rope_apply_append.restype = _i32
    lib.qkv_rope_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _i32, _i64, _i64, _i64, _i32, _i32, _vp]
    lib.qkv_rope_append.restype = _i32
    lib.chunk_causal_attn_workspace_bytes.argtypes = [_i32, _i32, _i64, _i64, _i64, _i64, _i32]
    lib.chunk_causal_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.chunk_causal_attn.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                      ctypes.c_size_t, _i32, _i32, _i32, _i64, ctypes.c_float, _vp]
    lib.chunk_causal_attn.restype = _i32
    lib.chunk_causal_attn_noalloc.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp,
                                              _i32, _i32, _i32, _i64, ctypes.c_float, _vp]
    lib.chunk_causal_attn_noalloc.restype = _i32
    lib.chunk_causal_attn_rope.argtypes = [_vp, _vp, _i32, _i32, _i32, _i64, _i32, _i32, _vp, _vp,
                                           _i64, _i64, _i64, _i64, _vp, _vp, _vp, ctypes.c_size_t,
                                           _i32, _i32, _i32, _i64, ctypes.c_float, _vp]
    lib.chunk_causal_attn_rope.restype = _i32
    lib.hsa_pool_bytes.argtypes = [_i32, _i32, _i64, _i32, _i32]
    lib.hsa_pool_bytes.restype = ctypes.c_size_t
    lib.hsa_pool_keys.argtypes = [_vp, _i64, _i64, _i64, _i32, _vp, _i32, _i32, _i32, _vp]
    lib.hsa_pool_keys.restype = _i32
    lib.hsa_select.argtypes = [_vp, _vp, _i64, _i64, _i32, _i64, _i64, _i32, _i32, _vp, _i32,
                               _i32, _i32, _i64, _vp]
    lib.hsa_select.restype = _i32
    lib.hsa_attn.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _i32, _vp, _vp,
                             _i32, _i32, _i32, _i64, ctypes.c_float, _vp]
    lib.hsa_attn.restype = _i32
    lib.svg2_kmeans_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
    lib.svg2_kmeans_workspace_bytes.restype = ctypes.c_size_t
    lib.svg2_kmeans.argtypes = [_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _vp, _i64, _vp, _i64, _vp, _i64, _vp, ctypes.c_size_t, _vp]
    lib.svg2_kmeans.restype = _i32
    lib.svg2_kmeans2.argtypes = [ctypes.POINTER(_KmProblem), _i32, _i32, _i32, _vp]
    lib.svg2_kmeans2.restype = _i32
    lib.svg2_n_slots.argtypes = [_i64, _i32]
    lib.svg2_n_slots.restype = _i32
    lib.svg2_plan.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                              _i64, _i64, ctypes.c_float, ctypes.c_float, _vp, _vp, _i64, _vp,
                              _vp, _i32, _vp]
    lib.svg2_plan.restype = _i32
    lib.svg2_attn_workspace_bytes.argtypes = [_i32, _i32, _i64, _i32, _i32, _i32]
    lib.svg2_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.svg2_attn.argtypes = [_vp, _vp, _vp, _i64, _vp, _vp, _i32, _vp, _i64, _vp, _i32, _i32,
                              _vp, _vp, _vp, ctypes.c_size_t, _i32, _i32, _i32, _i64,
                              ctypes.c_float, _vp]
    lib.svg2_attn.restype = _i32
    lib.crattn_last_error.argtypes = []
    lib.crattn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def crattn_last_error() -> str:
    return load().crattn_last_error().decode()


def _raise(status: int):
    if status != CRATTN_OK:
        raise CrattnError(status, crattn_last_error())


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CRATTN_BF16
    if t.dtype == torch.float32:
        return CRATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def rope_table_bytes(head_dim: int, max_t: int, max_h: int, max_w: int) -> int:
    return int(load().rope_table_bytes(head_dim, max_t, max_h, max_w))


def rope_precompute(table: torch.Tensor, head_dim: int, max_t: int, max_h: int, max_w: int,
                    theta: float = 10000.0, stream=None) -> torch.Tensor:
    """Fill ``table`` (float32 device tensor of rope_table_bytes/4 elements)."""
    need = rope_table_bytes(head_dim, max_t, max_h, max_w)
    if table.dtype != torch.float32 or table.numel() * 4 < need:
        raise ValueError(f"table must be float32 with at least {need} bytes")
    _raise(load().rope_precompute(_ptr(table), head_dim, max_t, max_h, max_w, float(theta),
                                  _stream(stream)))
    return table


def rope_apply_append(q: torch.Tensor | None, q_out: torch.Tensor | None, k: torch.Tensor,
                      v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      cache_pos: int, table: torch.Tensor, max_t: int, max_h: int, max_w: int,
                      t0: int, tok_off: int, grid_h: int, grid_w: int, stream=None) -> None:
    """q, q_out, k, v: [B, n, H, D]; caches [B, H, cap, D]; same dtype (bf16 or fp32)."""
    B, n, H, D = k.shape
    cap = k_cache.shape[2]
    for t in (q, q_out, v):
        if t is not None and (tuple(t.shape) != (B, n, H, D) or t.dtype != k.dtype):
            raise ValueError("q, q_out, k, v must share shape [B, n, H, D] and dtype")
    for t in (k_cache, v_cache):
        if tuple(t.shape) != (B, H, cap, D) or t.dtype != k.dtype:
            raise ValueError("caches must be [B, H, cap, D] of k's dtype")
    if table.dtype != torch.float32:
        raise ValueError("table must be float32")
    _raise(load().rope_apply_append(_ptr(q), _ptr(q_out), _ptr(k), _ptr(v), _ptr(k_cache),
                                    _ptr(v_cache), cap, cache_pos, _ptr(table), max_t, max_h,
                                    max_w, B, H, D, n, t0, tok_off, grid_h, grid_w,
                                    _dtype_code(k), _stream(stream)))


def qkv_rope_append(x: torch.Tensor, w: torch.Tensor, q_out: torch.Tensor | None,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, cache_pos: int,
                    table: torch.Tensor, max_t: int, max_h: int, max_w: int, t0: int,
                    tok_off: int, grid_h: int, grid_w: int, stream=None) -> None:
    """x: [B, n, C] bf16; w: [3*H*D, C] bf16; q_out: [B, n, H, D] bf16 or None;
    caches [B, H, cap, D] bf16."""
    B, n, C = x.shape
    _, H, cap, D = k_cache.shape
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("x and w must be bfloat16")
    if tuple(w.shape) != (3 * H * D, C):
        raise ValueError("w must be [3*H*D, C] for the caches' H and D")
    if q_out is not None and (tuple(q_out.shape) != (B, n, H, D) or q_out.dtype != x.dtype):
        raise ValueError("q_out must be [B, n, H, D] bfloat16")
    for t in (k_cache, v_cache):
        if tuple(t.shape) != (B, H, cap, D) or t.dtype != x.dtype:
            raise ValueError("caches must be [B, H, cap, D] bfloat16")
    if table.dtype != torch.float32:
        raise ValueError("table must be float32")
    _raise(load().qkv_rope_append(_ptr(x), _ptr(w), _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
                                  cap, cache_pos, _ptr(table), max_t, max_h, max_w, B, H, D, C,
                                  n, t0, tok_off, grid_h, grid_w, _stream(stream)))


def chunk_causal_attn_workspace_bytes(B: int, H: int, Lq: int, kv_len: int, q_pos0: int,
                                      chunk_tokens: int, D: int) -> int:
    return int(load().chunk_causal_attn_workspace_bytes(B, H, Lq, kv_len, q_pos0, chunk_tokens,
                                                         D))


def chunk_causal_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len: int,
                      q_pos0: int, chunk_tokens: int, out: torch.Tensor,
                      lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      scale: float = 0.0, stream=None) -> torch.Tensor:
    """q, out: [B, Lq, H, D] bf16; caches [B, H, cap, D] bf16; lse [B, H, Lq] fp32."""
    B, Lq, H, D = q.shape
    cap = k_cache.shape[2]
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16")
    if tuple(out.shape) != (B, Lq, H, D):
        raise ValueError("out must have q's shape")
    for t in (k_cache, v_cache):
        if tuple(t.shape) != (B, H, cap, D) or t.dtype != torch.bfloat16:
            raise ValueError("caches must be bf16 [B, H, cap, D]")
    if lse is not None and (tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, H, Lq]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _raise(load().chunk_causal_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), cap, kv_len, q_pos0,
                                    chunk_tokens, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                    B, H, D, Lq, float(scale), _stream(stream)))
    return out


def chunk_causal_attn_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              kv_len: int, q_pos0: int, chunk_tokens: int, out: torch.Tensor,
                              lse: torch.Tensor | None = None, scale: float = 0.0,
                              stream=None) -> torch.Tensor:
    """chunk_causal_attn with no workspace argument: split partials go to the
    library's fixed per-device scratch (calls on one device must not overlap)."""
    B, Lq, H, D = q.shape
    cap = k_cache.shape[2]
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16")
    if tuple(out.shape) != (B, Lq, H, D):
        raise ValueError("out must have q's shape")
    for t in (k_cache, v_cache):
        if tuple(t.shape) != (B, H, cap, D) or t.dtype != torch.bfloat16:
            raise ValueError("caches must be bf16 [B, H, cap, D]")
    if lse is not None and (tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, H, Lq]")
    _raise(load().chunk_causal_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), cap, kv_len,
                                            q_pos0, chunk_tokens, _ptr(out), _ptr(lse), B, H, D,
                                            Lq, float(scale), _stream(stream)))
    return out


def chunk_causal_attn_rope(q: torch.Tensor, table: torch.Tensor, max_t: int, max_h: int,
                           max_w: int, t0: int, grid_h: int, grid_w: int, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, kv_len: int, q_pos0: int, chunk_tokens: int,
                           out: torch.Tensor, lse: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, scale: float = 0.0,
                           stream=None) -> torch.Tensor:
    """As chunk_causal_attn, with q not yet rotated: the Causal-RoPE of each
    query row (token (q_pos0 mod chunk_tokens) + i of the chunk starting at
    time index t0) is applied on load."""
    B, Lq, H, D = q.shape
    cap = k_cache.shape[2]
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16")
    if tuple(out.shape) != (B, Lq, H, D):
        raise ValueError("out must have q's shape")
    for t in (k_cache, v_cache):
        if tuple(t.shape) != (B, H, cap, D) or t.dtype != torch.bfloat16:
            raise ValueError("caches must be bf16 [B, H, cap, D]")
    if lse is not None and (tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, H, Lq]")
    if table.dtype != torch.float32:
        raise ValueError("table must be float32")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _raise(load().chunk_causal_attn_rope(_ptr(q), _ptr(table), max_t, max_h, max_w, t0, grid_h,
                                         grid_w, _ptr(k_cache), _ptr(v_cache), cap, kv_len,
                                         q_pos0, chunk_tokens, _ptr(out), _ptr(lse),
                                         _ptr(workspace), ws_bytes, B, H, D, Lq, float(scale),
                                         _stream(stream)))
    return out


def hsa_pool_bytes(B: int, H: int, cap: int, D: int, per_frame: int) -> int:
    return int(load().hsa_pool_bytes(B, H, cap, D, per_frame))


def hsa_pool_keys(k_cache: torch.Tensor, row0: int, nrows: int, per_frame: int,
                  pool: torch.Tensor, stream=None) -> torch.Tensor:
    """Pool the keys of cache rows [row0, row0 + nrows) (whole frames) into
    `pool` (float32, hsa_pool_bytes bytes): frame means then block means."""
    B, H, cap, D = k_cache.shape
    if k_cache.dtype != torch.bfloat16:
        raise ValueError("k_cache must be bf16 [B, H, cap, D]")
    if pool.dtype != torch.float32 or pool.numel() * 4 < hsa_pool_bytes(B, H, cap, D, per_frame):
        raise ValueError("pool must be float32 of at least hsa_pool_bytes(...) bytes")
    _raise(load().hsa_pool_keys(_ptr(k_cache), cap, row0, nrows, per_frame, _ptr(pool), B, H, D,
                                _stream(stream)))
    return pool


def hsa_select(q: torch.Tensor, pool: torch.Tensor, cap: int, kv_len: int, per_frame: int,
               q_pos0: int, chunk_tokens: int, kf: int, kb: int, sel: torch.Tensor,
               stream=None) -> torch.Tensor:
    """q: [B, Lq, H, D] bf16 (rotated); sel: int32 [B, H, ceil(Lq/256), kb].
    History = the frames of rows [0, kv_len) outside the own chunk
    (q_pos0 // chunk_tokens)."""
    B, Lq, H, D = q.shape
    if q.dtype != torch.bfloat16 or pool.dtype != torch.float32:
        raise ValueError("q must be bf16 and pool float32")
    nqb = -(-Lq // HSA_QBLOCK)
    if sel.dtype != torch.int32 or tuple(sel.shape) != (B, H, nqb, kb):
        raise ValueError(f"sel must be int32 [{B}, {H}, {nqb}, {kb}]")
    _raise(load().hsa_select(_ptr(q), _ptr(pool), cap, kv_len, per_frame, q_pos0, chunk_tokens,
                             kf, kb, _ptr(sel), B, H, D, Lq, _stream(stream)))
    return sel


def hsa_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len: int,
             q_pos0: int, chunk_tokens: int, per_frame: int, sel: torch.Tensor, out: torch.Tensor,
             lse: torch.Tensor | None = None, scale: float = 0.0, stream=None) -> torch.Tensor:
    """Attention over the own chunk plus the selected history blocks of sel
    (history: the frames of rows [0, kv_len) outside the own chunk)."""
    B, Lq, H, D = q.shape
    cap = k_cache.shape[2]
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16")
    if tuple(out.shape) != (B, Lq, H, D):
        raise ValueError("out must have q's shape")
    for t in (k_cache, v_cache):
        if tuple(t.shape) != (B, H, cap, D) or t.dtype != torch.bfloat16:
            raise ValueError("caches must be bf16 [B, H, cap, D]")
    if lse is not None and (tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, H, Lq]")
    nqb = -(-Lq // HSA_QBLOCK)
    if sel.dtype != torch.int32 or sel.dim() != 4 or tuple(sel.shape[:3]) != (B, H, nqb):
        raise ValueError(f"sel must be int32 [{B}, {H}, {nqb}, kb]")
    _raise(load().hsa_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), cap, kv_len, q_pos0,
                           chunk_tokens, per_frame, _ptr(sel), sel.shape[3], _ptr(out), _ptr(lse),
                           B, H, D, Lq, float(scale), _stream(stream)))
    return out



def svg2_kmeans_workspace_bytes(B: int, H: int, n: int, C: int) -> int:
    return int(load().svg2_kmeans_workspace_bytes(B, H, n, C))


def _view_ptr(t: torch.Tensor, what: str, dtype: torch.dtype, inner: int):
    """Start of a strided device view whose last `inner` dims are dense, and
    its per-head stride (batch stride = H x head stride)."""
    if not t.is_cuda or t.dtype != dtype:
        raise ValueError(f"{what} must be a {dtype} device tensor")
    size, st = t.shape, t.stride()
    dense = 1
    for d in range(t.dim() - 1, t.dim() - 1 - inner, -1):
        if st[d] != dense:
            raise ValueError(f"{what}: the last {inner} dims must be contiguous")
        dense *= size[d]
    if size[0] > 1 and st[0] != size[1] * st[1]:
        raise ValueError(f"{what}: batch stride must be H x head stride")
    return t.data_ptr(), st[1]


def _km_problem(x: torch.Tensor, C: int, centroids: torch.Tensor, perm: torch.Tensor,
                offsets: torch.Tensor, workspace: torch.Tensor):
    B, H, n, D = x.shape
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.stride(3) != 1:
        raise ValueError("x must be a bf16 device view with a dense last dim")
    if tuple(centroids.shape) != (B, H, C, D) or tuple(perm.shape) != (B, H, n) or \
            tuple(offsets.shape) != (B, H, C + 1):
        raise ValueError("centroids [B, H, C, D], perm [B, H, n], offsets [B, H, C+1] required")
    cp, cs = _view_ptr(centroids, "centroids", torch.float32, 2)
    pp, ps = _view_ptr(perm, "perm", torch.int32, 1)
    op, os_ = _view_ptr(offsets, "offsets", torch.int32, 1)
    return _KmProblem(x.data_ptr(), x.stride(0), x.stride(1), x.stride(2), B, H, n, C, cp, cs,
                      pp, ps, op, os_, _ptr(workspace),
                      workspace.numel() * workspace.element_size()), D


def svg2_kmeans(x: torch.Tensor, C: int, iters: int, from_tokens: bool,
                centroids: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor,
                workspace: torch.Tensor, stream=None):
    """k-means of the tokens of every head, then their reordering by cluster.

    x: a bf16 view with logical shape [B, H, n, D] (any strides, last dim
    dense): q.permute(0, 2, 1, 3) for queries [B, Lq, H, D], or
    k_cache[:, :, r0:r0 + n] for one chunk slot of a cache.  centroids: float
    view [B, H, C, D] (in/out); perm: int32 view [B, H, n]; offsets: int32
    view [B, H, C + 1] (each dense inside a head, e.g. slices [:, :, s] of
    per-slot arrays)."""
    p, D = _km_problem(x, C, centroids, perm, offsets, workspace)
    _raise(load().svg2_kmeans(p.x, p.stride_b, p.stride_h, p.stride_row, p.B, p.H, p.n, D, C,
                              iters, int(bool(from_tokens)), p.centroids, p.cent_stride, p.perm,
                              p.perm_stride, p.offsets, p.off_stride, p.workspace, p.ws_bytes,
                              _stream(stream)))
    return centroids, perm, offsets


def svg2_kmeans2(first: tuple, second: tuple, iters: int, from_tokens: bool, stream=None):
    """svg2_kmeans of two problems in one launch sequence (same head_dim,
    iters and start).  Each problem is the tuple (x, C, centroids, perm,
    offsets, workspace) of svg2_kmeans's arguments; the two must not share
    any buffer."""
    p0, d0 = _km_problem(*first)
    p1, d1 = _km_problem(*second)
    if d0 != d1:
        raise ValueError("both problems need the same head_dim")
    arr = (_KmProblem * 2)(p0, p1)
    _raise(load().svg2_kmeans2(arr, d0, iters, int(bool(from_tokens)), _stream(stream)))


def svg2_n_slots(Lq: int, Cq: int) -> int:
    return int(load().svg2_n_slots(Lq, Cq))


def svg2_plan(q_cent: torch.Tensor, q_off: torch.Tensor, k_cent: torch.Tensor,
              k_off: torch.Tensor, k_perm: torch.Tensor, n_vis: int, Lq: int, p: float,
              sel: torch.Tensor, lists: torch.Tensor, list_len: torch.Tensor,
              slots: torch.Tensor, scale: float = 0.0, stream=None):
    """q_cent [B, H, Cq, D] f32, q_off [B, H, Cq+1] i32; k_cent [B, H, S, Ck, D],
    k_off [B, H, S, Ck+1], k_perm [B, H, S, L]; lists [B, H, Cq, list_cap],
    list_len [B, H, Cq], slots [B, H, n_slots, 4], sel [B, H, Cq, n_vis*Ck]
    (all int32 but the centroids)."""
    B, H, Cq, D = q_cent.shape
    _, _, S, Ck, _ = k_cent.shape
    L = k_perm.shape[3]
    for t, name in ((q_off, "q_off"), (k_off, "k_off"), (k_perm, "k_perm"), (lists, "lists"),
                    (list_len, "list_len"), (slots, "slots")):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if q_cent.dtype != torch.float32 or k_cent.dtype != torch.float32:
        raise ValueError("centroids must be float32")
    if tuple(q_off.shape) != (B, H, Cq + 1) or tuple(k_off.shape) != (B, H, S, Ck + 1) or \
            tuple(k_perm.shape[:3]) != (B, H, S) or tuple(lists.shape[:3]) != (B, H, Cq) or \
            tuple(list_len.shape) != (B, H, Cq) or slots.dim() != 4 or \
            tuple(slots.shape[:2]) != (B, H) or slots.shape[3] != 4:
        raise ValueError("inconsistent shapes")
    if sel.dtype != torch.int32 or tuple(sel.shape) != (B, H, Cq, n_vis * Ck):
        raise ValueError(f"sel must be int32 [{B}, {H}, {Cq}, {n_vis * Ck}]")
    _raise(load().svg2_plan(_ptr(q_cent), _ptr(q_off), _ptr(k_cent), _ptr(k_off), _ptr(k_perm),
                            B, H, D, Cq, Ck, S, n_vis, L, Lq, float(p), float(scale), _ptr(sel),
                            _ptr(lists), lists.shape[3], _ptr(list_len), _ptr(slots),
                            slots.shape[2], _stream(stream)))
    return sel, lists, list_len, slots


def svg2_attn_workspace_bytes(B: int, H: int, Lq: int, D: int, n_slots: int, splits: int) -> int:
    return int(load().svg2_attn_workspace_bytes(B, H, Lq, D, n_slots, splits))


def svg2_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              q_perm: torch.Tensor, slots: torch.Tensor, lists: torch.Tensor,
              list_len: torch.Tensor, out: torch.Tensor, lse: torch.Tensor | None = None,
              splits: int = 1, workspace: torch.Tensor | None = None, scale: float = 0.0,
              stream=None) -> torch.Tensor:
    """Attention of the query tiles of `slots` over their clusters' key lists.
    q, out: [B, Lq, H, D] bf16; caches [B, H, cap, D] bf16; q_perm [B, H, Lq];
    workspace: a device buffer of svg2_attn_workspace_bytes(...) bytes
    (required: it holds the work counter of the persistent launch)."""
    B, Lq, H, D = q.shape
    cap = k_cache.shape[2]
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be bf16 of one shape")
    for t in (k_cache, v_cache):
        if tuple(t.shape) != (B, H, cap, D) or t.dtype != torch.bfloat16:
            raise ValueError("caches must be bf16 [B, H, cap, D]")
    if tuple(q_perm.shape) != (B, H, Lq) or q_perm.dtype != torch.int32:
        raise ValueError("q_perm must be int32 [B, H, Lq]")
    if lse is not None and (tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, H, Lq]")
    Cq, list_cap = lists.shape[2], lists.shape[3]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _raise(load().svg2_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), cap, _ptr(q_perm),
                            _ptr(slots), slots.shape[2], _ptr(lists), list_cap, _ptr(list_len),
                            Cq, splits, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, B, H, D,
                            Lq, float(scale), _stream(stream)))
    return out
