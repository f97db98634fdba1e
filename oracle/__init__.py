"""CPU reference (fp64) for the Causal-RoPE chunk-causal attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library never loads it, and it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain fp64 C loops, compiled by
``oracle/build.py`` into ``liboracle.so``); this module only marshals NumPy
arrays through ctypes.  Every array argument is float64 (or int64), C-order.

What is computed, and where it comes from (pages cited by title/section):

* 3D rotary position embedding with a global time index -- "Accelerating
  Video Generation Inference with Sequential-Parallel 3D Positional Encoding
  Using a Global Time Index", §2.B (t_global = t + s; local rotation from the
  start offset and the local index).
* cos/sin tables precomputed once -- same page, §2.C.
* KV-cache append -- same page, §1 (KV caching, rolling windows); "Wave
  Forcing" abstract (the cache update is its own forward pass).
* chunk-causal attention: bidirectional inside a chunk, causal across
  chunks -- "Wave Forcing" abstract (chunk-based causal attention over
  earlier chunks).
* the QKV projection with Causal-RoPE fused into it -- same page as the
  rotary code, §2.C (RoPE fused into the QKV projection).  The projection is
  the plain linear map y = x W^T (W stored [3*H*D, C], the usual linear-layer
  layout), columns ordered Q, K, V with heads contiguous; no bias.  The
  matrix product is numpy's (a library primitive); the rotation is the C
  oracle's.
* the log-sum-exp merge of two key subsets -- the exact identity
  attn(A u B) = merge(attn(A), attn(B)); it has no page of its own and is
  pinned by the tests against the oracle's own whole-set attention.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _ptr(a: np.ndarray, kind=_f64p):
    return a.ctypes.data_as(kind)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(status: int, what: str):
    if status != 0:
        raise ValueError(f"oracle {what}: status {status}")


def default_threads() -> int:
    """Host threads the oracle uses: OMP_NUM_THREADS if set, else all cores."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


class Oracle:
    """ctypes view of one compiled copy of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_split.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 3
        lib.oracle_split.restype = ctypes.c_int
        lib.oracle_rope_table.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.oracle_rope_table.restype = ctypes.c_int
        lib.oracle_positions.argtypes = [ctypes.c_int64] * 5 + [_i64p]
        lib.oracle_positions.restype = ctypes.c_int
        lib.oracle_rope_pos.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_int, _i64p, ctypes.c_double]
        lib.oracle_rope_pos.restype = ctypes.c_int
        lib.oracle_rope.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_double]
        lib.oracle_rope.restype = ctypes.c_int
        lib.oracle_append.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64]
        lib.oracle_append.restype = ctypes.c_int
        lib.oracle_attn.argtypes = [_f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, _f64p, _f64p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_double, _i64p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_attn.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def split(self, D: int) -> tuple[int, int, int]:
        """(D_t, D_h, D_w): h and w get 2*floor(D/6) dims each, t the rest."""
        a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(self.lib.oracle_split(D, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
               "split")
        return a.value, b.value, c.value

    def rope_table(self, D: int, max_t: int, max_h: int, max_w: int, theta: float = 10000.0):
        """fp64 (cos, sin) of p * theta^(-2j/D_a) for every axis a, position p < max_a
        and pair j < D_a/2; axis t first, then h, then w; p-major inside an axis."""
        dt, dh, dw = self.split(D)
        n = max_t * dt // 2 + max_h * dh // 2 + max_w * dw // 2
        c = np.empty(n, np.float64)
        s = np.empty(n, np.float64)
        _check(self.lib.oracle_rope_table(_ptr(c), _ptr(s), D, max_t, max_h, max_w, theta),
               "rope_table")
        return c, s

    def positions(self, n: int, t0: int, tok_off: int, grid_h: int, grid_w: int) -> np.ndarray:
        """[n, 3] int64 (p_t, p_h, p_w) of tokens tok_off .. tok_off+n-1 of a chunk
        whose first frame has global time index t0."""
        out = np.empty((n, 3), np.int64)
        _check(self.lib.oracle_positions(n, t0, tok_off, grid_h, grid_w, _ptr(out, _i64p)),
               "positions")
        return out

    def rope_pos(self, x, pos, theta: float = 10000.0) -> np.ndarray:
        """Rotate x [B, n, H, D] by explicit positions pos [n, 3]."""
        x = _f64(x)
        B, n, H, D = x.shape
        pos = np.ascontiguousarray(pos, dtype=np.int64)
        assert pos.shape == (n, 3)
        y = np.empty_like(x)
        _check(self.lib.oracle_rope_pos(_ptr(x), _ptr(y), B, n, H, D, _ptr(pos, _i64p), theta),
               "rope_pos")
        return y

    def rope(self, x, t0: int, tok_off: int, grid_h: int, grid_w: int,
             theta: float = 10000.0) -> np.ndarray:
        """Rotate x [B, n, H, D]: tokens tok_off.. of a chunk starting at frame t0."""
        x = _f64(x)
        B, n, H, D = x.shape
        y = np.empty_like(x)
        _check(self.lib.oracle_rope(_ptr(x), _ptr(y), B, n, H, D, t0, tok_off, grid_h, grid_w,
                                    theta), "rope")
        return y

    def append(self, cache: np.ndarray, x, cache_pos: int) -> None:
        """In place: cache[b, h, cache_pos + i, :] = x[b, i, h, :]; cache [B, H, cap, D]."""
        assert cache.dtype == np.float64 and cache.flags.c_contiguous
        x = _f64(x)
        B, n, H, D = x.shape
        assert cache.shape[0] == B and cache.shape[1] == H and cache.shape[3] == D
        _check(self.lib.oracle_append(_ptr(x), _ptr(cache), B, n, H, D, cache.shape[2],
                                      cache_pos), "append")

    def attn(self, q, k, v, kv_len: int, q_pos0: int, chunk_tokens: int,
             scale: float | None = None, rows=None, threads: int | None = None):
        """Chunk-causal attention.  q [B, Lq, H, D]; k, v [B, H, cap, D].

        Returns (o, lse): o [B, R, H, D] and lse [B, H, R] (natural log), with
        R = Lq, or R = len(rows) when a list of query rows is given.
        """
        q = _f64(q)
        k = _f64(k)
        v = _f64(v)
        B, Lq, H, D = q.shape
        assert k.shape == v.shape and k.shape[0] == B and k.shape[1] == H and k.shape[3] == D
        cap = k.shape[2]
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        if rows is None:
            R = Lq
            rows_p = ctypes.cast(None, _i64p)
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            R = rows_arr.shape[0]
            rows_p = _ptr(rows_arr, _i64p)
        o = np.empty((B, R, H, D), np.float64)
        lse = np.empty((B, H, R), np.float64)
        st = self.lib.oracle_attn(_ptr(q), _ptr(k), _ptr(v), cap, kv_len, q_pos0,
                                  chunk_tokens, _ptr(o), _ptr(lse), B, H, D, Lq, float(scale),
                                  rows_p, R, int(threads or default_threads()))
        _check(st, "attn")
        return o, lse


_default: Oracle | None = None


def _get() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build

            _build.build()
        _default = Oracle(_LIB_PATH)
    return _default


def split(D):
    return _get().split(D)


def rope_table(D, max_t, max_h, max_w, theta=10000.0):
    return _get().rope_table(D, max_t, max_h, max_w, theta)


def positions(n, t0, tok_off, grid_h, grid_w):
    return _get().positions(n, t0, tok_off, grid_h, grid_w)


def rope_pos(x, pos, theta=10000.0):
    return _get().rope_pos(x, pos, theta)


def rope(x, t0, tok_off, grid_h, grid_w, theta=10000.0):
    return _get().rope(x, t0, tok_off, grid_h, grid_w, theta)


def append(cache, x, cache_pos):
    return _get().append(cache, x, cache_pos)


def attn(q, k, v, kv_len, q_pos0, chunk_tokens, scale=None, rows=None, threads=None):
    return _get().attn(q, k, v, kv_len, q_pos0, chunk_tokens, scale, rows, threads)


def qkv_project(x, w, H, D):
    """y = x W^T split into Q, K, V of shape [B, n, H, D] (fp64).

    x: [B, n, C]; w: [3*H*D, C].  Columns [0, HD) are Q, [HD, 2HD) K and
    [2HD, 3HD) V; inside each, head h owns columns [h*D, (h+1)*D)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, n, C = x.shape
    assert w.shape == (3 * H * D, C)
    y = np.matmul(x.reshape(B * n, C), w.T).reshape(B, n, 3, H, D)
    return y[:, :, 0], y[:, :, 1], y[:, :, 2]


def qkv_rope(x, w, H, D, t0, tok_off, grid_h, grid_w, theta=10000.0):
    """The fused projection's outputs: rotated Q', rotated K' and V, each
    [B, n, H, D] fp64 (the caller rounds to the storage dtype and appends
    K', V to the cache)."""
    q, k, v = qkv_project(x, w, H, D)
    return (rope(np.ascontiguousarray(q), t0, tok_off, grid_h, grid_w, theta),
            rope(np.ascontiguousarray(k), t0, tok_off, grid_h, grid_w, theta), v)


def qkv_abs(x, w, H, D):
    """sum_c |x_c| |w_c| for every output of the projection (error bounds)."""
    return qkv_project(np.abs(x), np.abs(w), H, D)


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge attention over two disjoint key sets A and B.

    o_*: [B, R, H, D], lse_*: [B, H, R].  With lse = ln(e^lse_a + e^lse_b):
    o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.
    """
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.exp(lse_a - lse).transpose(0, 2, 1)[..., None]
    wb = np.exp(lse_b - lse).transpose(0, 2, 1)[..., None]
    return wa * o_a + wb * o_b, lse


def round_bf16(x) -> np.ndarray:
    """Round to bfloat16 (round to nearest even) and return as float64.

    Used where the HIP path stores bf16 (rotated Q/K, the cache, the output),
    so that the oracle consumes exactly the values the kernels consume.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
