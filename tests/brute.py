"""Brute-force NumPy forms of RoPE and chunk-causal attention, for tiny inputs.

These are written independently of ``oracle/`` (no shared code) and in a
different shape: RoPE as an explicit D x D block-diagonal rotation matrix per
token, attention as a full masked score matrix with a dense softmax.  They
exist only to pin the oracle on small cases.
"""
from __future__ import annotations

import numpy as np


def axis_dims(D: int) -> list[int]:
    hw = 2 * (D // 6)
    return [D - 2 * hw, hw, hw]


def rotation_matrix(D: int, p_t: int, p_h: int, p_w: int, theta: float = 10000.0) -> np.ndarray:
    """D x D block-diagonal matrix: one 2 x 2 rotation per adjacent feature pair."""
    R = np.zeros((D, D))
    base = 0
    for Da, p in zip(axis_dims(D), (p_t, p_h, p_w)):
        for j in range(Da // 2):
            ang = p * theta ** (-(2.0 * j) / Da)
            c, s = np.cos(ang), np.sin(ang)
            r = base + 2 * j
            R[r, r], R[r, r + 1] = c, -s
            R[r + 1, r], R[r + 1, r + 1] = s, c
        base += Da
    return R


def raster_positions(n: int, t0: int, tok_off: int, gh: int, gw: int) -> np.ndarray:
    """Enumerate the chunk in raster order (frame, row, column) by nested loops,
    then take tokens tok_off .. tok_off + n - 1."""
    out = []
    f = 0
    while len(out) < tok_off + n:
        for r in range(gh):
            for c in range(gw):
                out.append((t0 + f, r, c))
        f += 1
    return np.array(out[tok_off:tok_off + n], dtype=np.int64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """x [B, n, H, D] -> R(pos_i) x[b, i, h] for every token, via the matrix."""
    B, n, H, D = x.shape
    y = np.empty_like(x, dtype=np.float64)
    for i in range(n):
        R = rotation_matrix(D, *pos[i], theta=theta)
        y[:, i] = np.einsum("ed,bhd->bhe", R, x[:, i])
    return y


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_len: int, q_pos0: int,
              chunk_tokens: int, scale: float):
    """Full score matrix with -inf outside the chunk-causal mask, dense softmax.

    q [B, Lq, H, D], k/v [B, H, cap, D] -> o [B, Lq, H, D], lse [B, H, Lq].
    """
    B, Lq, H, D = q.shape
    kk = k[:, :, :kv_len]
    vv = v[:, :, :kv_len]
    qi = (q_pos0 + np.arange(Lq))[:, None] // chunk_tokens
    kj = np.arange(kv_len)[None, :] // chunk_tokens
    mask = kj <= qi                                         # [Lq, kv_len]
    S = np.einsum("bihd,bhjd->bhij", q, kk) * scale         # [B, H, Lq, kv_len]
    S = np.where(mask[None, None], S, -np.inf)
    mx = S.max(axis=-1, keepdims=True)
    E = np.exp(S - mx)
    Z = E.sum(axis=-1, keepdims=True)
    P = E / Z
    o = np.einsum("bhij,bhjd->bihd", P, vv)
    lse = (mx + np.log(Z))[..., 0]
    return o, lse, P
