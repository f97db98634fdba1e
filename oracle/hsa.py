"""CPU reference (fp64) for hierarchical block-sparse chunk-causal attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.

Source: "LIGHT FORCING" technical summary, §2.2 (Hierarchical Sparse
Attention, HSA): queries and keys are compressed by mean pooling at block
and at frame level; for every query block a few history frames are chosen
with the frame-level keys, then the critical blocks inside those frames
with the block-level keys; attention is computed over the chosen blocks
only, so its cost does not grow with the number of history frames.

Readings of what the page leaves open (each is stated where it is used):

* Key blocks are runs of ``bk`` consecutive tokens inside one frame (raster
  order), the last block of a frame holding the remainder; a frame is
  ``per_frame`` tokens and frames are consecutive in the cache.
* Query blocks are runs of ``bq`` consecutive query rows of the call.
* History = the frames of the visible cache rows [0, kv_len) outside the
  query's own chunk.  While a ring of chunk slots fills, the own chunk is
  the last visible slot and the history is the chunks before it; once the
  ring is full, every other slot is history, whatever its position in the
  ring (attention does not depend on key order, "Sparse VideoGen2" §2.A).
  The query's own chunk is always attended in full (attention inside a
  chunk is bidirectional and dense); selection applies to history only.
  Candidate frames are ranked in ascending frame order (ties go to the
  lower frame).
* Scores are plain dot products of the pooled vectors (a positive scale
  does not change a top-k).  Top-k keeps the k largest scores; equal scores
  are ordered by the lower index first.
* The block candidates are all blocks of the selected frames; the kb best
  of them are kept (one top-k over the union, not kb per frame).
* The final attention is the chunk-causal softmax attention restricted to
  the own chunk plus the selected blocks (two-pass softmax, fp64).
"""
from __future__ import annotations

import numpy as np


def blocks_per_frame(per_frame: int, bk: int = 64) -> int:
    return -(-per_frame // bk)


def block_range(block: int, per_frame: int, bk: int = 64) -> tuple[int, int]:
    """Cache rows [start, end) of global block id `block` (frame-major)."""
    nbf = blocks_per_frame(per_frame, bk)
    f, j = divmod(block, nbf)
    start = f * per_frame + j * bk
    return start, min(start + bk, (f + 1) * per_frame)


def pool_keys(k: np.ndarray, per_frame: int, bk: int = 64):
    """k: [B, H, rows, D] with rows a whole number of frames.  Returns the
    frame means [B, H, nf, D] and the block means [B, H, nf * nbf, D]."""
    k = np.asarray(k, dtype=np.float64)
    B, H, rows, D = k.shape
    if rows % per_frame:
        raise ValueError("rows must be whole frames")
    nf, nbf = rows // per_frame, blocks_per_frame(per_frame, bk)
    frames = k.reshape(B, H, nf, per_frame, D).mean(axis=3)
    blocks = np.empty((B, H, nf * nbf, D))
    for blk in range(nf * nbf):
        s, e = block_range(blk, per_frame, bk)
        blocks[:, :, blk] = k[:, :, s:e].mean(axis=2)
    return frames, blocks


def pool_queries(q: np.ndarray, bq: int = 256) -> np.ndarray:
    """q: [B, Lq, H, D] -> [B, H, ceil(Lq / bq), D], the mean of each run of
    bq rows (the last run holds the remainder)."""
    q = np.asarray(q, dtype=np.float64)
    B, Lq, H, D = q.shape
    nqb = -(-Lq // bq)
    out = np.empty((B, H, nqb, D))
    for i in range(nqb):
        out[:, :, i] = q[:, i * bq:min(Lq, (i + 1) * bq)].mean(axis=1)
    return out


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores (all of them if fewer), larger score
    first and, among equal scores, lower index first; returned ascending."""
    scores = np.asarray(scores, dtype=np.float64)
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def history_frames(kv_len: int, q_pos0: int, chunk_tokens: int, per_frame: int) -> np.ndarray:
    """Frame ids of the history of a call whose row 0 sits at q_pos0: every
    whole frame of the visible rows [0, kv_len) outside the own chunk
    (chunk q_pos0 // chunk_tokens), ascending."""
    if kv_len % per_frame or chunk_tokens % per_frame:
        raise ValueError("kv_len and chunk_tokens must be whole frames")
    own = q_pos0 // chunk_tokens
    fc = chunk_tokens // per_frame
    return np.array([f for f in range(kv_len // per_frame) if f // fc != own], dtype=np.int64)


def select(q: np.ndarray, k_frames: np.ndarray, k_blocks: np.ndarray, hist,
           per_frame: int, kf: int, kb: int, bq: int = 256, bk: int = 64):
    """Two-level selection for every (b, h, query block).

    q: [B, Lq, H, D] rotated queries of the call; k_frames / k_blocks: pooled
    keys (pool_keys); hist: the history frame ids (history_frames), or an
    int n meaning frames 0..n-1 (the own chunk after them).
    Returns sel [B, H, nqb, kb] int64: the chosen block ids ascending, padded
    with -1 when fewer than kb blocks exist in the chosen frames."""
    hist = (np.arange(hist, dtype=np.int64) if np.isscalar(hist)
            else np.asarray(hist, dtype=np.int64))
    nbf = blocks_per_frame(per_frame, bk)
    qp = pool_queries(q, bq)
    B, H, nqb, _ = qp.shape
    sel = np.full((B, H, nqb, kb), -1, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                if len(hist) == 0:
                    continue
                # candidate c is history frame hist[c]: ranked in ascending
                # frame order, so ties go to the lower frame
                fs = k_frames[b, h, hist] @ qp[b, h, i]
                frames = hist[topk(fs, kf)]
                cand = np.concatenate([np.arange(f * nbf, (f + 1) * nbf) for f in frames])
                bs = k_blocks[b, h, cand] @ qp[b, h, i]
                chosen = cand[topk(bs, kb)]
                sel[b, h, i, :len(chosen)] = np.sort(chosen)
    return sel


def visible_keys(sel_row: np.ndarray, own_begin: int, own_end: int, per_frame: int,
                 bk: int = 64) -> np.ndarray:
    """Cache rows a query attends to: its own chunk [own_begin, own_end) and
    every row of the selected blocks (ids >= 0), ascending."""
    parts = [np.arange(own_begin, own_end)]
    for blk in sel_row:
        if blk >= 0:
            s, e = block_range(int(blk), per_frame, bk)
            parts.append(np.arange(s, e))
    return np.sort(np.concatenate(parts))


def attn(q, k, v, sel, own_begin: int, own_end: int, per_frame: int, bq: int = 256,
         bk: int = 64, scale=None, rows=None):
    """Attention of each query row over its own chunk plus its query block's
    selected blocks: two-pass softmax in fp64.

    q: [B, Lq, H, D]; k, v: [B, H, cap, D]; sel: [B, H, nqb, kb].
    Returns o [B, len(rows), H, D] and lse [B, H, len(rows)] (natural log)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Lq, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    o = np.empty((B, len(rows), H, D))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            cache = {}
            for n, r in enumerate(rows):
                qb = int(r) // bq
                if qb not in cache:
                    cache[qb] = visible_keys(sel[b, h, qb], own_begin, own_end, per_frame, bk)
                keys = cache[qb]
                s = (k[b, h, keys] @ q[b, r, h]) * scale
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                o[b, n, h] = (p @ v[b, h, keys]) / l
                lse[b, h, n] = m + np.log(l)
    return o, lse
