"""CPU reference (fp64) for semantic-aware permutation with centroid top-p
sparse attention, inside a chunk-by-chunk rollout with a KV cache.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` use it; the product library never
loads it and shares no code with it.

Source: "Sparse VideoGen2" summary, §2.A-§2.C.  Queries and keys are
clustered separately by k-means; tokens are reordered so that every cluster
is contiguous; attention scores are estimated between cluster centroids;
each query cluster takes key clusters in decreasing estimated score until
their cumulative share reaches p; attention then runs over the selected
clusters, dense over the contiguous queries of a cluster, loading the
selected keys sparsely; the previous denoising step's centroids may start
k-means.  Full attention is unchanged by the reordering (§2.A).

Readings of what the page leaves open:

* k-means is Lloyd's algorithm with squared Euclidean distance on the raw
  vectors of one (batch, head): each iteration assigns every token to its
  nearest centroid (the lowest index on a tie), then moves every centroid
  to the mean of its tokens; an empty cluster keeps its centroid.  Without
  a previous step's centroids, centroid c starts at token floor(c n / C).
* The reordering is the stable sort of the tokens by cluster id: cluster c
  owns rows offsets[c] .. offsets[c+1] of the reordered sequence, its tokens
  in ascending order.
* Keys are clustered per chunk of the cache (each chunk slot holds its own
  C_k clusters of its own rows): a chunk's clean keys never change once
  stored, so their clusters are made once, when the chunk is stored, and
  only the current chunk's keys are clustered again at each denoising call.
  The candidates of a call are the clusters of every visible chunk.
* The estimated share of key cluster j for a query cluster with centroid
  qc is n_j exp(scale qc . kc_j), normalised over the non-empty candidate
  clusters (every one of the cluster's n_j keys is stood in for by the
  centroid), scale = 1/sqrt(D) as in the attention.  Clusters are taken in
  decreasing share, the lower id first on a tie, until the cumulative share
  reaches p; at least one is taken.  Candidate j is cluster j mod C_k of
  visible chunk slot j div C_k.
* Every query of a cluster attends to every key of the selected clusters,
  and to nothing else (no separate causal rule: the candidates are the
  visible chunks only).
"""
from __future__ import annotations

import numpy as np


def kmeans(x: np.ndarray, C: int, iters: int, init: np.ndarray | None = None):
    """x: [n, D] tokens of one (batch, head).  Returns (centroids [C, D],
    assign [n]) after `iters` Lloyd iterations: centroids are the means of
    the final assignment's clusters (empty clusters keep theirs)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    cent = (x[[c * n // C for c in range(C)]].copy() if init is None
            else np.array(init, dtype=np.float64))
    assign = np.zeros(n, dtype=np.int64)
    for _ in range(iters):
        d = ((x[:, None, :] - cent[None, :, :]) ** 2).sum(-1)
        assign = d.argmin(axis=1)  # first minimum: the lowest index on a tie
        for c in range(C):
            members = x[assign == c]
            if len(members):
                cent[c] = members.mean(axis=0)
    return cent, assign


def permutation(assign: np.ndarray, C: int):
    """Stable sort by cluster: perm[r] = token at reordered row r; offsets
    [C + 1] bound each cluster's rows."""
    assign = np.asarray(assign)
    perm = np.argsort(assign, kind="stable")
    counts = np.bincount(assign, minlength=C)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return perm, offsets


def cluster(x: np.ndarray, C: int, iters: int, init: np.ndarray | None = None):
    """k-means then the reordering: (centroids, perm, offsets)."""
    cent, assign = kmeans(x, C, iters, init)
    perm, off = permutation(assign, C)
    return cent, perm, off


def shares(qc: np.ndarray, kc: np.ndarray, counts: np.ndarray, scale: float) -> np.ndarray:
    """Estimated attention share of every candidate cluster (0 for empty
    ones) for the query centroid qc."""
    counts = np.asarray(counts)
    live = counts > 0
    z = np.full(len(counts), -np.inf)
    z[live] = scale * (np.asarray(kc, dtype=np.float64)[live] @ np.asarray(qc, dtype=np.float64))
    w = np.zeros(len(counts))
    w[live] = counts[live] * np.exp(z[live] - z[live].max())
    return w / w.sum()


def select_top_p(qc: np.ndarray, kc: np.ndarray, counts: np.ndarray, p: float,
                 scale: float) -> np.ndarray:
    """Candidate clusters kept for one query centroid: ascending ids."""
    w = shares(qc, kc, counts, scale)
    order = sorted(np.flatnonzero(np.asarray(counts) > 0), key=lambda j: (-w[j], j))
    cum, kept = 0.0, []
    for j in order:
        kept.append(j)
        cum += w[j]
        if cum >= p:
            break
    return np.array(sorted(kept), dtype=np.int64)


def key_list(sel: np.ndarray, key_slots, Ck: int) -> np.ndarray:
    """Cache rows of the selected candidates, cluster by cluster in ascending
    id.  key_slots[s] = (centroids, perm, offsets, first cache row)."""
    parts = []
    for j in sel:
        _, perm, off, base = key_slots[j // Ck]
        c = j % Ck
        parts.append(base + np.asarray(perm[off[c]:off[c + 1]], dtype=np.int64))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def plan(qc: np.ndarray, q_perm: np.ndarray, q_off: np.ndarray, key_slots, Ck: int, p: float,
         scale: float):
    """For every non-empty query cluster: (its query rows, the cache rows it
    attends to, the selected candidate ids)."""
    kc = np.concatenate([np.asarray(s[0], dtype=np.float64) for s in key_slots])
    counts = np.concatenate([np.diff(s[2]) for s in key_slots])
    groups = []
    for i in range(len(q_off) - 1):
        rows = np.asarray(q_perm[q_off[i]:q_off[i + 1]], dtype=np.int64)
        if len(rows) == 0:
            continue
        sel = select_top_p(qc[i], kc, counts, p, scale)
        groups.append((rows, key_list(sel, key_slots, Ck), sel))
    return groups


def attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, groups, scale=None):
    """Attention of one (batch, head): q [Lq, D], k, v [cap, D]; each group
    (rows, keys, ...) attends its query rows to its key rows.  Two-pass
    softmax in fp64; returns o [Lq, D] and lse [Lq] (natural log) in the
    original query order (rows in no group stay NaN)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    Lq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    o = np.full((Lq, D), np.nan)
    lse = np.full(Lq, np.nan)
    for g in groups:
        rows, keys = g[0], g[1]
        s = (q[rows] @ k[keys].T) * scale
        m = s.max(axis=1, keepdims=True)
        pr = np.exp(s - m)
        l = pr.sum(axis=1, keepdims=True)
        o[rows] = (pr @ v[keys]) / l
        lse[rows] = (m + np.log(l))[:, 0]
    return o, lse
