"""Host driver of the attention step of a chunk-by-chunk video rollout.

Self-Forcing-style generation produces a video chunk by chunk; each chunk is
denoised in several steps that attend to the KV cache of earlier chunks, then
a cache-update pass stores the chunk's clean K and V ("Wave Forcing"
abstract: the cache update is a second forward pass; "Accelerating Video
Generation Inference with Sequential-Parallel 3D Positional Encoding Using a
Global Time Index" §1: KV caching with rolling windows, §2.B: rotation from
the chunk's start frame).

Optionally the attention of each denoising step is the hierarchical
block-sparse attention of "LIGHT FORCING" §2.2 (HSA): the keys of each
chunk are mean-pooled per frame and per 64-token block when its clean K/V
are stored, and every denoising call keeps, per 256-row query block, the kf
best history frames and the kb best blocks inside them.

Or it is the semantic-permutation attention of "Sparse VideoGen2" §2: every
chunk slot's keys are clustered by k-means when its clean K/V are stored,
and every denoising call clusters the current chunk's keys and queries
(started from the previous call's centroids, §2.C), keeps for each query
cluster the key clusters of highest estimated share until p, and attends
over them.

This class only sequences the C-ABI calls; every step runs in the library's
kernels.  Cache layout: ``window`` chunk slots of ``chunk_tokens`` rows per
(batch, head); chunk c lives in slot c mod window.  While the ring fills, a
chunk's queries see slots 0..c (chunk-causal); once it is full they see every
slot, which is exact because attention does not depend on key order
("Sparse VideoGen2" §2.A).
"""
from __future__ import annotations

import torch

from . import (HSA_QBLOCK, chunk_causal_attn, chunk_causal_attn_workspace_bytes, hsa_attn,
               hsa_pool_bytes, hsa_pool_keys, hsa_select, rope_apply_append, rope_precompute,
               rope_table_bytes, svg2_attn, svg2_attn_workspace_bytes, svg2_kmeans,
               svg2_kmeans2, svg2_kmeans_workspace_bytes, svg2_n_slots, svg2_plan)


class ChunkRollout:
    def __init__(self, B: int, H: int, D: int, frames: int, grid_h: int, grid_w: int,
                 window: int, max_chunks: int, theta: float = 10000.0,
                 device: str | torch.device = "cuda", dtype: torch.dtype = torch.bfloat16,
                 hsa: tuple[int, int] | None = None,
                 svg2: tuple[int, int, float] | None = None, svg2_iters: int = 2,
                 svg2_splits: int = 2):
        """hsa = (kf, kb) switches the denoising attention to HSA with kf
        frames and kb blocks kept per query block; the selection's history is
        every visible slot but the chunk's own (the slots before it while the
        ring fills, all other slots once it is full).

        svg2 = (Cq, Ck, p) switches it to the semantic-permutation attention:
        Cq query clusters, Ck key clusters per chunk slot, top-p threshold p;
        svg2_iters Lloyd iterations per call from the cached centroids (3
        from tokens the first time a slot or the queries are clustered).
        Denoising calls then cover whole chunks."""
        if hsa is not None and svg2 is not None:
            raise ValueError("hsa and svg2 are alternatives")
        self.B, self.H, self.D = B, H, D
        self.frames, self.grid_h, self.grid_w = frames, grid_h, grid_w
        self.window = window
        self.L = frames * grid_h * grid_w
        self.cap = window * self.L
        self.max_t = max_chunks * frames
        self.dtype = dtype
        dev = torch.device(device)
        self.table = torch.empty(rope_table_bytes(D, self.max_t, grid_h, grid_w) // 4,
                                 dtype=torch.float32, device=dev)
        rope_precompute(self.table, D, self.max_t, grid_h, grid_w, theta)
        self.k_cache = torch.zeros(B, H, self.cap, D, dtype=dtype, device=dev)
        self.v_cache = torch.zeros(B, H, self.cap, D, dtype=dtype, device=dev)
        ws = max(self.workspace_bytes(c) for c in range(min(max_chunks, window + 1)))
        self.workspace = torch.empty(max(ws, 16) // 4 + 4, dtype=torch.float32, device=dev)
        self.hsa = hsa
        if hsa is not None:
            self.per_frame = grid_h * grid_w
            self.pool = torch.empty(hsa_pool_bytes(B, H, self.cap, D, self.per_frame) // 4,
                                    dtype=torch.float32, device=dev)
            self.sel = torch.empty(B, H, -(-self.L // HSA_QBLOCK), hsa[1], dtype=torch.int32,
                                   device=dev)
        self.svg2 = svg2
        if svg2 is not None:
            Cq, Ck, _ = svg2
            W, L = window, self.L
            self.svg2_iters, self.svg2_splits = svg2_iters, svg2_splits
            f32, i32 = dict(dtype=torch.float32, device=dev), dict(dtype=torch.int32, device=dev)
            self.kcent = torch.zeros(B, H, W, Ck, D, **f32)
            self.kperm = torch.zeros(B, H, W, L, **i32)
            self.koff = torch.zeros(B, H, W, Ck + 1, **i32)
            self.k_warm = [False] * W
            self.qcent = torch.zeros(B, H, Cq, D, **f32)
            self.qperm = torch.zeros(B, H, L, **i32)
            self.qoff = torch.zeros(B, H, Cq + 1, **i32)
            self.q_warm = False
            self.list_cap = -(-self.cap // 64) * 64
            self.lists = torch.empty(B, H, Cq, self.list_cap, **i32)
            self.llen = torch.empty(B, H, Cq, **i32)
            self.n_slots = svg2_n_slots(L, Cq)
            self.slots = torch.empty(B, H, self.n_slots, 4, **i32)
            self.ksel = torch.empty(B, H, Cq, W * Ck, **i32)
            kb = max(svg2_kmeans_workspace_bytes(B, H, L, Ck),
                     svg2_kmeans_workspace_bytes(B, H, L, Cq))
            self.ws_k = torch.empty(kb // 4 + 4, **f32)
            self.ws_q = torch.empty(kb // 4 + 4, **f32)
            self.ws_a = torch.empty(
                svg2_attn_workspace_bytes(B, H, L, D, self.n_slots, svg2_splits) // 4 + 4, **f32)
            self.side = torch.cuda.Stream(device=dev)  # default priority

    def slot(self, c: int) -> int:
        return c % self.window

    def t0(self, c: int) -> int:
        return c * self.frames

    def visible(self, c: int) -> tuple[int, int]:
        """(kv_len, q_pos0 of row 0) of chunk c's attention call."""
        if c < self.window:
            return (c + 1) * self.L, c * self.L
        return self.cap, (self.window - 1) * self.L

    def workspace_bytes(self, c: int, lq: int | None = None, tok_off: int = 0) -> int:
        kv_len, q0 = self.visible(c)
        return chunk_causal_attn_workspace_bytes(self.B, self.H, lq or self.L, kv_len,
                                                 q0 + tok_off, self.L, self.D)

    def rope_append(self, c: int, q, q_out, k, v, tok_off: int = 0):
        """Rotate Q (if given) and K of chunk c, write Q' and append K', V to
        the chunk's slot (one rope_apply_append call)."""
        rope_apply_append(q, q_out, k, v, self.k_cache, self.v_cache,
                          self.slot(c) * self.L + tok_off, self.table, self.max_t, self.grid_h,
                          self.grid_w, self.t0(c), tok_off, self.grid_h, self.grid_w)

    def _cluster_slot(self, c: int, stream=None):
        """k-means of chunk c's slot of keys, from its cached centroids once
        the slot has been clustered before."""
        s = self.slot(c)
        Ck = self.svg2[1]
        warm = self.k_warm[s]
        svg2_kmeans(self.k_cache[:, :, s * self.L:(s + 1) * self.L], Ck,
                    self.svg2_iters if warm else 3, not warm, self.kcent[:, :, s],
                    self.kperm[:, :, s], self.koff[:, :, s], self.ws_k, stream=stream)
        self.k_warm[s] = True

    def _svg2_attend(self, c: int, q_out, out, lse):
        Cq, _, p = self.svg2
        n_vis = min(c + 1, self.window)
        s = self.slot(c)
        if self.q_warm == self.k_warm[s]:
            # the queries' and the keys' k-means in one launch sequence
            warm, Ck, L = self.q_warm, self.svg2[1], self.L
            svg2_kmeans2((self.k_cache[:, :, s * L:(s + 1) * L], Ck, self.kcent[:, :, s],
                          self.kperm[:, :, s], self.koff[:, :, s], self.ws_k),
                         (q_out.permute(0, 2, 1, 3), Cq, self.qcent, self.qperm, self.qoff,
                          self.ws_q), self.svg2_iters if warm else 3, not warm)
            self.k_warm[s] = True
        else:
            main = torch.cuda.current_stream(q_out.device)
            # the queries' k-means on a second stream, beside the keys'
            self.side.wait_stream(main)
            svg2_kmeans(q_out.permute(0, 2, 1, 3), Cq, self.svg2_iters if self.q_warm else 3,
                        not self.q_warm, self.qcent, self.qperm, self.qoff, self.ws_q,
                        stream=self.side)
            self._cluster_slot(c)
            main.wait_stream(self.side)
        self.q_warm = True
        B, H, Ck = self.B, self.H, self.svg2[1]
        sel = self.ksel.view(-1)[:B * H * Cq * n_vis * Ck].view(B, H, Cq, n_vis * Ck)
        svg2_plan(self.qcent, self.qoff, self.kcent, self.koff, self.kperm, n_vis, self.L, p,
                  sel, self.lists, self.llen, self.slots)
        svg2_attn(q_out, self.k_cache, self.v_cache, self.qperm, self.slots, self.lists,
                  self.llen, out, lse, self.svg2_splits, self.ws_a)
        return out

    def denoise(self, c: int, q, k, v, q_out, out, lse=None, tok_off: int = 0):
        """One denoising step of chunk c: rotate Q/K, write the (noisy) K/V into
        the chunk's slot, attend.  q, k, v, q_out, out: [B, n, H, D]."""
        if self.svg2 is not None and (tok_off != 0 or q.shape[1] != self.L):
            raise NotImplementedError("semantic-permutation attention covers whole chunks")
        self.rope_append(c, q, q_out, k, v, tok_off)
        return self.attend(c, q_out, out, lse, tok_off)

    def attend(self, c: int, q_out, out, lse=None, tok_off: int = 0):
        """The attention of a denoising step of chunk c on its rotated
        queries q_out (dense, HSA or semantic-permutation)."""
        kv_len, q0 = self.visible(c)
        if self.svg2 is not None:
            return self._svg2_attend(c, q_out, out, lse)
        if self.hsa is None:
            chunk_causal_attn(q_out, self.k_cache, self.v_cache, kv_len, q0 + tok_off, self.L,
                              out, lse, self.workspace)
            return out
        # HSA: the own chunk is the chunk's actual slot (the dense call's
        # "last slot" convention would put it elsewhere in a full ring)
        n = q_out.shape[1]
        sel = self.sel[:, :, :-(-n // HSA_QBLOCK)].contiguous() if n != self.L else self.sel
        own = self.slot(c) * self.L + tok_off
        hsa_select(q_out, self.pool, self.cap, kv_len, self.per_frame, own, self.L,
                   self.hsa[0], self.hsa[1], sel)
        hsa_attn(q_out, self.k_cache, self.v_cache, kv_len, own, self.L, self.per_frame, sel,
                 out, lse)
        return out

    def update(self, c: int, k, v, tok_off: int = 0):
        """Cache update of chunk c: rotate the clean K and store it with V
        (and, with HSA, pool the chunk's keys once the whole chunk is in)."""
        self.rope_append(c, None, None, k, v, tok_off)
        if self.hsa is not None and tok_off + k.shape[1] == self.L:
            hsa_pool_keys(self.k_cache, self.slot(c) * self.L, self.L, self.per_frame, self.pool)
        if self.svg2 is not None and tok_off + k.shape[1] == self.L:
            self._cluster_slot(c)
