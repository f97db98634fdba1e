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
               rope_table_bytes)


class ChunkRollout:
    def __init__(self, B: int, H: int, D: int, frames: int, grid_h: int, grid_w: int,
                 window: int, max_chunks: int, theta: float = 10000.0,
                 device: str | torch.device = "cuda", dtype: torch.dtype = torch.bfloat16,
                 hsa: tuple[int, int] | None = None):
        """hsa = (kf, kb) switches the denoising attention to HSA with kf
        frames and kb blocks kept per query block (chunks 0 .. window-1: the
        selection's history is the slots before the chunk's own)."""
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

    def _rope(self, c, q, q_out, k, v, tok_off):
        rope_apply_append(q, q_out, k, v, self.k_cache, self.v_cache,
                          self.slot(c) * self.L + tok_off, self.table, self.max_t, self.grid_h,
                          self.grid_w, self.t0(c), tok_off, self.grid_h, self.grid_w)

    def denoise(self, c: int, q, k, v, q_out, out, lse=None, tok_off: int = 0):
        """One denoising step of chunk c: rotate Q/K, write the (noisy) K/V into
        the chunk's slot, attend.  q, k, v, q_out, out: [B, n, H, D]."""
        if self.hsa is not None and c >= self.window:
            raise NotImplementedError("HSA in a full ring window: the selection's history is "
                                      "the slots before the chunk's own")
        self._rope(c, q, q_out, k, v, tok_off)
        kv_len, q0 = self.visible(c)
        if self.hsa is None:
            chunk_causal_attn(q_out, self.k_cache, self.v_cache, kv_len, q0 + tok_off, self.L,
                              out, lse, self.workspace)
            return out
        n = q_out.shape[1]
        sel = self.sel[:, :, :-(-n // HSA_QBLOCK)].contiguous() if n != self.L else self.sel
        hsa_select(q_out, self.pool, self.cap, self.per_frame, q0 + tok_off, self.L,
                   self.hsa[0], self.hsa[1], sel)
        hsa_attn(q_out, self.k_cache, self.v_cache, q0 + tok_off, self.L, self.per_frame, sel,
                 out, lse)
        return out

    def update(self, c: int, k, v, tok_off: int = 0):
        """Cache update of chunk c: rotate the clean K and store it with V
        (and, with HSA, pool the chunk's keys once the whole chunk is in)."""
        self._rope(c, None, None, k, v, tok_off)
        if self.hsa is not None and tok_off + k.shape[1] == self.L:
            hsa_pool_keys(self.k_cache, self.slot(c) * self.L, self.L, self.per_frame, self.pool)
