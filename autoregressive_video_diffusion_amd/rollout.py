"""Host driver of the attention step of a chunk-by-chunk video rollout.

Self-Forcing-style generation produces a video chunk by chunk; each chunk is
denoised in several steps that attend to the KV cache of earlier chunks, then
a cache-update pass stores the chunk's clean K and V ("Wave Forcing"
abstract: the cache update is a second forward pass; "Accelerating Video
Generation Inference with Sequential-Parallel 3D Positional Encoding Using a
Global Time Index" §1: KV caching with rolling windows, §2.B: rotation from
the chunk's start frame).

This class only sequences the C-ABI calls; every step runs in the library's
kernels.  Cache layout: ``window`` chunk slots of ``chunk_tokens`` rows per
(batch, head); chunk c lives in slot c mod window.  While the ring fills, a
chunk's queries see slots 0..c (chunk-causal); once it is full they see every
slot, which is exact because attention does not depend on key order
("Sparse VideoGen2" §2.A).
"""
from __future__ import annotations

import torch

from . import (chunk_causal_attn, chunk_causal_attn_workspace_bytes, rope_apply_append,
               rope_precompute, rope_table_bytes)


class ChunkRollout:
    def __init__(self, B: int, H: int, D: int, frames: int, grid_h: int, grid_w: int,
                 window: int, max_chunks: int, theta: float = 10000.0,
                 device: str | torch.device = "cuda", dtype: torch.dtype = torch.bfloat16):
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
        self._rope(c, q, q_out, k, v, tok_off)
        kv_len, q0 = self.visible(c)
        chunk_causal_attn(q_out, self.k_cache, self.v_cache, kv_len, q0 + tok_off, self.L, out,
                          lse, self.workspace)
        return out

    def update(self, c: int, k, v, tok_off: int = 0):
        """Cache update of chunk c: rotate the clean K and store it with V."""
        self._rope(c, None, None, k, v, tok_off)
