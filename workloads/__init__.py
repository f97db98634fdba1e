"""Synthetic workloads and seeded input generators.

This module holds shapes, seeds and random draws only -- none of the
method's arithmetic.  Both the HIP path and the CPU oracle receive the
identical host tensors it produces.

The shapes are those of Wan2.1-class 480P/720P video latents, as used by the
Causal-RoPE SP, Wave Forcing and Light Forcing pages: a chunk is F latent
frames of a Gh x Gw token grid, tokens in raster order (frame, row, column).
Every tensor is N(0, 1) float32 from a CPU ``torch.Generator``; bf16 tensors
are the float32 draw rounded to nearest even.  Seeds: 1000 * workload_index +
call_index for the per-call Q, K, V (drawn in that order), and
1000 * workload_index + 999 for the prior-chunk cache contents.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # seed namespace
    B: int
    H: int
    D: int
    frames: int           # latent frames per chunk
    grid_h: int
    grid_w: int
    t0: int               # global time index of the current chunk's first frame
    slot: int             # cache slot (in chunks) the current chunk is appended to
    kv_chunks: int        # chunks present in the cache, own chunk included
    lq: int               # query rows in the call
    tok_off: int          # chunk-local raster index of the first query token
    dtype: str            # "f32" (RoPE/append in fp32) or "bf16"
    window: bool = False  # ring window: every cached key is visible
    theta: float = 10000.0
    note: str = field(default="", compare=False)

    @property
    def chunk_tokens(self) -> int:
        return self.frames * self.grid_h * self.grid_w

    @property
    def cap(self) -> int:
        return self.kv_chunks * self.chunk_tokens

    @property
    def kv_len(self) -> int:
        return self.kv_chunks * self.chunk_tokens

    @property
    def cache_pos(self) -> int:
        return self.slot * self.chunk_tokens + self.tok_off

    @property
    def q_pos0(self) -> int:
        # in a ring window the current chunk may sit in any slot; attention
        # then sees every slot, which the last-slot position expresses
        last = (self.kv_chunks - 1) if self.window else self.slot
        return last * self.chunk_tokens + self.tok_off

    def table_extents(self) -> tuple[int, int, int]:
        """(max_t, max_h, max_w) the RoPE table must cover."""
        return (self.t0 + self.frames, self.grid_h, self.grid_w)


TINY = Workload("tiny_fp32_8x8_4chunks", 0, B=1, H=2, D=64, frames=1, grid_h=8, grid_w=8,
                t0=3, slot=3, kv_chunks=4, lq=64, tok_off=0, dtype="f32",
                note="2 heads, head_dim 64, 4 one-frame chunks of 8x8 tokens; last chunk queries")
STEP480 = Workload("wan1.3b_480p_chunk_step", 1, B=1, H=12, D=128, frames=3, grid_h=30,
                   grid_w=52, t0=18, slot=6, kv_chunks=7, lq=4680, tok_off=0, dtype="bf16",
                   note="12 heads, D 128, 3x30x52 chunk (4680 queries) vs 32760 keys, t0 18")
ROLLOUT480 = Workload("wan1.3b_480p_rollout", 2, B=1, H=12, D=128, frames=3, grid_h=30,
                      grid_w=52, t0=0, slot=0, kv_chunks=7, lq=4680, tok_off=0, dtype="bf16",
                      note="7 chunks in order, 4 denoising attention calls + 1 cache update each")
SP480 = Workload("wan1.3b_480p_sp_rank_slice", 3, B=1, H=12, D=128, frames=3, grid_h=30,
                 grid_w=52, t0=18, slot=6, kv_chunks=7, lq=585, tok_off=2925, dtype="bf16",
                 note="one sequence-parallel rank: 585 queries at chunk offset 2925")
WIN720 = Workload("wan14b_720p_window", 4, B=1, H=40, D=128, frames=3, grid_h=45, grid_w=80,
                  t0=81, slot=6, kv_chunks=7, lq=10800, tok_off=0, dtype="bf16", window=True,
                  note="40 heads, 3x45x80 chunk (10800 queries), 7-chunk ring window, t0 81")

ALL = (TINY, STEP480, ROLLOUT480, SP480, WIN720)
BY_NAME = {w.name: w for w in ALL}


def normal(shape, seed: int, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """N(0, 1) float32 draw from a seeded CPU generator, cast to dtype (RNE)."""
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def call_qkv(w: Workload, call_index: int, n: int | None = None, dtype=None):
    """Per-call Q, K, V [B, n, H, D], drawn in that order from one generator."""
    n = w.lq if n is None else n
    dt = dtype or torch_dtype(w)
    g = torch.Generator().manual_seed(1000 * w.index + call_index)
    out = []
    for _ in range(3):
        x = torch.randn(w.B, n, w.H, w.D, generator=g, dtype=torch.float32)
        out.append(x if dt == torch.float32 else x.to(dt))
    return tuple(out)


def prior_cache(w: Workload, dtype=None):
    """Cache contents [B, H, cap, D] for K and V, treated as already rotated."""
    dt = dtype or torch_dtype(w)
    g = torch.Generator().manual_seed(1000 * w.index + 999)
    out = []
    for _ in range(2):
        x = torch.randn(w.B, w.H, w.cap, w.D, generator=g, dtype=torch.float32)
        out.append(x if dt == torch.float32 else x.to(dt))
    return tuple(out)


def projection_inputs(w: Workload, call_index: int, hidden: int | None = None):
    """Hidden states x [B, lq, C] (N(0, 1)) and a QKV weight [3*H*D, C]
    (N(0, 1) / sqrt(C)), bf16, C = H*D unless given (the Wan-class models
    have hidden size = heads x head_dim)."""
    C = w.H * w.D if hidden is None else hidden
    g = torch.Generator().manual_seed(1000 * w.index + 500 + call_index)
    x = torch.randn(w.B, w.lq, C, generator=g, dtype=torch.float32).to(torch.bfloat16)
    wt = (torch.randn(3 * w.H * w.D, C, generator=g, dtype=torch.float32) / C ** 0.5)
    return x, wt.to(torch.bfloat16)



def planted_clusters(batch_shape, n: int, C: int, D: int, seed: int, spread: float = 0.05,
                     dtype: torch.dtype = torch.bfloat16):
    """Tokens grouped around C centres: x [*batch_shape, n, D] and the centre
    of every token, labels [*batch_shape, n] (int64).  Centres ~ N(0, 1);
    each token = its centre + spread * N(0, 1).  Token floor(c n / C) belongs
    to centre c, every other token to a uniformly drawn centre, so every
    centre has at least one token and the tokens of a centre are scattered
    over the sequence."""
    g = torch.Generator().manual_seed(int(seed))
    nb = 1
    for s in batch_shape:
        nb *= int(s)
    centres = torch.randn(nb, C, D, generator=g, dtype=torch.float32)
    labels = torch.randint(0, C, (nb, n), generator=g)
    labels[:, [c * n // C for c in range(C)]] = torch.arange(C)
    noise = torch.randn(nb, n, D, generator=g, dtype=torch.float32)
    x = torch.gather(centres, 1, labels[..., None].expand(nb, n, D)) + spread * noise
    x = x.reshape(*batch_shape, n, D)
    return (x if dtype == torch.float32 else x.to(dtype)), labels.reshape(*batch_shape, n)


def clustered_qk(w: Workload, n_qc: int = 20, n_kc: int = 64, scale: float = 1.6,
                 noise: float = 0.3, seed: int = 0):
    """Queries and cache keys with semantic structure: in every head the
    chunk's queries fall into n_qc groups and every chunk slot's keys into
    n_kc groups (planted_clusters), each token = scale * (its group's N(0, 1)
    centre) + noise * N(0, 1).  Returns q [B, lq, H, D] and k [B, H, cap, D]
    (bf16; every slot of the cache filled)."""
    L = w.chunk_tokens
    qh, _ = planted_clusters((w.B, w.H), w.lq, n_qc, w.D, 7000 + seed, spread=noise / scale,
                             dtype=torch.float32)
    q = (qh * scale).permute(0, 2, 1, 3).contiguous().to(torch.bfloat16)
    k = torch.empty(w.B, w.H, w.cap, w.D, dtype=torch.bfloat16)
    for s in range(w.cap // L):
        kh, _ = planted_clusters((w.B, w.H), L, n_kc, w.D, 7100 + seed + s, spread=noise / scale,
                                 dtype=torch.float32)
        k[:, :, s * L:(s + 1) * L] = (kh * scale).to(torch.bfloat16)
    return q, k
