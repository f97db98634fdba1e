"""Shared pieces of the GPU parity tests: device setup, tolerance checks and
conversions between device tensors and the oracle's float64 arrays."""
from __future__ import annotations

import numpy as np
import torch

import autoregressive_video_diffusion_amd as crattn

# bf16 attention tolerances (max-abs and relative L2 against the fp64 oracle)
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
# fp32 RoPE tolerance (absolute)
ROPE_F32_ABS = 1e-5


def dev():
    return torch.device("cuda:0")


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def table(D, max_t, max_h, max_w, theta=10000.0):
    t = torch.empty(crattn.rope_table_bytes(D, max_t, max_h, max_w) // 4, dtype=torch.float32,
                    device=dev())
    crattn.rope_precompute(t, D, max_t, max_h, max_w, theta)
    return t


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at the magnitude of x (x rounded to fp32)."""
    return np.spacing(np.abs(x).astype(np.float32)).astype(np.float64) * 65536.0


def assert_rope_bf16(got: np.ndarray, exact: np.ndarray, x: np.ndarray):
    """bf16 RoPE output within one bf16 ulp of the exact rotation, plus the
    fp32 evaluation error with fp32 cos/sin tables: each table entry carries
    up to 2^-25 absolute error and the products and sum up to 2^-24 relative
    each, so |error| <= 2^-22 * (|x| + |y|) for the input pair (x, y).  The
    second term only matters when the rotated value nearly cancels."""
    xa = np.abs(x)
    pair = xa[..., 0::2] + xa[..., 1::2]
    fp32_err = np.repeat(pair, 2, axis=-1) * 2.0 ** -22
    err = np.abs(got - exact)
    tol = np.maximum(bf16_ulp(exact), 2.0 ** -126) + fp32_err
    bad = err > tol
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} values outside one bf16 ulp + fp32 "
                           f"error; worst {float((err / tol).max()):.2f}x the bound")
    within_ulp = (err <= bf16_ulp(exact)).mean()
    assert within_ulp > 0.9999, within_ulp


def attn_errors(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    d = got - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    mx, rel = attn_errors(got, ref)
    print(f"  {what}: max-abs {mx:.3e} rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert mx <= ATTN_MAX_ABS and rel <= ATTN_REL_L2, (what, mx, rel)


def sample_rows(Lq: int, n_random: int = 40, seed: int = 0, bm: int = 256) -> np.ndarray:
    """Query rows spanning tile starts/ends, both halves of a wavefront, the
    ragged tail and a seeded random set."""
    fixed = {0, 1, 31, 32, 33, 63, 64, 127, 128, 255, Lq - 1, Lq - 2, Lq - 33}
    fixed |= {(Lq // bm) * bm, (Lq // bm) * bm - 1}
    rng = np.random.default_rng(seed)
    fixed |= set(rng.integers(0, Lq, n_random).tolist())
    return np.array(sorted(r for r in fixed if 0 <= r < Lq), dtype=np.int64)
