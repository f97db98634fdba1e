"""The allocation-free attention entry point against chunk_causal_attn with a
caller workspace: two calls in a row on the library's fixed scratch, the
second smaller, each equal bit for bit to the workspace call and within the
bf16 attention bar of the oracle (sampled rows)."""
import numpy as np
import pytest
import torch

import autoregressive_video_diffusion_amd as crattn
import oracle
from gpu_helpers import assert_attn_close, dev, f64, sample_rows
from workloads import SP480, normal

pytestmark = pytest.mark.gpu


def _case(B, H, D, L, Lq, q_pos0, kv_len, cap, seed):
    q = normal((B, Lq, H, D), seed).to(dev())
    kc = normal((B, H, cap, D), seed + 1).to(dev())
    vc = normal((B, H, cap, D), seed + 2).to(dev())
    return q, kc, vc


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_the_workspace_call_twice(order):
    w = SP480
    cases = [
        # the SP-rank slice: 585 queries x 32760 keys, split-KV partials in scratch
        (w.B, w.H, w.D, w.chunk_tokens, w.lq, w.q_pos0, w.kv_len, w.cap, 910),
        # then a smaller call: 2 heads, 300 queries over 3000 keys of 1000-token chunks
        (1, 2, 128, 1000, 300, 2700, 3000, 3072, 920),
    ]
    for i, (B, H, D, L, Lq, q_pos0, kv_len, cap, seed) in enumerate(cases):
        print(f"  noalloc call {i}: B{B} H{H} D{D} Lq{Lq} kv_len{kv_len}", flush=True)
        need = crattn.chunk_causal_attn_workspace_bytes(B, H, Lq, kv_len, q_pos0, L, D)
        assert need > 0, "the case must use the scratch"
        q, kc, vc = _case(B, H, D, L, Lq, q_pos0, kv_len, cap, seed)
        ws = torch.full((need // 4 + 4,), float("nan"), dtype=torch.float32, device=dev())
        ref = torch.empty_like(q)
        ref_lse = torch.empty(B, H, Lq, dtype=torch.float32, device=dev())
        crattn.chunk_causal_attn(q, kc, vc, kv_len, q_pos0, L, ref, ref_lse, ws)
        out = torch.empty_like(q)
        lse = torch.empty_like(ref_lse)
        crattn.chunk_causal_attn_noalloc(q, kc, vc, kv_len, q_pos0, L, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), f"call {i}"
        rows = sample_rows(Lq, n_random=20, seed=i)
        o_ref, lse_ref = oracle.attn(f64(q), f64(kc), f64(vc), kv_len, q_pos0, L, rows=rows)
        assert_attn_close(f64(out[:, rows]), o_ref, f"noalloc call {i}")
        np.testing.assert_allclose(f64(lse[:, :, rows]), lse_ref, atol=2e-3)
