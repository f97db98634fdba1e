"""GPU checks of chunk_causal_attn_rope (queries rotated on load).

The rotation on load uses the same fp32 arithmetic and single bf16 rounding
as rope_apply_append, so the fused call must equal rope_apply_append (writing
Q') followed by chunk_causal_attn on Q', bit for bit, output and LSE.  That
two-call path is itself checked against the oracle in test_gpu_rope.py and
test_gpu_attn.py; one small case here is also compared with the oracle run
on the oracle's own rotation, independently of the two-call path.
"""
import numpy as np
import pytest
import torch

import autoregressive_video_diffusion_amd as crattn
import oracle
from gpu_helpers import assert_attn_close, dev, f64, table
from workloads import SP480, STEP480, TINY, WIN720, call_qkv, prior_cache

pytestmark = pytest.mark.gpu


def _both(w, q, kc, vc, tab, ext, use_ws=True):
    """(fused out, fused lse), (two-call out, two-call lse) for query rows q."""
    B, Lq, H, D = q.shape
    mt, mh, mw = ext
    L = w.chunk_tokens
    wsb = crattn.chunk_causal_attn_workspace_bytes(B, H, Lq, w.kv_len, w.q_pos0, L, D)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=dev()) if use_ws and wsb else None
    out_f = torch.empty_like(q)
    lse_f = torch.empty(B, H, Lq, dtype=torch.float32, device=dev())
    crattn.chunk_causal_attn_rope(q, tab, mt, mh, mw, w.t0, w.grid_h, w.grid_w, kc, vc, w.kv_len,
                                  w.q_pos0, L, out_f, lse_f, ws)
    # two calls: rotate Q (the K/V append goes to a scratch copy of the cache,
    # so both paths read the same cache), then attention on Q'
    q_rot = torch.empty_like(q)
    kc2, vc2 = kc.clone(), vc.clone()
    crattn.rope_apply_append(q, q_rot, q, q, kc2, vc2, w.cache_pos, tab, mt, mh, mw, w.t0,
                             w.tok_off, w.grid_h, w.grid_w)
    out_t = torch.empty_like(q)
    lse_t = torch.empty_like(lse_f)
    crattn.chunk_causal_attn(q_rot, kc, vc, w.kv_len, w.q_pos0, L, out_t, lse_t, ws)
    torch.cuda.synchronize()
    return (out_f, lse_f), (out_t, lse_t), q_rot


@pytest.mark.parametrize("w", [STEP480, SP480], ids=lambda w: w.name)
def test_fused_rotation_equals_two_calls_bitwise(w):
    print(f"  {w.name}: Lq {w.lq} at q_pos0 {w.q_pos0}, kv_len {w.kv_len}", flush=True)
    ext = w.table_extents()
    tab = table(w.D, *ext)
    q, _, _ = call_qkv(w, 7)
    kc, vc = prior_cache(w)
    (of, lf), (ot, lt), _ = _both(w, q.to(dev()), kc.to(dev()), vc.to(dev()), tab, ext)
    assert torch.equal(of, ot)
    assert torch.equal(lf, lt)


def test_fused_rotation_ring_window_720p_bitwise():
    # 40 heads, 10800 queries of a 3x45x80 chunk at t0 81 in a full ring
    w = WIN720
    print(f"  {w.name}", flush=True)
    ext = w.table_extents()
    tab = table(w.D, *ext)
    q, _, _ = call_qkv(w, 3)
    kc, vc = prior_cache(w)
    (of, lf), (ot, lt), _ = _both(w, q.to(dev()), kc.to(dev()), vc.to(dev()), tab, ext)
    assert torch.equal(of, ot) and torch.equal(lf, lt)


def test_fused_rotation_tiny_d64_against_oracle():
    # head_dim 64 (table split 24/20/20) on bf16 copies of the tiny workload,
    # with and without the split-KV workspace; checked against the oracle's
    # own rotation followed by the oracle's attention
    w = TINY
    ext = w.table_extents()
    tab = table(w.D, *ext)
    q, _, _ = call_qkv(w, 5, dtype=torch.bfloat16)
    kc, vc = prior_cache(w, dtype=torch.bfloat16)
    qd, kcd, vcd = q.to(dev()), kc.to(dev()), vc.to(dev())
    for use_ws in (True, False):
        (of, lf), (ot, lt), q_rot = _both(w, qd, kcd, vcd, tab, ext, use_ws)
        assert torch.equal(of, ot) and torch.equal(lf, lt)
    q_e = oracle.round_bf16(oracle.rope(f64(q), w.t0, w.tok_off, w.grid_h, w.grid_w))
    o_e, lse_e = oracle.attn(q_e, f64(kc), f64(vc), w.kv_len, w.q_pos0, w.chunk_tokens)
    assert_attn_close(f64(of), o_e, "tiny fused rotation")
    np.testing.assert_allclose(f64(lf), lse_e, atol=2e-3)
