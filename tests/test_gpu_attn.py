"""GPU parity of chunk_causal_attn against the fp64 oracle.

Bar: max-abs <= 2e-2 and relative L2 <= 5e-3 for bf16 attention, on every
compared element (all rows at small sizes, sampled rows at the workload sizes
in the launch configuration the benchmark times).  Masks are checked bit for
bit: poisoning keys a row may not see leaves that row's output unchanged.
"""
import dataclasses

import numpy as np
import pytest
import torch

import autoregressive_video_diffusion_amd as crattn
import oracle
from autoregressive_video_diffusion_amd.rollout import ChunkRollout
from gpu_helpers import assert_attn_close, assert_rope_bf16, dev, f64, sample_rows, table
from workloads import ROLLOUT480, SP480, STEP480, TINY, WIN720, call_qkv, normal, prior_cache

pytestmark = pytest.mark.gpu


def run_attn(q, kc, vc, kv_len, q_pos0, L, want_lse=True, use_ws=True, scale=0.0):
    B, Lq, H, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(B, H, Lq, dtype=torch.float32, device=dev()) if want_lse else None
    wsb = crattn.chunk_causal_attn_workspace_bytes(B, H, Lq, kv_len, q_pos0, L, D)
    ws = None
    if use_ws and wsb > 0:
        ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=dev())
    crattn.chunk_causal_attn(q, kc, vc, kv_len, q_pos0, L, out, lse, ws, scale)
    torch.cuda.synchronize()
    return out, lse


def oracle_rows(q, kc, vc, kv_len, q_pos0, L, rows=None, scale=None, heads=None):
    """Oracle on the device tensors' exact values (optionally some heads only)."""
    if heads is not None:
        q = q[:, :, heads]
        kc, vc = kc[:, heads], vc[:, heads]
    return oracle.attn(f64(q), f64(kc), f64(vc), kv_len, q_pos0, L, scale=scale, rows=rows)


def rand_bf16(shape, seed, scale=1.0):
    return (normal(shape, seed, torch.float32) * scale).to(torch.bfloat16).to(dev())


# --------------------------------------------------------------------------- tiny


def test_tiny_workload_end_to_end():
    w = TINY
    mt, mh, mw = w.table_extents()
    tab = table(w.D, mt, mh, mw)
    q, k, v = call_qkv(w, 0)
    kc, vc = prior_cache(w)
    qd, kcd, vcd = q.to(dev()), kc.to(dev()), vc.to(dev())
    q_out = torch.empty_like(qd)
    crattn.rope_apply_append(qd, q_out, k.to(dev()), v.to(dev()), kcd, vcd, w.cache_pos, tab,
                             mt, mh, mw, w.t0, w.tok_off, w.grid_h, w.grid_w)
    # attention runs on bf16 copies of the fp32 rotated tensors
    q16, k16, v16 = q_out.bfloat16(), kcd.bfloat16(), vcd.bfloat16()
    out, lse = run_attn(q16, k16, v16, w.kv_len, w.q_pos0, w.chunk_tokens)
    o_ref, lse_ref = oracle_rows(q16, k16, v16, w.kv_len, w.q_pos0, w.chunk_tokens)
    assert_attn_close(f64(out), o_ref, "tiny unit")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)
    # end to end: the oracle's own RoPE, rounded to bf16 where the path stores bf16
    q_e = oracle.round_bf16(oracle.rope(f64(q), w.t0, 0, w.grid_h, w.grid_w))
    k_e = f64(kc)
    k_e[:, :, w.cache_pos:] = oracle.rope(f64(k), w.t0, 0, w.grid_h, w.grid_w).transpose(0, 2, 1, 3)
    v_e = f64(vc)
    v_e[:, :, w.cache_pos:] = f64(v).transpose(0, 2, 1, 3)
    o_e, _ = oracle.attn(q_e, oracle.round_bf16(k_e), oracle.round_bf16(v_e), w.kv_len, w.q_pos0,
                         w.chunk_tokens)
    assert_attn_close(f64(out), o_e, "tiny end-to-end")


@pytest.mark.parametrize("B,D", [(1, 64), (2, 64), (2, 128)])
def test_full_sequence_form_all_chunks(B, D):
    # queries of all 4 chunks in one call: 4 chunk segments, each its own mask
    H, L, n = 2, 64, 256
    q = rand_bf16((B, n, H, D), 11)
    kc = rand_bf16((B, H, n, D), 12)
    vc = rand_bf16((B, H, n, D), 13)
    out, lse = run_attn(q, kc, vc, n, 0, L)
    o_ref, lse_ref = oracle_rows(q, kc, vc, n, 0, L)
    assert_attn_close(f64(out), o_ref, f"full-seq B{B} D{D}")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)
    # the cache form of chunk c equals the chunk-c rows of the full form
    for c in range(4):
        part, _ = run_attn(q[:, c * L:(c + 1) * L].contiguous(), kc, vc, (c + 1) * L, c * L, L)
        assert torch.equal(part, out[:, c * L:(c + 1) * L])


@pytest.mark.parametrize("poison", [float("nan"), float("inf"), -float("inf"), 1e30])
def test_future_chunks_and_capacity_cannot_leak(poison):
    B, H, D, L, n, cap = 1, 2, 128, 100, 400, 520
    q = rand_bf16((B, n, H, D), 21)
    kc = torch.zeros(B, H, cap, D, dtype=torch.bfloat16, device=dev())
    vc = torch.zeros_like(kc)
    kc[:, :, :n] = rand_bf16((B, H, n, D), 22)
    vc[:, :, :n] = rand_bf16((B, H, n, D), 23)
    base, base_lse = run_attn(q, kc, vc, n, 0, L)
    kp, vp = kc.clone(), vc.clone()
    kp[:, :, 200:] = poison
    vp[:, :, 200:] = poison
    got, got_lse = run_attn(q, kp, vp, n, 0, L)
    assert torch.equal(got[:, :200], base[:, :200])
    assert torch.equal(got_lse[:, :, :200], base_lse[:, :, :200])
    # capacity beyond kv_len is never read by anyone
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[:, :, n:] = poison
    vc2[:, :, n:] = poison
    got2, _ = run_attn(q, kc2, vc2, n, 0, L)
    assert torch.equal(got2, base)


# --------------------------------------------------------------------------- ragged / stress


@pytest.mark.parametrize("D", [64, 128])
def test_ragged_segments_and_tails(D):
    # rows 0..49 in chunk 1, 50..149 in chunk 2, 150..249 in chunk 3
    B, H, L, Lq, q_pos0, kv_len, cap = 2, 3, 100, 250, 150, 400, 448
    q = rand_bf16((B, Lq, H, D), 31)
    kc = rand_bf16((B, H, cap, D), 32)
    vc = rand_bf16((B, H, cap, D), 33)
    out, lse = run_attn(q, kc, vc, kv_len, q_pos0, L)
    o_ref, lse_ref = oracle_rows(q, kc, vc, kv_len, q_pos0, L)
    assert_attn_close(f64(out), o_ref, f"ragged D{D}")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)


@pytest.mark.parametrize("D", [64, 128])
def test_split_key_range_all_rows(D):
    # Two chunk segments (2000 and 500 rows), 40 query tiles of 188 or 250 key
    # tiles whose key ranges are split between workgroups: every row is
    # compared with the oracle.  The workspace starts as garbage (NaN bytes)
    # and is then reused as is by a second call of another shape.
    B, H, L, Lq, q_pos0, kv_len, cap = 2, 2, 4000, 2500, 10000, 16000, 16384
    q = rand_bf16((B, Lq, H, D), 51)
    kc = rand_bf16((B, H, cap, D), 52)
    vc = rand_bf16((B, H, cap, D), 53)
    wsb = crattn.chunk_causal_attn_workspace_bytes(B, H, Lq, kv_len, q_pos0, L, D)
    assert wsb > 0
    ws = torch.full((wsb // 4 + 4,), float("nan"), dtype=torch.float32, device=dev())
    out = torch.empty_like(q)
    lse = torch.empty(B, H, Lq, dtype=torch.float32, device=dev())
    crattn.chunk_causal_attn(q, kc, vc, kv_len, q_pos0, L, out, lse, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_rows(q, kc, vc, kv_len, q_pos0, L)
    assert_attn_close(f64(out), o_ref, f"split D{D}")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)
    plain, plain_lse = run_attn(q, kc, vc, kv_len, q_pos0, L, use_ws=False)
    assert (out.float() - plain.float()).abs().max().item() <= 2e-3
    assert (lse - plain_lse).abs().max().item() <= 1e-3
    # second call: 2 x 8 heads x 2 tiles of 250 key tiles, same workspace
    B2, H2, Lq2, q_pos2 = 2, 8, 300, 15700
    assert 0 < crattn.chunk_causal_attn_workspace_bytes(B2, H2, Lq2, kv_len, q_pos2, L, D) <= wsb
    q2 = rand_bf16((B2, Lq2, H2, D), 54)
    kc2 = kc[:, :1].expand(B2, H2, cap, D).contiguous()
    vc2 = vc[:, 1:].expand(B2, H2, cap, D).contiguous()
    out2 = torch.empty_like(q2)
    crattn.chunk_causal_attn(q2, kc2, vc2, kv_len, q_pos2, L, out2, None, ws)
    torch.cuda.synchronize()
    o_ref2, _ = oracle_rows(q2, kc2, vc2, kv_len, q_pos2, L)
    assert_attn_close(f64(out2), o_ref2, f"split reuse D{D}")


@pytest.mark.parametrize("kind", ["peaked_q_x8", "key_ramp_1_to_4", "identical_keys",
                                  "tiny_scale"])
def test_stress_distributions(kind):
    B, H, D, L, Lq, kv_len = 1, 2, 128, 300, 300, 1200
    q = rand_bf16((B, Lq, H, D), 41)
    kc = rand_bf16((B, H, kv_len, D), 42)
    vc = rand_bf16((B, H, kv_len, D), 43)
    scale = 0.0
    if kind == "peaked_q_x8":
        q = (q.float() * 8).bfloat16()
    elif kind == "key_ramp_1_to_4":
        ramp = torch.linspace(1, 4, kv_len, device=dev())[None, None, :, None]
        kc = (kc.float() * ramp).bfloat16()
    elif kind == "identical_keys":
        kc = kc[:, :, :1].expand(B, H, kv_len, D).contiguous()
    elif kind == "tiny_scale":
        scale = 1e-3
    out, _ = run_attn(q, kc, vc, kv_len, 900, L, scale=scale)
    o_ref, _ = oracle_rows(q, kc, vc, kv_len, 900, L, scale=scale or None)
    assert_attn_close(f64(out), o_ref, kind)


def test_uniform_split_one_head_all_rows():
    # one head of the SP slice: 3 query tiles, each key range split 16 ways
    # and merged by the combine kernel; every row against the oracle, and
    # five reruns agree bit for bit
    w = SP480
    q = rand_bf16((1, w.lq, 1, w.D), 61)
    kc = rand_bf16((1, 1, w.cap, w.D), 62)
    vc = rand_bf16((1, 1, w.cap, w.D), 63)
    assert crattn.chunk_causal_attn_workspace_bytes(1, 1, w.lq, w.kv_len, w.q_pos0,
                                                    w.chunk_tokens, w.D) == 16 * w.lq * 129 * 4
    out, lse = run_attn(q, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens)
    o_ref, lse_ref = oracle_rows(q, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens)
    assert_attn_close(f64(out), o_ref, "16 splits")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)
    for _ in range(5):
        o2, l2 = run_attn(q, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens)
        assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_balanced_split_three_parts_all_rows():
    # 130 query tiles (a little over half the compute units) of 1024 key
    # tiles: the balanced split cuts each tile into 2 or 3 parts merged by
    # the last to finish; every row of 2 heads against the oracle, reruns
    # bit for bit
    B, H, D, L, Lq, kv_len, q_pos0 = 1, 65, 128, 512, 512, 65536, 65024
    assert crattn.chunk_causal_attn_workspace_bytes(B, H, Lq, kv_len, q_pos0, L, D) == \
        1024 + 2 * 256 * 256 * 129 * 4
    q = rand_bf16((B, Lq, H, D), 64)
    kc = rand_bf16((B, H, kv_len, D), 65)
    vc = rand_bf16((B, H, kv_len, D), 66)
    out, lse = run_attn(q, kc, vc, kv_len, q_pos0, L)
    heads = [0, 64]
    o_ref, lse_ref = oracle_rows(q, kc, vc, kv_len, q_pos0, L, heads=heads)
    assert_attn_close(f64(out[:, :, heads]), o_ref, "balanced split")
    np.testing.assert_allclose(f64(lse[:, heads]), lse_ref, atol=2e-3)
    for _ in range(3):
        o2, l2 = run_attn(q, kc, vc, kv_len, q_pos0, L)
        assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("kind", ["single_jump", "rising_steps", "jump_in_last_tile"])
def test_score_jumps_take_the_rescale_path(kind):
    # The key loop keeps the first tile's row maximum until a lane's row sum
    # passes 2^31; these keys make later scores jump by far more than 31
    # (base 2), so exact results need the rescale block (without it p would
    # overflow to inf).  All rows against the oracle, split and unsplit.
    # chunk 1 of 4083-key chunks: 8166 keys, the final tile holds 38
    B, H, D, L, Lq, kv_len, q_pos0 = 1, 2, 128, 4083, 300, 8166, 4083
    q = rand_bf16((B, Lq, H, D), 71)
    kc = normal((B, H, kv_len, D), 72, torch.float32)
    vc = rand_bf16((B, H, kv_len, D), 73)
    if kind == "single_jump":
        kc[:, :, 3000:3064] *= 40.0
    elif kind == "rising_steps":
        for i, t in enumerate(range(1000, 8000, 1500)):
            kc[:, :, t:t + 64] *= 10.0 * (i + 1)
    else:  # inside the partial final tile (keys 8128..8165)
        kc[:, :, 8140:8150] *= 60.0
    kc = kc.to(torch.bfloat16).to(dev())
    o_ref, lse_ref = oracle_rows(q, kc, vc, kv_len, q_pos0, L)
    for use_ws in (True, False):
        out, lse = run_attn(q, kc, vc, kv_len, q_pos0, L, use_ws=use_ws)
        assert_attn_close(f64(out), o_ref, f"{kind} ws={use_ws}")
        np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3, rtol=1e-6)


def test_deterministic_rerun():
    w = SP480
    q = rand_bf16((1, w.lq, w.H, w.D), 51)
    kc = rand_bf16((1, w.H, w.cap, w.D), 52)
    vc = rand_bf16((1, w.H, w.cap, w.D), 53)
    a, la = run_attn(q, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens)
    b, lb = run_attn(q, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens)
    assert torch.equal(a, b) and torch.equal(la, lb)


# --------------------------------------------------------------------------- workloads


def _step(w, call=0):
    """RoPE/append of one denoising call into a prefilled cache, then attention."""
    mt, mh, mw = w.table_extents()
    tab = table(w.D, mt, mh, mw)
    q, k, v = call_qkv(w, call)
    kc, vc = prior_cache(w)
    kcd, vcd = kc.to(dev()), vc.to(dev())
    qd = q.to(dev())
    q_out = torch.empty_like(qd)
    crattn.rope_apply_append(qd, q_out, k.to(dev()), v.to(dev()), kcd, vcd, w.cache_pos, tab,
                             mt, mh, mw, w.t0, w.tok_off, w.grid_h, w.grid_w)
    return (q, k, v, kc, vc), (q_out, kcd, vcd)


def test_step480_every_row():
    # the headline call (4680 queries x 32760 keys, 12 heads) in the launch
    # configuration the benchmark times: every row of every head against the
    # oracle fed the GPU's own rotated queries and cache (~10 s of host time)
    w = STEP480
    (q, k, v, kc, vc), (q_out, kcd, vcd) = _step(w)
    out, lse = run_attn(q_out, kcd, vcd, w.kv_len, w.q_pos0, w.chunk_tokens)
    o_ref, lse_ref = oracle_rows(q_out, kcd, vcd, w.kv_len, w.q_pos0, w.chunk_tokens)
    assert_attn_close(f64(out), o_ref, "480P unit (every row)")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)
    del o_ref, lse_ref
    rows = sample_rows(w.lq)
    # end to end for sampled rows: the oracle's own rotation of this chunk
    q_full = oracle.round_bf16(oracle.rope(f64(q), w.t0, 0, w.grid_h, w.grid_w))
    k_e = f64(kc)
    k_e[:, :, w.cache_pos:] = oracle.round_bf16(
        oracle.rope(f64(k), w.t0, 0, w.grid_h, w.grid_w)).transpose(0, 2, 1, 3)
    v_e = f64(vc)
    v_e[:, :, w.cache_pos:] = f64(v).transpose(0, 2, 1, 3)
    o_e, _ = oracle.attn(q_full, k_e, v_e, w.kv_len, w.q_pos0, w.chunk_tokens, rows=rows)
    assert_attn_close(f64(out[:, rows]), o_e, "480P end-to-end (sampled rows)")
    # properties at full size: finite, and each output row is a convex
    # combination of value rows, so it lies within their range
    assert torch.isfinite(out).all()
    vmax = vcd[:, :, :w.kv_len].float().amax(dim=2)       # [B, H, D]
    vmin = vcd[:, :, :w.kv_len].float().amin(dim=2)
    o32 = out.float().permute(0, 2, 1, 3)                 # [B, H, Lq, D]
    assert bool((o32 <= vmax[:, :, None] + 1e-2).all() and (o32 >= vmin[:, :, None] - 1e-2).all())


def test_step_replays_from_a_hip_graph():
    # one denoising call of the SP-rank slice (RoPE/append into the cache,
    # then the split-KV attention and its combine) captured once and
    # replayed: every replay writes the eager call's output, lse and cache
    # rows bit for bit, with eager calls between the replays and the
    # workspace poisoned before each (the path records no memset nodes)
    w = SP480
    mt, mh, mw = w.table_extents()
    tab = table(w.D, mt, mh, mw)
    q, k, v = (t.to(dev()) for t in call_qkv(w, 0))
    kc, vc = (t.to(dev()) for t in prior_cache(w))
    q_out = torch.empty_like(q)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.lq, dtype=torch.float32, device=dev())
    wsb = crattn.chunk_causal_attn_workspace_bytes(w.B, w.H, w.lq, w.kv_len, w.q_pos0,
                                                   w.chunk_tokens, w.D)
    assert wsb > 0  # the split-KV combine is part of the captured call
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=dev())

    def call():
        crattn.rope_apply_append(q, q_out, k, v, kc, vc, w.cache_pos, tab, mt, mh, mw, w.t0,
                                 w.tok_off, w.grid_h, w.grid_w)
        crattn.chunk_causal_attn(q_out, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens, out, lse, ws)

    call()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), kc.clone(), vc.clone())
    rows = sample_rows(w.lq)
    o_ref, _ = oracle_rows(q_out, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens, rows=rows)
    assert_attn_close(f64(out[:, rows]), o_ref, "SP slice before capture (sampled rows)")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for t in (out, lse, q_out):
            t.zero_()
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "lse", "k cache", "v cache"), (out, lse, kc, vc), ref):
            assert torch.equal(got, want), f"replay {rep}: {name}"
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])


def test_sp480_split_kv_and_unsplit():
    # one sequence-parallel rank's slice: every row of every head, split-KV
    # (as timed) and unsplit
    w = SP480
    (q, k, v, kc, vc), (q_out, kcd, vcd) = _step(w)
    assert crattn.chunk_causal_attn_workspace_bytes(w.B, w.H, w.lq, w.kv_len, w.q_pos0,
                                                    w.chunk_tokens, w.D) > 0
    out, lse = run_attn(q_out, kcd, vcd, w.kv_len, w.q_pos0, w.chunk_tokens)
    out1, lse1 = run_attn(q_out, kcd, vcd, w.kv_len, w.q_pos0, w.chunk_tokens, use_ws=False)
    o_ref, lse_ref = oracle_rows(q_out, kcd, vcd, w.kv_len, w.q_pos0, w.chunk_tokens)
    assert_attn_close(f64(out), o_ref, "sp rank split-KV (every row)")
    assert_attn_close(f64(out1), o_ref, "sp rank unsplit (every row)")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)
    np.testing.assert_allclose(f64(lse1), lse_ref, atol=2e-3)


def test_sp_slice_equals_rows_of_whole_chunk():
    # One rank's slice, rotated and appended from its global offsets, attends
    # exactly like the same rows of the whole-chunk call.
    full, w = STEP480, SP480
    (q, k, v, _, _), (q_out, kcd, vcd) = _step(full)
    # one workgroup per query tile (no workspace): rows are computed
    # independently, in the same order, whatever the call's extent
    outf, lsef = run_attn(q_out, kcd, vcd, full.kv_len, full.q_pos0, full.chunk_tokens,
                          use_ws=False)
    sl = slice(w.tok_off, w.tok_off + w.lq)
    mt, mh, mw = w.table_extents()
    tab = table(w.D, mt, mh, mw)
    kc2, vc2 = kcd.clone(), vcd.clone()
    q2 = torch.empty(1, w.lq, w.H, w.D, dtype=torch.bfloat16, device=dev())
    crattn.rope_apply_append(q[:, sl].contiguous().to(dev()), q2, k[:, sl].contiguous().to(dev()),
                             v[:, sl].contiguous().to(dev()), kc2, vc2, w.cache_pos, tab, mt, mh,
                             mw, w.t0, w.tok_off, w.grid_h, w.grid_w)
    assert torch.equal(q2, q_out[:, sl]) and torch.equal(kc2, kcd) and torch.equal(vc2, vcd)
    out1, lse1 = run_attn(q2, kc2, vc2, w.kv_len, w.q_pos0, w.chunk_tokens, use_ws=False)
    assert torch.equal(out1, outf[:, sl]) and torch.equal(lse1, lsef[:, :, sl])
    out, _ = run_attn(q2, kc2, vc2, w.kv_len, w.q_pos0, w.chunk_tokens)
    d = (out.float() - outf[:, sl].float()).abs().max().item()
    print(f"  split-KV slice vs whole-chunk rows: max-abs {d:.2e}", flush=True)
    assert d <= 2e-3
    # the whole chunk with the workspace (split if the planner splits it)
    outs, lses = run_attn(q_out, kcd, vcd, full.kv_len, full.q_pos0, full.chunk_tokens)
    d = (outs.float() - outf.float()).abs().max().item()
    dl = (lses - lsef).abs().max().item()
    print(f"  whole chunk with workspace vs without: max-abs {d:.2e}, lse {dl:.2e}",
          flush=True)
    assert d <= 2e-3 and dl <= 1e-3


def test_win720_ring_window_sampled():
    w = WIN720
    mt, mh, mw = w.table_extents()
    tab = table(w.D, mt, mh, mw)
    q, k, v = call_qkv(w, 0)
    kc, vc = prior_cache(w)
    kcd, vcd = kc.to(dev()), vc.to(dev())
    del kc, vc
    qd = q.to(dev())
    q_out = torch.empty_like(qd)
    crattn.rope_apply_append(qd, q_out, k.to(dev()), v.to(dev()), kcd, vcd, w.cache_pos, tab,
                             mt, mh, mw, w.t0, 0, w.grid_h, w.grid_w)
    out, lse = run_attn(q_out, kcd, vcd, w.kv_len, w.q_pos0, w.chunk_tokens)
    assert torch.isfinite(out).all()
    rows = sample_rows(w.lq, n_random=12)
    for h in (0, 17, 39):
        o_ref, lse_ref = oracle_rows(q_out, kcd, vcd, w.kv_len, w.q_pos0, w.chunk_tokens,
                                     rows=rows, heads=[h])
        assert_attn_close(f64(out[:, rows][:, :, [h]]), o_ref, f"720P window head {h}")
        np.testing.assert_allclose(f64(lse[:, [h]][:, :, rows]), lse_ref, atol=2e-3)
    # ring order does not matter: rotating the slots leaves the output unchanged
    # (within fp32 summation-order differences)
    sh = 3 * w.chunk_tokens
    kr = torch.roll(kcd, sh, dims=2)
    vr = torch.roll(vcd, sh, dims=2)
    outr, _ = run_attn(q_out, kr, vr, w.kv_len, w.q_pos0, w.chunk_tokens)
    d = (outr.float() - out.float()).abs().max().item()
    print(f"  ring rotation changes output by {d:.2e}", flush=True)
    assert d <= 1e-2


def test_rollout480_seven_chunks():
    w = ROLLOUT480
    ro = ChunkRollout(w.B, w.H, w.D, w.frames, w.grid_h, w.grid_w, window=7, max_chunks=7)
    n = w.chunk_tokens
    q_out = torch.empty(w.B, n, w.H, w.D, dtype=torch.bfloat16, device=dev())
    out = torch.empty_like(q_out)
    clean = []
    for c in range(7):
        for j in range(4):
            q, k, v = call_qkv(w, c * 5 + j)
            ro.denoise(c, q.to(dev()), k.to(dev()), v.to(dev()), q_out, out)
            if j == 3:
                # every chunk's last denoising call: all 12 heads, sampled rows
                kv_len, q0 = ro.visible(c)
                assert kv_len == (c + 1) * n and q0 == c * n
                rows = sample_rows(n, n_random=8, seed=c)
                o_ref, _ = oracle_rows(q_out, ro.k_cache, ro.v_cache, kv_len, q0, n, rows=rows)
                assert_attn_close(f64(out[:, rows]), o_ref, f"rollout chunk {c} step {j}")
        _, k, v = call_qkv(w, c * 5 + 4)
        ro.update(c, k.to(dev()), v.to(dev()))
        clean.append((k, v))
    torch.cuda.synchronize()
    # final cache: every slot holds its chunk's clean K (rotated at t0 = 3c) and V
    for c, (k, v) in enumerate(clean):
        rows = slice(c * n, (c + 1) * n)
        k_ref = oracle.rope(f64(k), 3 * c, 0, w.grid_h, w.grid_w).transpose(0, 2, 1, 3)
        assert_rope_bf16(f64(ro.k_cache[:, :, rows]), k_ref, f64(k).transpose(0, 2, 1, 3))
        assert torch.equal(ro.v_cache[:, :, rows].cpu(), v.permute(0, 2, 1, 3))
