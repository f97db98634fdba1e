"""GPU parity of the hierarchical block-sparse attention (HSA) path against
the fp64 oracle (oracle/hsa.py).

* Pooling: every frame and block mean within the fp32 summation bound
  (n + 1) * 2^-24 * mean|x| of its n rows.
* Selection: a float decides an integer here, so the GPU's choice (fp32) is
  checked for validity against the exact fp64 scores: its blocks come from
  at most kf frames that are a top-kf set within the fp32 score bound, the
  blocks are a top-kb set of those frames' blocks within the bound, the ids
  ascend, and -1 pads the rest.  Where the exact scores separate the sets by
  more than the bound, the choice must equal the oracle's.
* Attention: given the GPU's selection (unique output), every compared row
  within the bf16 attention bar (max-abs 2e-2, relative L2 5e-3) of the
  oracle's attention over the own chunk plus those blocks.
* Keys outside the selection are never read: NaN there leaves the output
  bit-identical; invalid ids in the list are skipped.
* Ring window: with the own chunk anywhere in a full ring, every other slot
  is history; a rollout through the wrapped ring is checked chunk by chunk.
"""
import numpy as np
import pytest
import torch

import autoregressive_video_diffusion_amd as crattn
import oracle
from gpu_helpers import assert_attn_close, dev, f64
from oracle import hsa
from workloads import STEP480, call_qkv, normal

pytestmark = pytest.mark.gpu
EPS = 2.0 ** -24


def _inputs(B, H, D, per_frame, F_c, chunks, Lq, q_off, seed, own=None):
    """Queries of one call and a cache of `chunks` whole chunks; the own
    chunk is the last one, or slot `own` of a full ring."""
    L = F_c * per_frame
    cap = chunks * L
    q = normal((B, Lq, H, D), seed).to(dev())
    kc = normal((B, H, cap, D), seed + 1).to(dev())
    vc = normal((B, H, cap, D), seed + 2).to(dev())
    return q, kc, vc, L, cap, (chunks - 1 if own is None else own) * L + q_off


def _pool(kc, per_frame):
    B, H, cap, D = kc.shape
    nbytes = crattn.hsa_pool_bytes(B, H, cap, D, per_frame)
    pool = torch.empty(nbytes // 4, dtype=torch.float32, device=dev())
    crattn.hsa_pool_keys(kc, 0, cap, per_frame, pool)
    torch.cuda.synchronize()
    nf, nbf = cap // per_frame, hsa.blocks_per_frame(per_frame)
    fr = pool[:B * H * nf * D].view(B, H, nf, D)
    bl = pool[B * H * nf * D:B * H * (nf + nf * nbf) * D].view(B, H, nf * nbf, D)
    return pool, f64(fr), f64(bl)


def _select(q, pool, cap, per_frame, q_pos0, L, kf, kb, kv_len=None):
    B, Lq, H, D = q.shape
    sel = torch.empty(B, H, -(-Lq // 256), kb, dtype=torch.int32, device=dev())
    crattn.hsa_select(q, pool, cap, kv_len or cap, per_frame, q_pos0, L, kf, kb, sel)
    torch.cuda.synchronize()
    return sel


def _hsa_attn(q, kc, vc, q_pos0, L, per_frame, sel, kv_len=None):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=dev())
    crattn.hsa_attn(q, kc, vc, kv_len or kc.shape[2], q_pos0, L, per_frame, sel, out, lse)
    torch.cuda.synchronize()
    return out, lse


def _check_pool(kc, per_frame, fr, bl):
    k = f64(kc)
    ef, eb = hsa.pool_keys(k, per_frame)
    af, ab = hsa.pool_keys(np.abs(k), per_frame)
    nbf = hsa.blocks_per_frame(per_frame)
    n_b = np.array([np.subtract(*hsa.block_range(j, per_frame)[::-1]) for j in range(nbf)])
    n_b = np.tile(n_b, eb.shape[2] // nbf)[None, None, :, None]
    assert np.all(np.abs(bl - eb) <= (n_b + 1) * EPS * ab + 1e-30)
    assert np.all(np.abs(fr - ef) <= (per_frame + 1) * EPS * af + 1e-30)


def _depths(D, per_frame):
    """Rounding steps on any path of the GPU's summation trees (hsa.hip):
    RG = 256 / (D/8) row groups; a thread adds its rows of the block (or
    query block) in order, the RG partials are added in order, then one
    division; a frame adds its block means times their lengths in block
    order, then divides.  The dot product: D/16 products per lane in steps
    of four, then a 4-level butterfly."""
    RG = 256 // (D // 8)
    q_mean = -(-256 // RG) + RG + 1
    b_mean = -(-64 // RG) + RG + 1
    f_mean = b_mean + 1 + hsa.blocks_per_frame(per_frame) + 1
    dot = D // 16 + 8
    return q_mean, b_mean, f_mean, dot


def _score_bound(qbar_abs, k_abs, qbar, kbar, cq, ck, cdot):
    """First-order bound of the fp32 pooled dot product's error: the query
    mean's and the key mean's summation errors (cq, ck rounding steps times
    the mean of |x|) and the dot product's own (cdot steps)."""
    return cq * EPS * (qbar_abs * np.abs(kbar)).sum(-1) + \
        ck * EPS * (np.abs(qbar) * k_abs).sum(-1) + \
        cdot * EPS * (np.abs(qbar) * np.abs(kbar)).sum(-1)


def _check_selection(q, kc, per_frame, L, q_pos0, kf, kb, sel, kv_len=None):
    """Validity of the GPU selection against exact scores; returns the number
    of query blocks whose choice had to match the oracle exactly.

    The frames are seen through their chosen blocks.  A kept frame may win no
    block, so instead of the frame set the check asks that the chosen blocks
    be a top-kb set (within the bound) of every block of the frames it could
    not have dropped: the seen frames plus every frame whose exact score beats
    the (kf+1)-th best by more than twice the bound.  Dropping such a frame
    is then caught whenever it changes the chosen blocks."""
    qe, ke = f64(q), f64(kc)
    B, Lq, H, D = qe.shape
    kv_len = kv_len or ke.shape[2]
    nbf = hsa.blocks_per_frame(per_frame)
    hist = hsa.history_frames(kv_len, q_pos0, L, per_frame)
    n_hist = len(hist)
    ef, eb = hsa.pool_keys(ke, per_frame)
    af, ab = hsa.pool_keys(np.abs(ke), per_frame)
    qp, qa = hsa.pool_queries(qe), hsa.pool_queries(np.abs(qe))
    ref = hsa.select(qe, ef, eb, hist, per_frame, kf, kb)
    cq, cb, cf, cdot = _depths(D, per_frame)
    s = sel.cpu().numpy()
    exact = 0
    for b in range(B):
        for h in range(H):
            for i in range(qp.shape[2]):
                got = s[b, h, i]
                n_valid = int((got >= 0).sum())
                assert (got[:n_valid] >= 0).all() and (got[n_valid:] == -1).all()
                assert np.all(np.diff(got[:n_valid]) > 0)
                n_cand = min(kf, n_hist) * nbf
                assert n_valid == min(kb, n_cand)
                if n_hist == 0:
                    continue
                frames = np.unique(got[:n_valid] // nbf)
                assert np.isin(frames, hist).all(), "a block outside the history"
                assert len(frames) <= kf
                fs = ef[b, h, hist] @ qp[b, h, i]                  # per history position
                ftol = _score_bound(qa[b, h, i], af[b, h, hist], qp[b, h, i],
                                    ef[b, h, hist], cq, cf, cdot)
                pos = np.searchsorted(hist, frames)
                srt = np.sort(fs)[::-1]
                kth = srt[min(kf, n_hist) - 1]
                # every seen frame is a top-kf frame up to the bound
                assert np.all(fs[pos] >= kth - ftol[pos] - ftol.max())
                # frames that must have been kept
                nxt = srt[kf] if n_hist > kf else -np.inf
                certain = hist[fs > nxt + 2 * ftol.max()]
                cand_frames = np.union1d(frames, certain)
                # a valid kept set holds every certain frame and every seen one
                assert len(cand_frames) <= kf, (b, h, i, "a certain frame was dropped")
                cand = np.concatenate([np.arange(f * nbf, (f + 1) * nbf) for f in cand_frames])
                bs = eb[b, h, got[:n_valid]] @ qp[b, h, i]
                btol = _score_bound(qa[b, h, i], ab[b, h, cand], qp[b, h, i], eb[b, h, cand],
                                    cq, cb, cdot).max()
                unchosen = np.setdiff1d(cand, got[:n_valid])
                if len(unchosen) and n_valid:
                    best_out = (eb[b, h, unchosen] @ qp[b, h, i]).max()
                    assert bs.min() >= best_out - 2 * btol, (b, h, i, "a better block was left")
                # unique where the exact scores are well separated
                f_sep = n_hist <= kf or srt[kf - 1] - srt[kf] > 4 * ftol.max()
                all_b = np.concatenate([np.arange(f * nbf, (f + 1) * nbf)
                                        for f in hist[hsa.topk(fs, kf)]])
                bsr = np.sort(eb[b, h, all_b] @ qp[b, h, i])[::-1]
                b_sep = len(bsr) <= kb or bsr[kb - 1] - bsr[kb] > 4 * btol
                if f_sep and b_sep:
                    assert np.array_equal(got, ref[b, h, i]), (b, h, i)
                    exact += 1
    return exact


def _separated(q, kc, per_frame, L, q_pos0, kf, kb, kv_len=None):
    """Query blocks whose choice is unique under the bound (from the exact
    scores alone, whatever the GPU did)."""
    qe, ke = f64(q), f64(kc)
    B, Lq, H, D = qe.shape
    nbf = hsa.blocks_per_frame(per_frame)
    hist = hsa.history_frames(kv_len or ke.shape[2], q_pos0, L, per_frame)
    ef, eb = hsa.pool_keys(ke, per_frame)
    af, ab = hsa.pool_keys(np.abs(ke), per_frame)
    qp, qa = hsa.pool_queries(qe), hsa.pool_queries(np.abs(qe))
    cq, cb, cf, cdot = _depths(D, per_frame)
    n = 0
    for b in range(B):
        for h in range(H):
            for i in range(qp.shape[2]):
                fs = ef[b, h, hist] @ qp[b, h, i]
                ftol = _score_bound(qa[b, h, i], af[b, h, hist], qp[b, h, i], ef[b, h, hist],
                                    cq, cf, cdot)
                srt = np.sort(fs)[::-1]
                f_sep = len(hist) <= kf or srt[kf - 1] - srt[kf] > 4 * ftol.max()
                all_b = np.concatenate([np.arange(f * nbf, (f + 1) * nbf)
                                        for f in hist[hsa.topk(fs, kf)]])
                btol = _score_bound(qa[b, h, i], ab[b, h, all_b], qp[b, h, i], eb[b, h, all_b],
                                    cq, cb, cdot).max()
                bsr = np.sort(eb[b, h, all_b] @ qp[b, h, i])[::-1]
                b_sep = len(bsr) <= kb or bsr[kb - 1] - bsr[kb] > 4 * btol
                n += int(f_sep and b_sep)
    return n


@pytest.mark.parametrize("B,H,D,gh,gw,F_c,chunks,Lq,q_off,kf,kb", [
    (1, 2, 64, 8, 8, 1, 4, 64, 0, 2, 3),          # tiny geometry: one block per frame
    (2, 2, 128, 10, 10, 2, 4, 200, 0, 3, 5),      # 100-token frames: blocks of 64 + 36
    (1, 3, 128, 12, 20, 1, 6, 240, 0, 4, 12),     # 240-token frames, 4 blocks each
    (1, 2, 64, 9, 9, 2, 3, 100, 62, 2, 64),       # a slice; kb above the candidates: -1 pads
])
def test_small_configs_every_row(B, H, D, gh, gw, F_c, chunks, Lq, q_off, kf, kb):
    per_frame = gh * gw
    q, kc, vc, L, cap, q_pos0 = _inputs(B, H, D, per_frame, F_c, chunks, Lq, q_off, 31 + D)
    pool, fr, bl = _pool(kc, per_frame)
    _check_pool(kc, per_frame, fr, bl)
    sel = _select(q, pool, cap, per_frame, q_pos0, L, kf, kb)
    _check_selection(q, kc, per_frame, L, q_pos0, kf, kb, sel)
    out, lse = _hsa_attn(q, kc, vc, q_pos0, L, per_frame, sel)
    s64 = sel.cpu().numpy().astype(np.int64)
    own0 = (q_pos0 // L) * L
    o_ref, lse_ref = hsa.attn(f64(q), f64(kc), f64(vc), s64, own0, own0 + L, per_frame)
    assert_attn_close(f64(out), o_ref, "hsa small")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)


def test_selecting_everything_matches_dense_attention():
    B, H, D, per_frame, F_c, chunks, Lq = 1, 2, 128, 100, 2, 5, 200
    q, kc, vc, L, cap, q_pos0 = _inputs(B, H, D, per_frame, F_c, chunks, Lq, 0, 77)
    pool, _, _ = _pool(kc, per_frame)
    n_hist = (chunks - 1) * F_c
    kb = n_hist * hsa.blocks_per_frame(per_frame)
    sel = _select(q, pool, cap, per_frame, q_pos0, L, n_hist, kb)
    assert (sel >= 0).all()
    out, lse = _hsa_attn(q, kc, vc, q_pos0, L, per_frame, sel)
    dense = torch.empty_like(q)
    dlse = torch.empty_like(lse)
    crattn.chunk_causal_attn(q, kc, vc, cap, q_pos0, L, dense, dlse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn(f64(q), f64(kc), f64(vc), cap, q_pos0, L)
    assert_attn_close(f64(out), o_ref, "hsa, everything selected")
    assert_attn_close(f64(dense), o_ref, "dense")
    np.testing.assert_allclose(f64(lse), f64(dlse), atol=1e-3)


def test_unselected_keys_are_never_read_and_bad_ids_are_skipped():
    B, H, D, per_frame, F_c, chunks, Lq = 1, 2, 128, 130, 1, 6, 130
    q, kc, vc, L, cap, q_pos0 = _inputs(B, H, D, per_frame, F_c, chunks, Lq, 0, 91)
    pool, _, _ = _pool(kc, per_frame)
    sel = _select(q, pool, cap, per_frame, q_pos0, L, 2, 3)
    out, lse = _hsa_attn(q, kc, vc, q_pos0, L, per_frame, sel)
    s = sel.cpu().numpy()
    kc2, vc2 = kc.clone(), vc.clone()
    for b in range(B):
        for h in range(H):
            keep = hsa.visible_keys(s[b, h, 0].astype(np.int64), q_pos0, q_pos0 + L, per_frame)
            drop = torch.tensor(np.setdiff1d(np.arange(cap), keep), device=dev())
            kc2[b, h, drop] = float("nan")
            vc2[b, h, drop] = float("nan")
    out2, lse2 = _hsa_attn(q, kc2, vc2, q_pos0, L, per_frame, sel)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # ids that are negative or outside the history are skipped: append junk
    nbf = hsa.blocks_per_frame(per_frame)
    n_hist_blocks = (chunks - 1) * nbf
    junk = torch.tensor([-5, n_hist_blocks, n_hist_blocks + 7, 1 << 30], dtype=torch.int32,
                        device=dev())
    sel_j = torch.cat([sel, junk.expand(B, H, sel.shape[2], 4)], dim=3).contiguous()
    out3, lse3 = _hsa_attn(q, kc, vc, q_pos0, L, per_frame, sel_j)
    assert torch.equal(out, out3) and torch.equal(lse, lse3)


def test_480p_chunk_sampled_rows():
    # the 1.3B-shape chunk at t0 18: 4680 queries, 12 heads, 7-chunk cache,
    # 6 of 18 history frames, 32 blocks of 64 keys kept per query block
    w = STEP480
    per_frame, L, cap = w.grid_h * w.grid_w, w.chunk_tokens, w.cap
    q = normal((1, w.lq, w.H, w.D), 4801).to(dev())
    kc = normal((1, w.H, cap, w.D), 4802).to(dev())
    vc = normal((1, w.H, cap, w.D), 4803).to(dev())
    pool, fr, bl = _pool(kc, per_frame)
    _check_pool(kc, per_frame, fr, bl)
    sel = _select(q, pool, cap, per_frame, w.q_pos0, L, 6, 32)
    exact = _check_selection(q, kc, per_frame, L, w.q_pos0, 6, 32, sel)
    total = sel.shape[1] * sel.shape[2]
    print(f"  480P: {exact} of {total} query blocks matched exactly", flush=True)
    # Which blocks are compared exactly follows from the exact fp64 scores
    # and the bound alone (not from the GPU): on this seeded input 202 of the
    # 228.  Every one of them must match, and the count itself is checked so
    # that a change of bound or input cannot quietly shrink the coverage.
    assert exact == _separated(q, kc, per_frame, L, w.q_pos0, 6, 32) >= 0.85 * total
    out, lse = _hsa_attn(q, kc, vc, w.q_pos0, L, per_frame, sel)
    rows = np.unique(np.concatenate([np.arange(0, w.lq, 97), [w.lq - 1, 255, 256, 4607, 4608]]))
    s64 = sel.cpu().numpy().astype(np.int64)
    o_ref, lse_ref = hsa.attn(f64(q), f64(kc), f64(vc), s64, w.q_pos0, w.q_pos0 + L, per_frame,
                              rows=rows)
    assert_attn_close(f64(out)[:, rows], o_ref, "hsa 480P")
    np.testing.assert_allclose(f64(lse)[:, :, rows], lse_ref, atol=2e-3)


def test_rollout_with_hsa_every_chunk():
    # a 4-chunk rollout (one 8x8 frame per chunk, 2 heads of 64) with HSA
    # keeping 2 frames and 2 blocks: each denoising call is checked against
    # the oracle on the rollout's own selection and cache contents
    from autoregressive_video_diffusion_amd.rollout import ChunkRollout

    B, H, D, gh, gw = 1, 2, 64, 8, 8
    ro = ChunkRollout(B, H, D, 1, gh, gw, window=4, max_chunks=5, device=dev(), hsa=(2, 2))
    L = ro.L
    for c in range(4):
        q = normal((B, L, H, D), 700 + 3 * c).to(dev())
        k = normal((B, L, H, D), 701 + 3 * c).to(dev())
        v = normal((B, L, H, D), 702 + 3 * c).to(dev())
        q_out, out = torch.empty_like(q), torch.empty_like(q)
        ro.denoise(c, q, k, v, q_out, out)
        torch.cuda.synchronize()
        sel = ro.sel.cpu().numpy().astype(np.int64)
        if c == 0:
            assert (sel == -1).all()
        else:
            assert (sel[..., :min(2, c)] >= 0).all()
        o_ref, _ = hsa.attn(f64(q_out), f64(ro.k_cache), f64(ro.v_cache), sel, c * L, (c + 1) * L,
                            gh * gw)
        assert_attn_close(f64(out), o_ref, f"hsa rollout chunk {c}")
        ro.update(c, k, v)


def test_hsa_call_replays_from_a_hip_graph():
    # pooling, selection and the block-sparse attention captured once and
    # replayed: every replay writes the eager call's pool, selection and
    # output bit for bit, with eager calls between the replays
    B, H, D, per_frame, F_c, chunks, Lq, kf, kb = 1, 2, 128, 100, 2, 5, 200, 3, 6
    q, kc, vc, L, cap, q_pos0 = _inputs(B, H, D, per_frame, F_c, chunks, Lq, 0, 91)
    pool = torch.empty(crattn.hsa_pool_bytes(B, H, cap, D, per_frame) // 4, dtype=torch.float32,
                       device=dev())
    sel = torch.empty(B, H, -(-Lq // 256), kb, dtype=torch.int32, device=dev())
    out = torch.empty_like(q)
    lse = torch.empty(B, H, Lq, dtype=torch.float32, device=dev())

    def call():
        crattn.hsa_pool_keys(kc, 0, cap, per_frame, pool)
        crattn.hsa_select(q, pool, cap, cap, per_frame, q_pos0, L, kf, kb, sel)
        crattn.hsa_attn(q, kc, vc, cap, q_pos0, L, per_frame, sel, out, lse)

    call()
    torch.cuda.synchronize()
    ref = (pool.clone(), sel.clone(), out.clone(), lse.clone())
    assert (ref[1] >= 0).any()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        pool.fill_(float("nan"))
        sel.fill_(-7)
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("pool", "sel", "out", "lse"), (pool, sel, out, lse), ref):
            assert torch.equal(got, want), f"replay {rep}: {name}"
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[2])


# --------------------------------------------------------------------------- ring window


@pytest.mark.parametrize("own,Lq,q_off,kf,kb", [(2, 200, 0, 3, 5), (0, 100, 62, 2, 7),
                                                 (4, 200, 0, 8, 40)])
def test_full_ring_own_slot_anywhere_every_row(own, Lq, q_off, kf, kb):
    # a full ring of 5 slots, the own chunk in slot `own`: every other slot
    # is history ("LIGHT FORCING" §2.2 over the rolling window)
    B, H, D, per_frame, F_c, chunks = 1, 2, 128, 100, 2, 5
    q, kc, vc, L, cap, q_pos0 = _inputs(B, H, D, per_frame, F_c, chunks, Lq, q_off, 300 + own,
                                        own=own)
    pool, fr, bl = _pool(kc, per_frame)
    sel = _select(q, pool, cap, per_frame, q_pos0, L, kf, kb)
    _check_selection(q, kc, per_frame, L, q_pos0, kf, kb, sel)
    nbf = hsa.blocks_per_frame(per_frame)
    s = sel.cpu().numpy()
    assert not (((s // nbf) // F_c == own) & (s >= 0)).any(), "own chunk selected"
    out, lse = _hsa_attn(q, kc, vc, q_pos0, L, per_frame, sel)
    own0 = own * L
    o_ref, lse_ref = hsa.attn(f64(q), f64(kc), f64(vc), s.astype(np.int64), own0, own0 + L,
                              per_frame)
    assert_attn_close(f64(out), o_ref, f"hsa ring own slot {own}")
    np.testing.assert_allclose(f64(lse), lse_ref, atol=2e-3)
    if kf >= (chunks - 1) * F_c and kb >= (chunks - 1) * F_c * nbf:
        # everything selected: the dense attention over the whole ring
        o_d, _ = oracle.attn(f64(q), f64(kc), f64(vc), cap, (chunks - 1) * L + q_off, L)
        assert_attn_close(f64(out), o_d, "hsa ring, everything selected, vs dense")


def test_select_with_nan_and_inf_scores_stays_in_bounds():
    # a NaN query block and an infinite pooled frame: the selection still
    # writes at most kb valid, ascending history ids per row and nothing past
    # its rows (the output buffer has a guard tail)
    B, H, D, per_frame, F_c, chunks, Lq, kf, kb = 1, 2, 128, 400, 2, 5, 600, 3, 5
    q, kc, vc, L, cap, q_pos0 = _inputs(B, H, D, per_frame, F_c, chunks, Lq, 0, 401, own=1)
    q[:, 256:300] = float("nan")               # query block 1 has NaN rows
    pool, _, _ = _pool(kc, per_frame)
    nf = cap // per_frame
    pool.view(-1)[:B * H * nf * D].view(B, H, nf, D)[:, :, 6, 0] = float("inf")   # frame 6
    pool.view(-1)[:B * H * nf * D].view(B, H, nf, D)[:, 1, 7, :] = float("nan")   # frame 7, head 1
    nqb = -(-Lq // 256)
    n = B * H * nqb * kb
    buf = torch.full((n + 256,), 12345, dtype=torch.int32, device=dev())
    sel = buf[:n].view(B, H, nqb, kb)
    crattn.hsa_select(q, pool, cap, cap, per_frame, q_pos0, L, kf, kb, sel)
    torch.cuda.synchronize()
    assert (buf[n:] == 12345).all(), "write past the selection"
    nbf = hsa.blocks_per_frame(per_frame)
    hist = hsa.history_frames(cap, q_pos0, L, per_frame)
    s = sel.cpu().numpy()
    for idx in np.ndindex(s.shape[:3]):
        row = s[idx]
        v = row[row >= 0]
        assert len(v) == kb and (row[len(v):] == -1).all()
        assert np.all(np.diff(v) > 0) and np.isin(v // nbf, hist).all()
        assert len(np.unique(v // nbf)) <= kf
    # the attention over that selection stays in bounds too (finite rows)
    out, _ = _hsa_attn(q, kc, vc, q_pos0, L, per_frame, sel)
    assert torch.isfinite(out[:, :256]).all() and torch.isfinite(out[:, 300:]).all()


def test_rollout480_hsa_through_the_wrapped_ring():
    # ten 480P chunks through a 7-slot ring with HSA (6 frames, 32 blocks):
    # chunks 7..9 sit in slots 0..2 of a full ring, with history on both
    # sides of the own slot.  The last denoising call of every chunk is
    # checked: its selection for validity against exact scores, and its
    # attention on sampled rows of all 12 heads against the oracle over that
    # selection and the rollout's cache.
    from autoregressive_video_diffusion_amd.rollout import ChunkRollout
    from gpu_helpers import sample_rows
    from workloads import ROLLOUT480 as w

    kf, kb = 6, 32
    ro = ChunkRollout(w.B, w.H, w.D, w.frames, w.grid_h, w.grid_w, window=7, max_chunks=10,
                      device=dev(), hsa=(kf, kb))
    n, per_frame = ro.L, w.grid_h * w.grid_w
    q_out = torch.empty(w.B, n, w.H, w.D, dtype=torch.bfloat16, device=dev())
    out = torch.empty_like(q_out)
    for c in range(10):
        for j in range(4):
            q, k, v = (t.to(dev()) for t in call_qkv(w, 100 + c * 5 + j))
            ro.denoise(c, q, k, v, q_out, out)
        torch.cuda.synchronize()
        kv_len = min(c + 1, 7) * n
        own0 = ro.slot(c) * n
        sel = ro.sel.clone()
        if c > 0:
            _check_selection(q_out, ro.k_cache, per_frame, n, own0, kf, kb, sel, kv_len=kv_len)
        rows = sample_rows(n, n_random=6, seed=c)
        o_ref, _ = hsa.attn(f64(q_out), f64(ro.k_cache), f64(ro.v_cache),
                            sel.cpu().numpy().astype(np.int64), own0, own0 + n, per_frame,
                            rows=rows)
        assert_attn_close(f64(out)[:, rows], o_ref, f"hsa rollout chunk {c} (slot {ro.slot(c)})")
        _, k, v = call_qkv(w, 100 + c * 5 + 4)
        ro.update(c, k.to(dev()), v.to(dev()))


def test_win720_hsa_sampled_rows():
    # the 720P window at t0 = 81 with HSA (6 of 18 history frames, 32
    # blocks): selection validity on 3 heads, attention on sampled rows
    from gpu_helpers import sample_rows
    from workloads import WIN720 as w

    per_frame, L, cap = w.grid_h * w.grid_w, w.chunk_tokens, w.cap
    heads = [0, 17, 39]
    q = normal((1, w.lq, w.H, w.D), 7201).to(dev())
    kc = normal((1, w.H, cap, w.D), 7202).to(dev())
    vc = normal((1, w.H, cap, w.D), 7203).to(dev())
    own0 = w.slot * L
    pool = torch.empty(crattn.hsa_pool_bytes(1, w.H, cap, w.D, per_frame) // 4,
                       dtype=torch.float32, device=dev())
    crattn.hsa_pool_keys(kc, 0, cap, per_frame, pool)
    sel = _select(q, pool, cap, per_frame, own0, L, 6, 32)
    out, lse = _hsa_attn(q, kc, vc, own0, L, per_frame, sel)
    assert torch.isfinite(out).all()
    qh, kh, vh, sh = q[:, :, heads], kc[:, heads], vc[:, heads], sel[:, heads]
    _check_selection(qh, kh, per_frame, L, own0, 6, 32, sh)
    rows = sample_rows(w.lq, n_random=10)
    o_ref, lse_ref = hsa.attn(f64(qh), f64(kh), f64(vh), sh.cpu().numpy().astype(np.int64), own0,
                              own0 + L, per_frame, rows=rows)
    assert_attn_close(f64(out[:, rows][:, :, heads]), o_ref, "hsa 720P window")
    np.testing.assert_allclose(f64(lse[:, heads][:, :, rows]), lse_ref, atol=2e-3)
