"""Pins of the hierarchical block-sparse attention oracle (oracle/hsa.py)
against facts that do not come from the oracle itself.

Source: "LIGHT FORCING" technical summary, §2.2 (HSA: mean-pooled block
and frame keys, frame selection, block selection inside the selected
frames, attention over the selected blocks only, cost constant in the
number of history frames)."""
import itertools

import numpy as np
import pytest

import oracle
from oracle import hsa


def _rng(seed):
    return np.random.default_rng(seed)


def test_block_layout_ragged_frames():
    # frames of 100 tokens, 64-token blocks: 64 + 36 per frame, frame-major
    assert hsa.blocks_per_frame(100) == 2
    assert [hsa.block_range(b, 100) for b in range(5)] == [(0, 64), (64, 100), (100, 164),
                                                           (164, 200), (200, 264)]
    # the 480P frame: 1560 tokens = 24 full blocks + one of 24
    assert hsa.blocks_per_frame(1560) == 25 and hsa.block_range(24, 1560) == (1536, 1560)


def test_pooled_score_is_the_mean_of_the_score_block():
    # q_bar . k_bar = mean over the block pair of q_i . k_j (bilinearity):
    # pins both pooling ranges against the full score matrix
    rng = _rng(1)
    per_frame, bk, bq = 100, 64, 32
    q = rng.standard_normal((1, 70, 1, 8))
    k = rng.standard_normal((1, 1, 300, 8))
    frames, blocks = hsa.pool_keys(k, per_frame, bk)
    qp = hsa.pool_queries(q, bq)
    S = q[0, :, 0] @ k[0, 0].T  # [70, 300] full scores
    for i in range(qp.shape[2]):
        rows = slice(i * bq, min(70, (i + 1) * bq))
        for blk in range(blocks.shape[2]):
            s, e = hsa.block_range(blk, per_frame, bk)
            assert np.isclose(qp[0, 0, i] @ blocks[0, 0, blk], S[rows, s:e].mean())
        for f in range(frames.shape[2]):
            cols = slice(f * per_frame, (f + 1) * per_frame)
            assert np.isclose(qp[0, 0, i] @ frames[0, 0, f], S[rows, cols].mean())


def test_topk_against_brute_force_subsets():
    rng = _rng(2)
    for n, k in [(6, 2), (7, 3), (5, 5), (4, 6)]:
        for _ in range(20):
            s = np.round(rng.standard_normal(n), 1)  # coarse values: ties happen
            got = hsa.topk(s, k)
            kk = min(k, n)
            # the best subset: largest score sum, then the lexicographically
            # smallest index set among equal sums
            best = max(itertools.combinations(range(n), kk),
                       key=lambda c: (round(sum(s[list(c)]), 9), [-x for x in c]))
            assert list(got) == sorted(best), (s, k, got, best)


def test_blocks_come_only_from_selected_frames():
    # frame 0 has the highest-scoring single block but a low frame mean;
    # with kf = 1 the hierarchy must take frame 1's blocks, a flat top-k
    # over all blocks would take frame 0's
    per_frame, bk, D = 128, 64, 4
    k = np.zeros((1, 1, 3 * per_frame, D))
    k[0, 0, 0:64, 0] = 10.0      # frame 0, block 0: strong
    k[0, 0, 64:128, 0] = -9.5    # frame 0, block 1: pulls frame 0's mean down
    k[0, 0, 128:256, 0] = 2.0    # frame 1: uniformly good
    k[0, 0, 256:384, 0] = 1.0    # frame 2: current chunk, not history
    q = np.zeros((1, 16, 1, D))
    q[..., 0] = 1.0
    frames, blocks = hsa.pool_keys(k, per_frame, bk)
    sel = hsa.select(q, frames, blocks, hist=2, per_frame=per_frame, kf=1, kb=1, bq=16, bk=bk)
    assert list(sel[0, 0, 0]) == [2]    # block 0 of frame 1
    flat = hsa.topk(blocks[0, 0, :4] @ np.eye(D)[0], 1)
    assert list(flat) == [0]
    # with kf = 2 the strong block is reachable and wins
    sel2 = hsa.select(q, frames, blocks, hist=2, per_frame=per_frame, kf=2, kb=1, bq=16, bk=bk)
    assert list(sel2[0, 0, 0]) == [0]


def test_padding_when_the_frames_hold_fewer_blocks():
    rng = _rng(3)
    per_frame = 100
    k = rng.standard_normal((1, 2, 300, 8))
    q = rng.standard_normal((1, 40, 2, 8))
    frames, blocks = hsa.pool_keys(k, per_frame)
    sel = hsa.select(q, frames, blocks, hist=2, per_frame=per_frame, kf=1, kb=5, bq=64)
    assert sel.shape == (1, 2, 1, 5)
    assert (sel[..., :2] >= 0).all() and (sel[..., 2:] == -1).all()
    # no history: nothing selected
    sel0 = hsa.select(q, frames, blocks, hist=0, per_frame=per_frame, kf=2, kb=3, bq=64)
    assert (sel0 == -1).all()


@pytest.mark.parametrize("B,H,D,F_c,gh,gw,chunks,Lq,q_off", [
    (1, 2, 64, 1, 8, 8, 4, 64, 0),      # tiny geometry, the last chunk's queries
    (2, 1, 16, 2, 5, 7, 3, 70, 0),      # 35-token frames: one ragged block each
    (1, 2, 32, 1, 10, 10, 3, 37, 50),   # a slice of the last chunk
])
def test_selecting_everything_is_dense_chunk_causal_attention(B, H, D, F_c, gh, gw, chunks, Lq,
                                                               q_off):
    # with every history frame and block chosen, HSA is the dense
    # chunk-causal attention of the C oracle (pages: cost falls, result is
    # the dense one when nothing is dropped)
    rng = _rng(4)
    per_frame = gh * gw
    L = F_c * per_frame
    cap = chunks * L
    q = rng.standard_normal((B, Lq, H, D))
    k = rng.standard_normal((B, H, cap, D))
    v = rng.standard_normal((B, H, cap, D))
    frames, blocks = hsa.pool_keys(k, per_frame)
    n_hist = (chunks - 1) * F_c
    nbf = hsa.blocks_per_frame(per_frame)
    sel = hsa.select(q, frames, blocks, n_hist, per_frame, kf=n_hist, kb=n_hist * nbf, bq=32)
    assert (sel >= 0).all()
    q_pos0 = (chunks - 1) * L + q_off
    o, lse = hsa.attn(q, k, v, sel, (chunks - 1) * L, cap, per_frame, bq=32)
    o_d, lse_d = oracle.attn(q, k, v, cap, q_pos0, L)
    np.testing.assert_allclose(o, o_d, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(lse, lse_d, atol=1e-12, rtol=1e-12)


def test_unselected_keys_do_not_matter_and_selected_ones_do():
    rng = _rng(5)
    per_frame, F_c, chunks, D = 64, 2, 4, 16
    L = F_c * per_frame
    cap = chunks * L
    q = rng.standard_normal((1, 50, 1, D))
    k = rng.standard_normal((1, 1, cap, D))
    v = rng.standard_normal((1, 1, cap, D))
    frames, blocks = hsa.pool_keys(k, per_frame)
    n_hist = (chunks - 1) * F_c
    sel = hsa.select(q, frames, blocks, n_hist, per_frame, kf=2, kb=1, bq=64)
    o, _ = hsa.attn(q, k, v, sel, (chunks - 1) * L, cap, per_frame, bq=64)
    keep = hsa.visible_keys(sel[0, 0, 0], (chunks - 1) * L, cap, per_frame)
    k2, v2 = k.copy(), v.copy()
    drop = np.setdiff1d(np.arange(cap), keep)
    k2[0, 0, drop] = np.nan
    v2[0, 0, drop] = np.nan
    o2, _ = hsa.attn(q, k2, v2, sel, (chunks - 1) * L, cap, per_frame, bq=64)
    assert np.array_equal(o, o2)
    blk_rows = np.arange(*hsa.block_range(int(sel[0, 0, 0, 0]), per_frame))
    v3 = v.copy()
    v3[0, 0, blk_rows] += 1.0
    o3, _ = hsa.attn(q, k, v3, sel, (chunks - 1) * L, cap, per_frame, bq=64)
    assert not np.allclose(o, o3)


def test_budget_is_constant_in_history_length():
    # the number of attended keys is the own chunk plus at most kb blocks,
    # whatever the number of history chunks
    rng = _rng(6)
    per_frame, F_c, D, kf, kb = 100, 1, 8, 2, 3
    for chunks in (3, 6, 12):
        cap = chunks * per_frame
        k = rng.standard_normal((1, 1, cap, D))
        q = rng.standard_normal((1, 30, 1, D))
        frames, blocks = hsa.pool_keys(k, per_frame)
        sel = hsa.select(q, frames, blocks, chunks - 1, per_frame, kf, kb, bq=64)
        keys = hsa.visible_keys(sel[0, 0, 0], cap - per_frame, cap, per_frame)
        assert per_frame < len(keys) <= per_frame + kb * 64


# --------------------------------------------------------------------------- ring window


def test_history_frames_of_a_filling_and_of_a_full_ring():
    # 3 frames of 10 tokens per chunk; ring of 7 slots
    per_frame, L = 10, 30
    # filling: chunk 2 in slot 2 sees slots 0..2, history = frames 0..5
    assert list(hsa.history_frames(3 * L, 2 * L, L, per_frame)) == list(range(6))
    # chunk 0: no history
    assert len(hsa.history_frames(L, 5, L, per_frame)) == 0
    # full ring, own chunk in slot 3: every other slot's frames, ascending
    want = list(range(0, 9)) + list(range(12, 21))
    assert list(hsa.history_frames(7 * L, 3 * L + 7, L, per_frame)) == want
    # the integer form is the filling case
    rng = _rng(7)
    k = rng.standard_normal((1, 1, 4 * L, 8))
    q = rng.standard_normal((1, 20, 1, 8))
    frames, blocks = hsa.pool_keys(k, per_frame, bk=4)
    a = hsa.select(q, frames, blocks, 9, per_frame, kf=4, kb=5, bq=8, bk=4)
    b = hsa.select(q, frames, blocks, hsa.history_frames(4 * L, 3 * L, L, per_frame), per_frame,
                   kf=4, kb=5, bq=8, bk=4)
    assert np.array_equal(a, b)


def _rotate_slots(x, r, L, axis):
    """Move the content of ring slot i to slot (i + r) mod W along `axis`."""
    return np.roll(x, r * L, axis=axis)


@pytest.mark.parametrize("own,r", [(2, 1), (0, 3), (4, 2), (1, 4)])
def test_ring_rotation_moves_the_selection_with_the_slots(own, r):
    # "Sparse VideoGen2" §2.A: attention does not depend on where a key sits.
    # Rotating the ring's slots (and the own slot with them) must rotate the
    # chosen blocks with their frames and leave every output unchanged.
    rng = _rng(10 + own)
    W, F_c, gh, gw, D, H = 5, 2, 4, 5, 16, 2
    per_frame = gh * gw
    L = F_c * per_frame
    cap = W * L
    nbf = hsa.blocks_per_frame(per_frame, 8)
    q = rng.standard_normal((1, 24, H, D))
    k = rng.standard_normal((1, H, cap, D))
    v = rng.standard_normal((1, H, cap, D))

    def run(k, v, own):
        frames, blocks = hsa.pool_keys(k, per_frame, bk=8)
        hist = hsa.history_frames(cap, own * L, L, per_frame)
        assert len(hist) == (W - 1) * F_c
        sel = hsa.select(q, frames, blocks, hist, per_frame, kf=3, kb=4, bq=8, bk=8)
        o, lse = hsa.attn(q, k, v, sel, own * L, (own + 1) * L, per_frame, bq=8, bk=8)
        return sel, o, lse

    sel, o, lse = run(k, v, own)
    sel_r, o_r, lse_r = run(_rotate_slots(k, r, L, 2), _rotate_slots(v, r, L, 2), (own + r) % W)

    def move(blk):
        f, j = divmod(int(blk), nbf)
        s, fi = divmod(f, F_c)
        return (((s + r) % W) * F_c + fi) * nbf + j

    for idx in np.ndindex(sel.shape[:3]):
        assert sorted(move(b) for b in sel[idx] if b >= 0) == [b for b in sel_r[idx] if b >= 0]
    # the own slot is never a candidate
    assert not any((b // nbf) // F_c == own for b in sel.ravel() if b >= 0)
    np.testing.assert_allclose(o_r, o, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(lse_r, lse, atol=1e-12)


@pytest.mark.parametrize("own", [0, 2, 4])
def test_full_ring_selecting_everything_is_dense_attention(own):
    # own chunk anywhere in a full ring, every history block chosen: the
    # dense attention over every slot (the dense oracle sees every key when
    # the query sits in the last chunk of a full cache)
    rng = _rng(20 + own)
    W, F_c, per_frame, D, H, Lq, q_off = 5, 2, 36, 16, 2, 50, 11
    L = F_c * per_frame
    cap = W * L
    q = rng.standard_normal((1, Lq, H, D))
    k = rng.standard_normal((1, H, cap, D))
    v = rng.standard_normal((1, H, cap, D))
    frames, blocks = hsa.pool_keys(k, per_frame)
    hist = hsa.history_frames(cap, own * L + q_off, L, per_frame)
    nbf = hsa.blocks_per_frame(per_frame)
    sel = hsa.select(q, frames, blocks, hist, per_frame, kf=len(hist), kb=len(hist) * nbf, bq=16)
    assert (sel >= 0).all()
    o, lse = hsa.attn(q, k, v, sel, own * L, (own + 1) * L, per_frame, bq=16)
    o_d, lse_d = oracle.attn(q, k, v, cap, (W - 1) * L + q_off, L)
    np.testing.assert_allclose(o, o_d, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(lse, lse_d, atol=1e-12)
