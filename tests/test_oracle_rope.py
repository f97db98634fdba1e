"""Pins of the oracle's 3D RoPE, position decode, table and append (CPU only).

Each test checks the oracle against something other than itself: the
workload statement's fixtures, closed forms, group/invariance properties of
rotations, or the brute-force matrix form in tests/brute.py.
"""
import math
import os

import numpy as np
import pytest

import brute
import oracle
from workloads import SP480, STEP480, TINY, WIN720

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


def test_split_matches_workload_statement():
    for D, dt, dh, dw in _rows("head_dim_splits.txt"):
        assert oracle.split(int(D)) == (int(dt), int(dh), int(dw))


def test_chunk_geometry_fixture():
    for row in _rows("chunk_geometry.txt"):
        name, H, D, F, gh, gw, Lc, nc, kv, t0, off, n = row[0], *map(int, row[1:])
        assert F * gh * gw == Lc and nc * Lc == kv
    w = {r[0]: list(map(int, r[1:])) for r in _rows("chunk_geometry.txt")}
    for wl, key in ((TINY, "tiny"), (STEP480, "step480"), (SP480, "sp480"), (WIN720, "win720")):
        H, D, F, gh, gw, Lc, nc, kv, t0, off, n = w[key]
        assert (wl.H, wl.D, wl.frames, wl.grid_h, wl.grid_w) == (H, D, F, gh, gw)
        assert (wl.chunk_tokens, wl.kv_len, wl.t0, wl.tok_off, wl.lq) == (Lc, kv, t0, off, n)


@pytest.mark.parametrize("t0,tok_off,n,gh,gw", [(3, 0, 64, 8, 8), (0, 0, 256, 8, 8),
                                                 (18, 2925, 585, 30, 52), (18, 0, 4680, 30, 52),
                                                 (81, 0, 10800, 45, 80), (5, 7, 200, 3, 5)])
def test_positions_match_raster_enumeration(t0, tok_off, n, gh, gw):
    got = oracle.positions(n, t0, tok_off, gh, gw)
    want = brute.raster_positions(n, t0, tok_off, gh, gw)
    np.testing.assert_array_equal(got, want)


def test_positions_sp_slice_closed_form():
    # frame size 30*52 = 1560; 2925 = 1*1560 + 26*52 + 13; 3509 = 2*1560 + 7*52 + 25
    pos = oracle.positions(585, 18, 2925, 30, 52)
    assert tuple(pos[0]) == (19, 26, 13)
    assert tuple(pos[-1]) == (20, 7, 25)
    # the slice crosses the frame boundary at chunk token 3120 = 2 * 1560
    assert int((pos[:, 0] == 19).sum()) == 3120 - 2925 == 195
    assert int((pos[:, 0] == 20).sum()) == 585 - 195


def test_identity_at_origin():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 1, 3, 64))
    y = oracle.rope(x, 0, 0, 8, 8)
    np.testing.assert_array_equal(y, x)


@pytest.mark.parametrize("D", [64, 128])
def test_table_closed_forms(D):
    dt, dh, dw = oracle.split(D)
    max_t, max_h, max_w = 84, 45, 80
    c, s = oracle.rope_table(D, max_t, max_h, max_w)
    assert c.shape == (max_t * dt // 2 + max_h * dh // 2 + max_w * dw // 2,)
    offs = [0, max_t * dt // 2, max_t * dt // 2 + max_h * dh // 2]
    for a, (Da, mx) in enumerate(zip((dt, dh, dw), (max_t, max_h, max_w))):
        for p in (0, 1, mx - 1):
            base = offs[a] + p * (Da // 2)
            # pair 0 rotates by exactly p radians (frequency theta^0 = 1)
            assert c[base] == pytest.approx(math.cos(p), abs=1e-15)
            assert s[base] == pytest.approx(math.sin(p), abs=1e-15)
            # the last pair has frequency theta^-(Da-2)/Da
            f_last = 10000.0 ** (-(Da - 2) / Da)
            last = base + Da // 2 - 1
            assert c[last] == pytest.approx(math.cos(p * f_last), abs=1e-15)
            assert s[last] == pytest.approx(math.sin(p * f_last), abs=1e-15)
    # unit circle
    np.testing.assert_allclose(c * c + s * s, 1.0, atol=1e-15)


def test_table_matches_rotation_matrix_entries():
    D = 64
    c, s = oracle.rope_table(D, 4, 8, 8)
    dt, dh, dw = oracle.split(D)
    offs = [0, 4 * dt // 2, 4 * dt // 2 + 8 * dh // 2]
    for (pt, ph, pw) in [(0, 0, 0), (3, 5, 7), (2, 7, 1)]:
        R = brute.rotation_matrix(D, pt, ph, pw)
        col = 0
        for a, (Da, p) in enumerate(zip((dt, dh, dw), (pt, ph, pw))):
            for j in range(Da // 2):
                e = offs[a] + p * (Da // 2) + j
                assert R[col, col] == pytest.approx(c[e], abs=1e-15)
                assert R[col + 1, col] == pytest.approx(s[e], abs=1e-15)
                col += 2


@pytest.mark.parametrize("D,t0", [(64, 3), (128, 81)])
def test_norm_preserved_per_pair(D, t0):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 50, 2, D)) * 3.0
    y = oracle.rope(x, t0, 17, 30, 52)
    nx = np.hypot(x[..., 0::2], x[..., 1::2])
    ny = np.hypot(y[..., 0::2], y[..., 1::2])
    np.testing.assert_allclose(ny, nx, rtol=1e-12)


def test_group_structure():
    rng = np.random.default_rng(3)
    D = 128
    x = rng.standard_normal((1, 20, 2, D))
    p = rng.integers(0, 90, size=(20, 3))
    p2 = rng.integers(0, 90, size=(20, 3))
    # R(p') R(p) = R(p + p')
    a = oracle.rope_pos(oracle.rope_pos(x, p), p2)
    b = oracle.rope_pos(x, p + p2)
    np.testing.assert_allclose(a, b, atol=1e-12)
    # R(p)^T = R(-p): rotating back restores x
    back = oracle.rope_pos(oracle.rope_pos(x, p), -p)
    np.testing.assert_allclose(back, x, atol=1e-12)


def test_relative_position_property():
    rng = np.random.default_rng(4)
    D = 128
    q = rng.standard_normal((1, 1, 1, D))
    k = rng.standard_normal((1, 1, 1, D))
    for _ in range(10):
        p = rng.integers(0, 84, size=(1, 3))
        pp = rng.integers(0, 84, size=(1, 3))
        lhs = float((oracle.rope_pos(q, p) * oracle.rope_pos(k, pp)).sum())
        rhs = float((q * oracle.rope_pos(k, pp - p)).sum())
        assert lhs == pytest.approx(rhs, abs=1e-12)


def test_time_shift_leaves_scores_unchanged():
    # The same chunk geometry at t0 = 81 and at t0 = 18: every q.k score within
    # the chunk and against a key at a shifted earlier frame is unchanged.
    rng = np.random.default_rng(5)
    D, n = 128, 120
    q = rng.standard_normal((1, n, 2, D))
    k = rng.standard_normal((1, n, 2, D))
    s_late = np.einsum("bihd,bjhd->bhij", oracle.rope(q, 81, 1000, 45, 80),
                       oracle.rope(k, 78, 1000, 45, 80))
    s_early = np.einsum("bihd,bjhd->bhij", oracle.rope(q, 18, 1000, 45, 80),
                        oracle.rope(k, 15, 1000, 45, 80))
    np.testing.assert_allclose(s_late, s_early, atol=1e-10)


def test_local_equals_slice_of_global():
    rng = np.random.default_rng(6)
    D = 128
    full = rng.standard_normal((1, 4680, 2, D))
    y_full = oracle.rope(full, 18, 0, 30, 52)
    y_slice = oracle.rope(full[:, 2925:3510], 18, 2925, 30, 52)
    np.testing.assert_array_equal(y_slice, y_full[:, 2925:3510])
    # chunk t0 = 18 alone equals its rows of a 21-frame sequence rotated from t0 = 0
    seq = rng.standard_normal((1, 21 * 1560 // 10, 1, D))  # first 3276 tokens
    y_seq = oracle.rope(seq, 0, 0, 30, 52)
    part = seq[:, 3 * 1560:3276]
    y_part = oracle.rope(part, 3, 0, 30, 52)
    np.testing.assert_array_equal(y_part, y_seq[:, 3 * 1560:3276])


def test_matches_brute_force_matrices_tiny():
    rng = np.random.default_rng(7)
    B, H, D = 2, 2, 64
    x = rng.standard_normal((B, 256, H, D))
    # all 256 tokens of the four one-frame 8x8 chunks, t0 = 0
    got = oracle.rope(x, 0, 0, 8, 8)
    want = brute.rope(x, brute.raster_positions(256, 0, 0, 8, 8))
    np.testing.assert_allclose(got, want, atol=1e-12)
    # the last chunk alone, from its global time index
    got3 = oracle.rope(x[:, 192:], 3, 0, 8, 8)
    np.testing.assert_allclose(got3, want[:, 192:], atol=1e-12)


def test_matches_brute_force_matrices_d128():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 40, 3, 128))
    got = oracle.rope(x, 18, 2925, 30, 52)
    want = brute.rope(x, brute.raster_positions(40, 18, 2925, 30, 52))
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_append_is_a_transposed_copy():
    rng = np.random.default_rng(9)
    B, n, H, D, cap, pos0 = 2, 7, 3, 8, 20, 5
    x = rng.standard_normal((B, n, H, D))
    cache = np.full((B, H, cap, D), -7.0)
    oracle.append(cache, x, pos0)
    np.testing.assert_array_equal(cache[:, :, pos0:pos0 + n], x.transpose(0, 2, 1, 3))
    assert (cache[:, :, :pos0] == -7.0).all() and (cache[:, :, pos0 + n:] == -7.0).all()
    with pytest.raises(ValueError):
        oracle.append(cache, x, cap - n + 1)
