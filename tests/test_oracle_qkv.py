"""Pins for the oracle's fused QKV projection + Causal-RoPE.

The projection is pinned against an explicit triple loop on tiny inputs
(column order Q, K, V, heads contiguous, W in [out, in] layout), and the
composition against the already pinned rotation: with weights that select
input columns, Q' must equal the oracle rotation of those columns exactly.
Rotations preserve each pair's norm, which pins the composition without
the rotary code (a dropped rotation or a swapped operand fails it)."""
import numpy as np

import oracle


def _loops(x, w, H, D):
    B, n, C = x.shape
    out = np.zeros((3, B, n, H, D))
    for b in range(B):
        for i in range(n):
            for part in range(3):
                for h in range(H):
                    for d in range(D):
                        row = part * H * D + h * D + d
                        out[part, b, i, h, d] = sum(x[b, i, c] * w[row, c] for c in range(C))
    return out


def test_projection_matches_explicit_loops():
    rng = np.random.default_rng(3)
    B, n, C, H, D = 2, 3, 5, 2, 4
    x = rng.standard_normal((B, n, C))
    w = rng.standard_normal((3 * H * D, C))
    q, k, v = oracle.qkv_project(x, w, H, D)
    ref = _loops(x, w, H, D)
    np.testing.assert_allclose(q, ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, ref[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(v, ref[2], rtol=0, atol=1e-12)


def test_selection_weights_reduce_to_the_pinned_rotation():
    # C = H*D; W_q = I, W_k = 2 I, W_v = column reversal: Q' = rope(x),
    # K' = 2 rope(x), V = x reversed along the features
    rng = np.random.default_rng(4)
    B, H, D, gh, gw = 1, 2, 64, 8, 8
    n = 2 * gh * gw
    C = H * D
    x = rng.standard_normal((B, n, C))
    eye = np.eye(C)
    w = np.concatenate([eye, 2 * eye, eye[::-1]], axis=0)
    q, k, v = oracle.qkv_rope(x, w, H, D, 3, 0, gh, gw)
    xr = x.reshape(B, n, H, D)
    rq = oracle.rope(np.ascontiguousarray(xr), 3, 0, gh, gw)
    np.testing.assert_allclose(q, rq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(k, 2 * rq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(v, x[:, :, ::-1].reshape(B, n, H, D), rtol=0, atol=0)


def test_rotation_preserves_pair_norms_of_the_projection():
    rng = np.random.default_rng(5)
    B, n, C, H, D = 1, 40, 48, 2, 64
    x = rng.standard_normal((B, n, C))
    w = rng.standard_normal((3 * H * D, C)) / np.sqrt(C)
    q0, k0, _ = oracle.qkv_project(x, w, H, D)
    q, k, _ = oracle.qkv_rope(x, w, H, D, 5, 17, 4, 10)
    for a, b in ((q0, q), (k0, k)):
        n0 = a[..., 0::2] ** 2 + a[..., 1::2] ** 2
        n1 = b[..., 0::2] ** 2 + b[..., 1::2] ** 2
        np.testing.assert_allclose(n1, n0, rtol=1e-12, atol=1e-12)
    # and it does rotate (positions are not all zero)
    assert np.abs(q - q0).max() > 1e-3


def test_abs_bound_dominates_the_outputs():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 7, 16))
    w = rng.standard_normal((3 * 2 * 8, 16))
    q, k, v = oracle.qkv_project(x, w, 2, 8)
    aq, ak, av = oracle.qkv_abs(x, w, 2, 8)
    for o, a in ((q, aq), (k, ak), (v, av)):
        assert (np.abs(o) <= a + 1e-12).all()
