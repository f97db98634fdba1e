"""Pins of the oracle's chunk-causal attention (CPU only).

Brute force (full masked score matrix), closed forms (constant V, identical
keys, one dominant key), torch's fp64 CPU scaled_dot_product_attention on a
single chunk, the mask (future perturbation leaves outputs bitwise unchanged),
cache form = full-sequence form, key-order invariance and the LSE merge.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import brute
import oracle

SC64 = 1.0 / math.sqrt(64)


def _tiny(seed=10, B=1, H=2, D=64, n=256):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n, H, D))
    k = rng.standard_normal((B, H, n, D))
    v = rng.standard_normal((B, H, n, D))
    return q, k, v


@pytest.mark.parametrize("B", [1, 2])
def test_matches_brute_force_full_sequence_tiny(B):
    q, k, v = _tiny(B=B)
    o, lse = oracle.attn(q, k, v, kv_len=256, q_pos0=0, chunk_tokens=64, threads=4)
    ob, lseb, P = brute.attention(q, k, v, 256, 0, 64, SC64)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, atol=1e-12)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)


def test_lse_is_natural_logsumexp():
    q, k, v = _tiny()
    o, lse = oracle.attn(q[:, 192:], k, v, kv_len=256, q_pos0=192, chunk_tokens=64)
    S = np.einsum("bihd,bhjd->bhij", q[:, 192:], k) * SC64
    np.testing.assert_allclose(lse, logsumexp(S, axis=-1), atol=1e-12)


def test_last_chunk_sees_all_keys_first_chunk_sees_itself():
    q, k, v = _tiny()
    o3, _ = oracle.attn(q[:, 192:], k, v, kv_len=256, q_pos0=192, chunk_tokens=64)
    ob, _, _ = brute.attention(q[:, 192:], k, v, 256, 192, 64, SC64)
    np.testing.assert_allclose(o3, ob, atol=1e-12)
    o0, _ = oracle.attn(q[:, :64], k, v, kv_len=256, q_pos0=0, chunk_tokens=64)
    o0b, _, _ = brute.attention(q[:, :64], k[:, :, :64], v[:, :, :64], 64, 0, 64, SC64)
    np.testing.assert_allclose(o0, o0b, atol=1e-12)


def test_constant_values_give_that_constant():
    q, k, _ = _tiny()
    v = np.full_like(k, 0.375)
    o, _ = oracle.attn(q, k, v, 256, 0, 64)
    np.testing.assert_allclose(o, 0.375, atol=1e-14)


def test_probabilities_via_one_hot_values_sum_to_one():
    # D >= visible keys: V = identity makes o the probability row itself.
    rng = np.random.default_rng(11)
    D, n = 64, 64
    q = rng.standard_normal((1, n, 1, D))
    k = rng.standard_normal((1, 1, n, D))
    v = np.eye(n)[None, None]
    o, lse = oracle.attn(q, k, v, n, 0, n)
    P = o[0, :, 0, :]
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-13)
    S = (q[0, :, 0] @ k[0, 0].T) * (1.0 / math.sqrt(D))
    np.testing.assert_allclose(P, np.exp(S - lse[0, 0][:, None]), atol=1e-13)


def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 64, 2, 64))
    k = np.broadcast_to(rng.standard_normal((1, 2, 1, 64)), (1, 2, 256, 64)).copy()
    v = rng.standard_normal((1, 2, 256, 64))
    # rows of chunk 1 see keys 0..127
    o, lse = oracle.attn(q, k, v, 256, 64, 64)
    want = v[:, :, :128].mean(axis=2)                         # [B, H, D]
    np.testing.assert_allclose(o, np.broadcast_to(want[:, None], o.shape), atol=1e-12)
    s = (q * k[:, :, 0][:, None]).sum(-1) * SC64              # [B, Lq, H]
    np.testing.assert_allclose(lse, s.transpose(0, 2, 1) + math.log(128), atol=1e-12)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(13)
    D = 64
    k = np.zeros((1, 1, 64, D))
    k[0, 0, np.arange(64), np.arange(64)] = 1.0               # orthonormal keys
    v = rng.standard_normal((1, 1, 64, D))
    j = 37
    q = (200.0 * k[0, 0, j])[None, None, None]                # q = alpha k_j
    o, _ = oracle.attn(q, k, v, 64, 0, 64)
    # weight of any other key is exp(-alpha/sqrt(D)) ~ 1.4e-11 relative
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, j], atol=1e-9)


def test_single_chunk_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(14)
    B, H, n, D = 2, 3, 96, 128
    q = rng.standard_normal((B, n, H, D))
    k = rng.standard_normal((B, H, n, D))
    v = rng.standard_normal((B, H, n, D))
    o, _ = oracle.attn(q, k, v, n, 0, n)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(k), torch.from_numpy(v))
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


@pytest.mark.parametrize("poison", [np.nan, np.inf, -np.inf, 1e30, "random"])
def test_future_chunks_and_capacity_do_not_leak(poison):
    q, k, v = _tiny(seed=15)
    cap = 300
    kk = np.zeros((1, 2, cap, 64))
    vv = np.zeros((1, 2, cap, 64))
    kk[:, :, :256], vv[:, :, :256] = k, v
    base, base_lse = oracle.attn(q, kk, vv, 256, 0, 64)
    kp, vp = kk.copy(), vv.copy()
    rng = np.random.default_rng(16)
    for arr in (kp, vp):
        if poison == "random":
            arr[:, :, 128:] = rng.standard_normal(arr[:, :, 128:].shape) * 1e3
        else:
            arr[:, :, 128:] = poison
    got, got_lse = oracle.attn(q, kp, vp, 256, 0, 64)
    # rows of chunks 0 and 1 see only keys < 128: bitwise unchanged
    np.testing.assert_array_equal(got[:, :128], base[:, :128])
    np.testing.assert_array_equal(got_lse[:, :, :128], base_lse[:, :, :128])
    # capacity beyond kv_len never matters to anyone
    kc, vc = kk.copy(), vv.copy()
    kc[:, :, 256:] = np.nan
    vc[:, :, 256:] = np.nan
    got2, _ = oracle.attn(q, kc, vc, 256, 0, 64)
    np.testing.assert_array_equal(got2, base)


def test_cache_form_equals_full_sequence_form():
    q, k, v = _tiny(seed=17)
    full, full_lse = oracle.attn(q, k, v, 256, 0, 64)
    for c in range(4):
        rows = slice(64 * c, 64 * (c + 1))
        part, part_lse = oracle.attn(q[:, rows], k, v, kv_len=64 * (c + 1), q_pos0=64 * c,
                                     chunk_tokens=64)
        np.testing.assert_array_equal(part, full[:, rows])
        np.testing.assert_array_equal(part_lse, full_lse[:, :, rows])


def test_row_sampling_equals_full_rows():
    q, k, v = _tiny(seed=18)
    full, full_lse = oracle.attn(q, k, v, 256, 0, 64)
    rows = [0, 5, 63, 64, 200, 255]
    part, part_lse = oracle.attn(q, k, v, 256, 0, 64, rows=rows, threads=3)
    np.testing.assert_array_equal(part, full[:, rows])
    np.testing.assert_array_equal(part_lse, full_lse[:, :, rows])


def test_thread_count_does_not_change_results():
    q, k, v = _tiny(seed=19)
    a, la = oracle.attn(q, k, v, 256, 0, 64, threads=1)
    b, lb = oracle.attn(q, k, v, 256, 0, 64, threads=7)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_key_order_invariance_ring_window():
    # A ring of 4 one-chunk slots where every key is visible: rotating the slot
    # order (and any permutation of key/value pairs) leaves o unchanged.
    q, k, v = _tiny(seed=20)
    qq = q[:, 192:]
    o, lse = oracle.attn(qq, k, v, 256, 192, 64)
    perm = np.random.default_rng(21).permutation(256)
    o2, lse2 = oracle.attn(qq, k[:, :, perm], v[:, :, perm], 256, 192, 64)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)
    ring = np.roll(np.arange(256), 64)
    o3, _ = oracle.attn(qq, k[:, :, ring], v[:, :, ring], 256, 192, 64)
    np.testing.assert_allclose(o3, o, atol=1e-12)


def test_lse_merge_of_disjoint_key_sets():
    q, k, v = _tiny(seed=22)
    qq = q[:, 192:]
    o, lse = oracle.attn(qq, k, v, 256, 192, 64)
    # split the visible keys [0, 256) into [0, 100) and [100, 256)
    oa, la = oracle.attn(qq, k[:, :, :100], v[:, :, :100], 100, 192, 64)
    ob, lb = oracle.attn(qq, k[:, :, 100:], v[:, :, 100:], 156, 192, 64)
    om, lm = oracle.lse_merge(oa, la, ob, lb)
    np.testing.assert_allclose(om, o, atol=1e-12)
    np.testing.assert_allclose(lm, lse, atol=1e-12)


def test_scale_argument_is_applied():
    q, k, v = _tiny(seed=23)
    o, _ = oracle.attn(q, k, v, 256, 0, 64, scale=0.3)
    ob, _, _ = brute.attention(q, k, v, 256, 0, 64, 0.3)
    np.testing.assert_allclose(o, ob, atol=1e-12)


def test_empty_visible_set_is_an_error():
    q, k, v = _tiny(seed=24)
    # kv_len = 0: no key exists at all
    with pytest.raises(ValueError):
        oracle.attn(q[:, :4], k, v, 0, 0, 64)
