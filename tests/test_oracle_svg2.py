"""Pins of the semantic-permutation sparse attention oracle (oracle/svg2.py)
against facts that do not come from the oracle itself.

Source: "Sparse VideoGen2" summary, §2.A (k-means clustering of Q and K,
contiguous reordering, the reordered attention equals the dense one), §2.B
(centroid score estimate, top-p selection), §2.C (centroids of the previous
step start k-means)."""
import collections
import itertools

import numpy as np
import pytest

import oracle
from oracle import svg2
from workloads import planted_clusters


def _rng(seed):
    return np.random.default_rng(seed)


def _inertia(x, cent, assign):
    return float(((x - cent[assign]) ** 2).sum())


def test_kmeans_recovers_planted_clusters():
    x, labels = planted_clusters((), 240, 7, 16, seed=3)
    x = x.double().numpy()
    labels = labels.numpy()
    cent, assign = svg2.kmeans(x, 7, 3)
    assert (assign == labels).all()
    # the centroids are the means of the planted groups (summed another way)
    sums = np.zeros((7, 16))
    np.add.at(sums, labels, x)
    np.testing.assert_allclose(cent, sums / np.bincount(labels)[:, None], rtol=0, atol=1e-12)


def test_kmeans_lloyd_objective_never_increases():
    x = _rng(1).standard_normal((300, 8))
    prev = np.inf
    for it in range(1, 7):
        cent, assign = svg2.kmeans(x, 9, it)
        cur = _inertia(x, cent, assign)
        assert cur <= prev + 1e-9
        prev = cur
    # a fixed point after enough iterations: every token is at its nearest
    # centroid (brute force) and every centroid is its members' mean
    cent, assign = svg2.kmeans(x, 9, 60)
    for i in range(len(x)):
        dists = [float(np.dot(x[i] - c, x[i] - c)) for c in cent]
        assert dists[assign[i]] <= min(dists) + 1e-12
    for c in range(9):
        members = [x[i] for i in range(len(x)) if assign[i] == c]
        if members:
            np.testing.assert_allclose(cent[c], np.sum(members, axis=0) / len(members), atol=1e-12)


def test_kmeans_first_assignment_is_the_nearest_initial_centroid():
    rng = _rng(2)
    x = rng.standard_normal((40, 5))
    init = rng.standard_normal((6, 5))
    _, assign = svg2.kmeans(x, 6, 1, init=init)
    for i in range(40):
        d = [float(((x[i] - init[c]) ** 2).sum()) for c in range(6)]
        assert assign[i] == d.index(min(d))


def test_kmeans_tie_and_empty_cluster_and_default_init():
    # token (1, 0) is equally far from (0, 0) and (2, 0): the lower index wins;
    # the centroid at (9, 9) gets no token and keeps its place
    x = np.array([[0.0, 0.0], [1.0, 0.0], [2.0, 0.0]])
    init = np.array([[0.0, 0.0], [2.0, 0.0], [9.0, 9.0]])
    cent, assign = svg2.kmeans(x, 3, 1, init=init)
    assert assign.tolist() == [0, 0, 1]
    np.testing.assert_array_equal(cent, [[0.5, 0.0], [2.0, 0.0], [9.0, 9.0]])
    # without a cache the centroids start at tokens floor(c n / C): 0, 3, 6
    x = np.arange(9.0)[:, None] * np.array([[1.0, -1.0]])
    cent, _ = svg2.kmeans(x, 3, 0)
    np.testing.assert_array_equal(cent, x[[0, 3, 6]])


def test_warm_start_from_converged_centroids_is_a_fixed_point():
    x = _rng(4).standard_normal((120, 6))
    cent, assign = svg2.kmeans(x, 5, 80)
    cent2, assign2 = svg2.kmeans(x, 5, 1, init=cent)
    assert (assign2 == assign).all()
    np.testing.assert_allclose(cent2, cent, atol=1e-12)


def test_permutation_is_a_stable_sort_by_cluster():
    assign = _rng(5).integers(0, 6, 100)
    assign[assign == 4] = 3  # cluster 4 is empty
    perm, off = svg2.permutation(assign, 6)
    assert sorted(perm.tolist()) == list(range(100))
    counts = collections.Counter(assign.tolist())
    assert off.tolist()[0] == 0 and off[-1] == 100
    for c in range(6):
        rows = perm[off[c]:off[c + 1]].tolist()
        assert len(rows) == counts.get(c, 0)
        assert rows == sorted(i for i in range(100) if assign[i] == c)


def test_shares_equal_the_attention_mass_of_constant_clusters():
    # keys that are exact copies of a few vectors: the centroid of a cluster
    # is its key, so the estimated share is the true softmax mass, computed
    # here by the dense attention oracle with one-hot values
    rng = _rng(6)
    D, n = 8, 23
    protos = rng.standard_normal((5, D))
    cid = np.array([c % 5 for c in range(n)])
    cid[[3, 9]] = 0  # uneven cluster sizes
    k = protos[cid]
    v = np.eye(D)[cid]
    q = rng.standard_normal(D)
    o, _ = oracle.attn(q[None, None, None, :], k[None, None], v[None, None], n, 0, n)
    counts = np.bincount(cid, minlength=5)
    w = svg2.shares(q, protos, counts, 1.0 / np.sqrt(D))
    np.testing.assert_allclose(w, o[0, 0, 0, :5], rtol=1e-12, atol=1e-15)


def test_top_p_extremes_and_empty_clusters():
    rng = _rng(7)
    kc = rng.standard_normal((9, 4))
    counts = np.array([5, 0, 3, 8, 1, 0, 2, 7, 4])
    qc = rng.standard_normal(4)
    live = np.flatnonzero(counts > 0)
    assert svg2.select_top_p(qc, kc, counts, 1.0, 0.5).tolist() == live.tolist()
    w = svg2.shares(qc, kc, counts, 0.5)
    assert svg2.select_top_p(qc, kc, counts, 1e-9, 0.5).tolist() == [int(np.argmax(w))]
    assert w[1] == 0 and w[5] == 0


def test_top_p_keeps_a_smallest_set_reaching_p():
    # greedy by decreasing share gives a set of the fewest clusters whose
    # shares reach p: checked against every subset
    rng = _rng(8)
    for trial in range(20):
        m = 7
        kc = rng.standard_normal((m, 3)) * 2
        counts = rng.integers(1, 9, m)
        qc = rng.standard_normal(3)
        p = float(rng.uniform(0.2, 0.95))
        w = svg2.shares(qc, kc, counts, 0.7)
        sel = svg2.select_top_p(qc, kc, counts, p, 0.7)
        assert w[sel].sum() >= p - 1e-12
        fewest = min(r for r in range(1, m + 1)
                     if any(w[list(s)].sum() >= p for s in itertools.combinations(range(m), r)))
        assert len(sel) == fewest
        # and it holds the largest shares
        rest = np.setdiff1d(np.arange(m), sel)
        assert len(rest) == 0 or w[sel].min() >= w[rest].max()


def test_key_list_concatenates_clusters_in_id_order():
    # two chunk slots of 6 rows, 2 clusters each; slot 1 starts at row 6
    slot0 = (None, np.array([1, 4, 0, 2, 3, 5]), np.array([0, 2, 6]), 0)
    slot1 = (None, np.array([5, 0, 1, 2, 3, 4]), np.array([0, 1, 6]), 6)
    assert svg2.key_list(np.array([0, 2, 3]), [slot0, slot1], 2).tolist() == \
        [1, 4, 11, 6, 7, 8, 9, 10]


@pytest.mark.parametrize("seed", [0, 1])
def test_attention_with_p_one_is_dense_attention(seed):
    # §2.A: with every key cluster selected each query attends to every
    # visible key; clustering and reordering change nothing
    rng = _rng(10 + seed)
    D, L, slots = 16, 24, 3
    q = rng.standard_normal((L, D))
    k = rng.standard_normal((slots * L, D))
    v = rng.standard_normal((slots * L, D))
    key_slots = [svg2.cluster(k[s * L:(s + 1) * L], 4, 3) + (s * L,) for s in range(slots)]
    qc, qperm, qoff = svg2.cluster(q, 5, 3)
    groups = svg2.plan(qc, qperm, qoff, key_slots, 4, 1.0, 1.0 / np.sqrt(D))
    o, lse = svg2.attn(q, k, v, groups)
    o_ref, lse_ref = oracle.attn(q[None, :, None, :], k[None, None], v[None, None], slots * L,
                                 (slots - 1) * L, L)
    np.testing.assert_allclose(o, o_ref[0, :, 0], atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref[0, 0], atol=1e-12)


def test_attention_over_a_key_subset_is_dense_attention_of_the_subset():
    rng = _rng(12)
    D = 8
    q = rng.standard_normal((10, D))
    k = rng.standard_normal((30, D))
    v = rng.standard_normal((30, D))
    rows = np.array([7, 2, 5])
    keys = np.array([3, 17, 4, 29, 11])
    o, lse = svg2.attn(q, k, v, [(rows, keys)])
    o_ref, lse_ref = oracle.attn(q[rows][None, :, None, :], k[keys][None, None],
                                 v[keys][None, None], 5, 0, 5)
    np.testing.assert_allclose(o[rows], o_ref[0, :, 0], atol=1e-12)
    np.testing.assert_allclose(lse[rows], lse_ref[0, 0], atol=1e-12)
    assert np.isnan(o[0]).all()
