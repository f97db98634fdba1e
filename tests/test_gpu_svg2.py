"""GPU parity of the semantic-permutation sparse attention path (k-means and
reordering, centroid top-p selection, attention over key lists) against the
fp64 oracle (oracle/svg2.py).

* Planted clusters (well separated): the k-means assignment is unambiguous,
  so the GPU's reorderings and offsets equal the oracle's exactly, its
  centroids are within the fp32 summation bound, and with p chosen away from
  every cut the selections and key lists are equal and the attention is
  within the bf16 attention bar (max-abs 2e-2, relative L2 5e-3).
* p = 1 on random inputs: every query attends to every visible key whatever
  the clustering, so the output is the dense oracle attention.
* Random inputs (ambiguous clusters): a float decides an integer, so the GPU
  results are checked for validity.  Assignment: each token's centroid is
  nearest within the fp32 distance bound; centroids are the fp64 means of
  the GPU's clusters within the fp32 bound; the reordering is a stable sort.
  Selection: against fp64 shares of the GPU's centroids, the kept clusters
  are the largest shares within a bound, reach p within it, and dropping the
  smallest falls short of p; the lists are exactly those clusters' rows.
  Attention: given the GPU's lists (its unique output), every compared row
  within the bf16 bar of the oracle's attention over those keys.
* Keys outside every list are never read: NaN there leaves the output
  bit-identical.
"""
import numpy as np
import pytest
import torch

import autoregressive_video_diffusion_amd as crattn
import oracle
from gpu_helpers import assert_attn_close, dev, f64
from oracle import svg2
from workloads import normal, planted_clusters

pytestmark = pytest.mark.gpu
EPS = 2.0 ** -24


def _ws(nbytes):
    return torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=dev())


def _kmeans(x_view, C, iters, init=None):
    B, H, n, D = x_view.shape
    cent = (torch.empty(B, H, C, D, dtype=torch.float32, device=dev()) if init is None
            else init.clone())
    perm = torch.empty(B, H, n, dtype=torch.int32, device=dev())
    off = torch.empty(B, H, C + 1, dtype=torch.int32, device=dev())
    ws = _ws(crattn.svg2_kmeans_workspace_bytes(B, H, n, C))
    crattn.svg2_kmeans(x_view, C, iters, init is None, cent, perm, off, ws)
    torch.cuda.synchronize()
    return cent, perm, off


def _pipeline(q, kc, vc, L, n_vis, Cq, Ck, iters, p, splits=1):
    B, Lq, H, D = q.shape
    S = kc.shape[2] // L
    kcent = torch.zeros(B, H, S, Ck, D, dtype=torch.float32, device=dev())
    kperm = torch.zeros(B, H, S, L, dtype=torch.int32, device=dev())
    koff = torch.zeros(B, H, S, Ck + 1, dtype=torch.int32, device=dev())
    ws = _ws(max(crattn.svg2_kmeans_workspace_bytes(B, H, L, Ck),
                 crattn.svg2_kmeans_workspace_bytes(B, H, Lq, Cq)))
    for s in range(n_vis):
        crattn.svg2_kmeans(kc[:, :, s * L:(s + 1) * L], Ck, iters, True, kcent[:, :, s],
                           kperm[:, :, s], koff[:, :, s], ws)
    qcent = torch.empty(B, H, Cq, D, dtype=torch.float32, device=dev())
    qperm = torch.empty(B, H, Lq, dtype=torch.int32, device=dev())
    qoff = torch.empty(B, H, Cq + 1, dtype=torch.int32, device=dev())
    crattn.svg2_kmeans(q.permute(0, 2, 1, 3), Cq, iters, True, qcent, qperm, qoff, ws)
    cap_l = -(-n_vis * L // 64) * 64
    lists = torch.full((B, H, Cq, cap_l), -7, dtype=torch.int32, device=dev())
    llen = torch.empty(B, H, Cq, dtype=torch.int32, device=dev())
    ns = crattn.svg2_n_slots(Lq, Cq)
    slots = torch.empty(B, H, ns, 4, dtype=torch.int32, device=dev())
    sel = torch.empty(B, H, Cq, n_vis * Ck, dtype=torch.int32, device=dev())
    crattn.svg2_plan(qcent, qoff, kcent, koff, kperm, n_vis, Lq, p, sel, lists, llen, slots)
    out = torch.empty_like(q)
    lse = torch.empty(B, H, Lq, dtype=torch.float32, device=dev())
    wsa = _ws(crattn.svg2_attn_workspace_bytes(B, H, Lq, D, ns, splits))
    crattn.svg2_attn(q, kc, vc, qperm, slots, lists, llen, out, lse, splits, wsa)
    torch.cuda.synchronize()
    return dict(kcent=kcent, kperm=kperm, koff=koff, qcent=qcent, qperm=qperm, qoff=qoff,
                lists=lists, llen=llen, slots=slots, sel=sel, out=out, lse=lse, wsa=wsa)


def _planted_inputs(B, H, D, L, S, Lq, Cq, Ck, seed):
    qh, _ = planted_clusters((B, H), Lq, Cq, D, seed)
    q = qh.permute(0, 2, 1, 3).contiguous().to(dev())
    kc = torch.empty(B, H, S * L, D, dtype=torch.bfloat16)
    for s in range(S):
        kc[:, :, s * L:(s + 1) * L] = planted_clusters((B, H), L, Ck, D, seed + 1 + s)[0]
    vc = normal((B, H, S * L, D), seed + 100)
    return q, kc.to(dev()), vc.to(dev())


def _check_sort(perm, off, assign, C):
    """perm/off (int arrays of one head) are the stable sort of assign."""
    exp_perm, exp_off = svg2.permutation(assign, C)
    assert (perm == exp_perm).all() and (off == exp_off).all()


# ---------------------------------------------------------------- k-means

@pytest.mark.parametrize("D,n,C,layout", [(64, 200, 7, "cache"), (128, 333, 12, "queries"),
                                          (128, 64, 1, "cache"), (64, 1000, 40, "queries")])
def test_kmeans_planted_matches_oracle(D, n, C, layout):
    B, H = 1, 3
    xh, labels = planted_clusters((B, H), n, C, D, seed=D + n)
    if layout == "queries":
        x = xh.permute(0, 2, 1, 3).contiguous().to(dev())
        view = x.permute(0, 2, 1, 3)
    else:
        cache = torch.zeros(B, H, n + 96, D, dtype=torch.bfloat16)
        cache[:, :, 32:32 + n] = xh
        cache = cache.to(dev())
        view = cache[:, :, 32:32 + n]
    cent, perm, off = _kmeans(view, C, 3)
    x64 = xh.double().numpy()
    for b in range(B):
        for h in range(H):
            c_ref, a_ref = svg2.kmeans(x64[b, h], C, 3)
            assert (a_ref == labels[b, h].numpy()).all()
            _check_sort(perm[b, h].cpu().numpy(), off[b, h].cpu().numpy(), a_ref, C)
            cnt = np.bincount(a_ref, minlength=C)[:, None]
            bound = (cnt + 2) * EPS * np.abs(x64[b, h]).max()
            assert (np.abs(f64(cent[b, h]) - c_ref) <= bound).all()


@pytest.mark.parametrize("D,warm", [(64, False), (128, False), (128, True)])
def test_kmeans_one_iteration_is_a_valid_lloyd_step(D, warm):
    # random tokens: the first assignment is against known centroids (the
    # tokens floor(c n / C), or given fp32 ones); every token must be at a
    # nearest one within the fp32 bound, and the new centroids the means
    B, H, n, C = 2, 2, 777, 19
    x = normal((B, H, n, D), 40 + D).to(dev())
    init = None
    if warm:
        init = normal((B, H, C, D), 41, torch.float32).to(dev())
    cent, perm, off = _kmeans(x, C, 1, init)
    x64 = f64(x)
    for b in range(B):
        for h in range(H):
            xs = x64[b, h]
            c0 = f64(init[b, h]) if warm else xs[[c * n // C for c in range(C)]]
            p, o = perm[b, h].cpu().numpy(), off[b, h].cpu().numpy()
            assign = np.empty(n, dtype=np.int64)
            for c in range(C):
                assert (np.diff(p[o[c]:o[c + 1]]) > 0).all()  # ascending inside a cluster
                assign[p[o[c]:o[c + 1]]] = c
            assert sorted(p.tolist()) == list(range(n)) and o[0] == 0 and o[-1] == n
            # distances up to |x|^2, exact in fp64
            e = (c0 ** 2).sum(1)[None, :] - 2.0 * xs @ c0.T
            got = e[np.arange(n), assign]
            bound = 4 * (D + 2) * EPS * (np.abs(xs) @ np.abs(c0).T + (c0 ** 2).sum(1)[None, :])
            assert (got <= e.min(1) + bound.max(1)).all()
            for c in range(C):
                m = p[o[c]:o[c + 1]]
                ref = xs[m].mean(0) if len(m) else c0[c]
                tol = (len(m) + 2) * EPS * (np.abs(xs).max() if len(m) else np.abs(c0[c]).max())
                assert (np.abs(f64(cent[b, h, c]) - ref) <= tol).all()


# ------------------------------------------------------- planted pipeline

def _choose_p(groups_fn, candidates=(0.6, 0.7, 0.8, 0.9, 0.5, 0.95)):
    """A p whose selections are stable under a 1e-4 change of p and whose
    last kept and first dropped shares differ by more than 1e-4 (so fp32
    shares cannot change the choice): the oracle's own numbers."""
    for p in candidates:
        if groups_fn(p):
            return p
    raise AssertionError("no p with clear selections")


@pytest.mark.parametrize("D,splits", [(64, 1), (128, 1), (128, 3)])
def test_planted_pipeline_matches_oracle(D, splits):
    B, H, L, S, n_vis, Lq, Cq, Ck = 1, 2, 200, 4, 3, 600, 2, 7
    q, kc, vc = _planted_inputs(B, H, D, L, S, Lq, Cq, Ck, seed=7 + D)
    kc[:, :, n_vis * L:] = float("nan")  # invisible slot: never read
    vc[:, :, n_vis * L:] = float("nan")
    q64, k64, v64 = f64(q), f64(kc), f64(vc)
    scale = 1.0 / np.sqrt(D)
    ref = []
    for b in range(B):
        for h in range(H):
            key_slots = [svg2.cluster(k64[b, h, s * L:(s + 1) * L], Ck, 3) + (s * L,)
                         for s in range(n_vis)]
            qc, qperm, qoff = svg2.cluster(q64[b, :, h], Cq, 3)
            ref.append((key_slots, qc, qperm, qoff))

    def clear(p):
        for key_slots, qc, qperm, qoff in ref:
            kcs = np.concatenate([s[0] for s in key_slots])
            cnt = np.concatenate([np.diff(s[2]) for s in key_slots])
            for i in range(Cq):
                a = svg2.select_top_p(qc[i], kcs, cnt, p - 1e-4, scale)
                c = svg2.select_top_p(qc[i], kcs, cnt, p + 1e-4, scale)
                if not np.array_equal(a, c):
                    return False
                w = np.sort(svg2.shares(qc[i], kcs, cnt, scale))[::-1]
                k = len(a)
                if k < len(w) and w[k - 1] - w[k] <= 1e-4:
                    return False
        return True

    p = _choose_p(clear)
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 3, p, splits)
    got = f64(r["out"])
    for idx, (key_slots, qc, qperm, qoff) in enumerate(ref):
        b, h = divmod(idx, H)
        assert (r["qperm"][b, h].cpu().numpy() == qperm).all()
        assert (r["qoff"][b, h].cpu().numpy() == qoff).all()
        for s in range(n_vis):
            assert (r["kperm"][b, h, s].cpu().numpy() == key_slots[s][1]).all()
            assert (r["koff"][b, h, s].cpu().numpy() == key_slots[s][2]).all()
        groups = svg2.plan(qc, qperm, qoff, key_slots, Ck, p, scale)
        assert len(groups) == Cq
        for i, (rows, keys, sel) in enumerate(groups):
            m = int(r["llen"][b, h, i])
            assert m == len(keys)
            assert (r["lists"][b, h, i, :m].cpu().numpy() == keys).all()
            s_gpu = r["sel"][b, h, i].cpu().numpy()
            assert (s_gpu[:len(sel)] == sel).all() and (s_gpu[len(sel):] == -1).all()
        o_ref, lse_ref = svg2.attn(q64[b, :, h], k64[b, h], v64[b, h], groups)
        assert_attn_close(got[b, :, h], o_ref, f"b{b} h{h}")
        np.testing.assert_allclose(f64(r["lse"][b, h]), lse_ref, atol=1e-3)


# ------------------------------------------------------------ p = 1

@pytest.mark.parametrize("D,splits", [(64, 1), (128, 1), (128, 3), (128, 16)])
def test_p_one_is_dense_attention(D, splits):
    B, H, L, n_vis, Lq, Cq, Ck = 1, 2, 520, 3, 450, 5, 6
    q = normal((B, Lq, H, D), 60).to(dev())
    kc = normal((B, H, (n_vis + 1) * L, D), 61).to(dev())
    vc = normal((B, H, (n_vis + 1) * L, D), 62).to(dev())
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 2, 1.0, splits)
    assert (r["llen"].cpu() == n_vis * L).all()
    o_ref, lse_ref = oracle.attn(f64(q), f64(kc), f64(vc), n_vis * L, (n_vis - 1) * L, L)
    assert_attn_close(f64(r["out"]), o_ref, "p = 1")
    np.testing.assert_allclose(f64(r["lse"]), lse_ref, atol=1e-3)


# ---------------------------------------------------- random validity

def _check_selection(r, b, h, n_vis, Ck, L, p, scale):
    qc = f64(r["qcent"][b, h])
    kc = f64(r["kcent"][b, h, :n_vis]).reshape(n_vis * Ck, -1)
    koff = r["koff"][b, h, :n_vis].cpu().numpy()
    kperm = r["kperm"][b, h, :n_vis].cpu().numpy()
    cnt = np.diff(koff, axis=1).reshape(-1)
    qoff = r["qoff"][b, h].cpu().numpy()
    for i in range(len(qoff) - 1):
        m = int(r["llen"][b, h, i])
        sel = r["sel"][b, h, i].cpu().numpy()
        if qoff[i + 1] == qoff[i]:
            assert m == 0 and (sel == -1).all()
            continue
        k = int((sel >= 0).sum())
        kept = sel[:k]
        assert k >= 1 and (sel[k:] == -1).all() and (np.diff(kept) > 0).all()
        assert (cnt[kept] > 0).all()
        w = svg2.shares(qc[i], kc, cnt, scale)
        tol = 1e-5
        dropped = np.setdiff1d(np.flatnonzero(cnt > 0), kept)
        if len(dropped):
            assert w[kept].min() >= w[dropped].max() - tol
            assert w[kept].sum() >= p - tol
        assert w[kept].sum() - w[kept].min() < p + tol
        # the list: the kept clusters' rows, cluster by cluster
        keys = np.concatenate([s * L + kperm[s, koff[s, c]:koff[s, c + 1]]
                               for s, c in (divmod(int(j), Ck) for j in kept)])
        assert m == len(keys) and (r["lists"][b, h, i, :m].cpu().numpy() == keys).all()


def _check_slots(r, b, h, Lq):
    sl = r["slots"][b, h].cpu().numpy()
    qoff = r["qoff"][b, h].cpu().numpy()
    used = sl[sl[:, 1] > 0]
    assert (used[:, 1] <= 256).all()
    covered = np.concatenate([np.arange(s, s + n) for s, n, _, _ in used])
    assert (np.sort(covered) == np.arange(Lq)).all()
    for s, n, c, _ in used:
        assert qoff[c] <= s and s + n <= qoff[c + 1]


@pytest.mark.parametrize("D,p,splits", [(64, 0.5, 1), (128, 0.8, 2), (128, 0.3, 1)])
def test_random_selection_valid_and_attention_over_lists(D, p, splits):
    B, H, L, n_vis, Lq, Cq, Ck = 2, 2, 300, 3, 300, 4, 9
    q = normal((B, Lq, H, D), 70).to(dev())
    kc = normal((B, H, n_vis * L, D), 71).to(dev())
    vc = normal((B, H, n_vis * L, D), 72).to(dev())
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 2, p, splits)
    q64, k64, v64, got = f64(q), f64(kc), f64(vc), f64(r["out"])
    for b in range(B):
        for h in range(H):
            _check_selection(r, b, h, n_vis, Ck, L, p, 1.0 / np.sqrt(D))
            _check_slots(r, b, h, Lq)
            qperm, qoff = r["qperm"][b, h].cpu().numpy(), r["qoff"][b, h].cpu().numpy()
            groups = [(qperm[qoff[i]:qoff[i + 1]],
                       r["lists"][b, h, i, :int(r["llen"][b, h, i])].cpu().numpy().astype(np.int64))
                      for i in range(Cq) if qoff[i + 1] > qoff[i]]
            o_ref, lse_ref = svg2.attn(q64[b, :, h], k64[b, h], v64[b, h], groups)
            assert_attn_close(got[b, :, h], o_ref, f"b{b} h{h}")
            np.testing.assert_allclose(f64(r["lse"][b, h]), lse_ref, atol=1e-3)


def test_keys_outside_the_lists_are_never_read():
    B, H, L, n_vis, Lq, Cq, Ck, D = 1, 2, 256, 2, 200, 3, 8, 128
    q = normal((B, Lq, H, D), 80).to(dev())
    kc = normal((B, H, n_vis * L, D), 81).to(dev())
    vc = normal((B, H, n_vis * L, D), 82).to(dev())
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 2, 0.4)
    used = torch.zeros(B, H, n_vis * L, dtype=torch.bool)
    for h in range(H):
        for i in range(Cq):
            used[0, h, r["lists"][0, h, i, :int(r["llen"][0, h, i])].long().cpu()] = True
    assert (~used).any()
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[~used.to(dev())] = float("nan")
    vc2[~used.to(dev())] = float("nan")
    out2 = torch.empty_like(q)
    crattn.svg2_attn(q, kc2, vc2, r["qperm"], r["slots"], r["lists"], r["llen"], out2,
                     workspace=r["wsa"])
    torch.cuda.synchronize()
    assert torch.equal(out2, r["out"])


# ------------------------------------------------------------ 480P

def test_480p_chunk_pipeline_sampled():
    # one 480P denoising call: 4680 queries, 7 visible chunk slots of 4680
    # keys (32760), 12 heads; 20 query and 64 key clusters per slot
    B, H, D, L, n_vis, Cq, Ck, p = 1, 12, 128, 4680, 7, 20, 64, 0.9
    q = normal((B, L, H, D), 90).to(dev())
    kc = normal((B, H, n_vis * L, D), 91).to(dev())
    vc = normal((B, H, n_vis * L, D), 92).to(dev())
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 3, p, splits=4)
    assert torch.isfinite(r["out"].float()).all()
    for h in (0, 11):
        _check_selection(r, 0, h, n_vis, Ck, L, p, 1.0 / np.sqrt(D))
        _check_slots(r, 0, h, L)
    rng = np.random.default_rng(5)
    q64, got = f64(q), f64(r["out"])
    for h in (0, 5, 11):
        qperm, qoff = r["qperm"][0, h].cpu().numpy(), r["qoff"][0, h].cpu().numpy()
        k64, v64 = f64(kc[0, h]), f64(vc[0, h])
        groups = []
        for i in rng.choice(Cq, 3, replace=False):
            rows = qperm[qoff[i]:qoff[i + 1]]
            if len(rows) == 0:
                continue
            rows = rng.choice(rows, min(8, len(rows)), replace=False)
            keys = r["lists"][0, h, i, :int(r["llen"][0, h, i])].cpu().numpy().astype(np.int64)
            groups.append((rows, keys))
        o_ref, _ = svg2.attn(q64[0, :, h], k64, v64, groups)
        rows = np.concatenate([g[0] for g in groups])
        assert_attn_close(got[0, rows, h], o_ref[rows], f"480P h{h}")


# ------------------------------------------------------------ rollout

@pytest.mark.parametrize("p", [0.7, 1.0])
def test_rollout_with_svg2_through_a_full_ring(p):
    # six one-frame chunks (8x8) through a ring of 4 slots; every denoising
    # call is checked against the oracle over the rollout's own lists, and
    # with p = 1 against the dense attention of the visible cache
    from autoregressive_video_diffusion_amd.rollout import ChunkRollout

    B, H, D, gh, gw = 1, 2, 64, 8, 8
    ro = ChunkRollout(B, H, D, 1, gh, gw, window=4, max_chunks=7, device=dev(),
                      svg2=(3, 4, p))
    L = ro.L
    for c in range(6):
        for step in range(2):
            q = normal((B, L, H, D), 800 + 5 * c + step).to(dev())
            k = normal((B, L, H, D), 820 + 5 * c + step).to(dev())
            v = normal((B, L, H, D), 840 + 5 * c + step).to(dev())
            q_out, out = torch.empty_like(q), torch.empty_like(q)
            ro.denoise(c, q, k, v, q_out, out)
            torch.cuda.synchronize()
            n_vis = min(c + 1, 4)
            q64, k64, v64 = f64(q_out), f64(ro.k_cache), f64(ro.v_cache)
            for h in range(H):
                qperm, qoff = ro.qperm[0, h].cpu().numpy(), ro.qoff[0, h].cpu().numpy()
                groups = []
                for i in range(3):
                    if qoff[i + 1] > qoff[i]:
                        keys = ro.lists[0, h, i, :int(ro.llen[0, h, i])].cpu().numpy()
                        assert (keys >= 0).all() and (keys < n_vis * L).all()
                        if p == 1.0:
                            assert len(keys) == n_vis * L
                        groups.append((qperm[qoff[i]:qoff[i + 1]], keys.astype(np.int64)))
                o_ref, _ = svg2.attn(q64[0, :, h], k64[0, h], v64[0, h], groups)
                assert_attn_close(f64(out[0, :, h]), o_ref, f"svg2 rollout c{c} s{step} h{h}")
            if p == 1.0:
                kv_len, q0 = ro.visible(c)
                o_d, _ = oracle.attn(q64, k64, v64, kv_len, q0, L)
                assert_attn_close(f64(out), o_d, f"svg2 rollout p=1 c{c}")
        ro.update(c, k, v)
    with pytest.raises(NotImplementedError):
        q = normal((B, L // 2, H, D), 900).to(dev())
        ro.denoise(6, q, q, q, torch.empty_like(q), torch.empty_like(q), tok_off=L // 2)


def test_720p_window_pipeline_sampled():
    # the 720P window: 40 heads, 10800 queries (40 clusters) against a full
    # ring of 7 slots of 10800 keys (64 clusters each, 448 candidates),
    # clustered inputs; selections checked for validity on two heads, the
    # attention on sampled rows of three
    from workloads import WIN720, clustered_qk

    w = WIN720
    Cq, Ck, p, L, n_vis = 40, 64, 0.9, w.chunk_tokens, w.cap // w.chunk_tokens
    q, kc = clustered_qk(w, n_qc=Cq, n_kc=Ck)
    q, kc = q.to(dev()), kc.to(dev())
    vc = normal((w.B, w.H, w.cap, w.D), 95).to(dev())
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 2, p, splits=2)
    assert torch.isfinite(r["out"].float()).all()
    dens = float(r["llen"].double().mean()) / (n_vis * L)
    print(f"  720P mean list density {dens:.3f}")
    for h in (0, 39):
        _check_selection(r, 0, h, n_vis, Ck, L, p, 1.0 / np.sqrt(w.D))
        _check_slots(r, 0, h, L)
    rng = np.random.default_rng(7)
    q64, got = f64(q), f64(r["out"])
    for h in (3, 20, 38):
        qperm, qoff = r["qperm"][0, h].cpu().numpy(), r["qoff"][0, h].cpu().numpy()
        k64, v64 = f64(kc[0, h]), f64(vc[0, h])
        groups = []
        for i in rng.choice(Cq, 3, replace=False):
            rows = qperm[qoff[i]:qoff[i + 1]]
            if len(rows) == 0:
                continue
            rows = rng.choice(rows, min(6, len(rows)), replace=False)
            keys = r["lists"][0, h, i, :int(r["llen"][0, h, i])].cpu().numpy().astype(np.int64)
            groups.append((rows, keys))
        o_ref, _ = svg2.attn(q64[0, :, h], k64, v64, groups)
        rows = np.concatenate([g[0] for g in groups])
        assert_attn_close(got[0, rows, h], o_ref[rows], f"720P h{h}")


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("n,C,D", [(10, 16, 64), (1, 3, 128), (57, 1, 128), (200, 200, 64)])
def test_kmeans_degenerate_sizes(n, C, D):
    # more clusters than tokens (duplicate starting centroids: the lower index
    # takes the ties, the rest stay empty and keep their centroid), a single
    # token, a single cluster, one token per cluster
    B, H = 1, 2
    x = normal((B, H, n, D), 300 + n + C).to(dev())
    cent, perm, off = _kmeans(x, C, 2)
    x64 = f64(x)
    for h in range(H):
        p, o = perm[0, h].cpu().numpy(), off[0, h].cpu().numpy()
        assert sorted(p.tolist()) == list(range(n)) and o[0] == 0 and o[-1] == n
        assert (np.diff(o) >= 0).all()
        for c in range(C):
            m = p[o[c]:o[c + 1]]
            assert (np.diff(m) > 0).all()
            if len(m):
                tol = (len(m) + 2) * EPS * np.abs(x64[0, h]).max()
                assert (np.abs(f64(cent[0, h, c]) - x64[0, h][m].mean(0)) <= tol).all()
        if C == 1:
            np.testing.assert_allclose(f64(cent[0, h, 0]), x64[0, h].mean(0), atol=1e-5)


def test_kmeans_largest_sizes():
    # 16384 tokens, 256 clusters (the LDS-staged maximum of both kernels):
    # one Lloyd step is valid against its known starting centroids
    B, H, n, C, D = 1, 2, 16384, 256, 128
    x = normal((B, H, n, D), 310).to(dev())
    cent, perm, off = _kmeans(x, C, 1)
    x64 = f64(x)
    for h in range(H):
        xs = x64[0, h]
        c0 = xs[[c * n // C for c in range(C)]]
        p, o = perm[0, h].cpu().numpy(), off[0, h].cpu().numpy()
        assert sorted(p.tolist()) == list(range(n))
        assign = np.empty(n, dtype=np.int64)
        for c in range(C):
            assert (np.diff(p[o[c]:o[c + 1]]) > 0).all()
            assign[p[o[c]:o[c + 1]]] = c
        e = (c0 ** 2).sum(1)[None, :] - 2.0 * xs @ c0.T
        bound = 4 * (D + 2) * EPS * (np.abs(xs) @ np.abs(c0).T + (c0 ** 2).sum(1)[None, :])
        assert (e[np.arange(n), assign] <= e.min(1) + bound.max(1)).all()


@pytest.mark.parametrize("Cq,Ck,n_vis,p", [(1, 256, 4, 0.9), (5, 8, 3, 1e-6), (3, 64, 2, 0.999)])
def test_plan_extremes(Cq, Ck, n_vis, p):
    # one query cluster with 1024 candidates (the maximum), a p so small that
    # one key cluster is kept per query cluster, and a p just below 1
    B, H, L, D = 1, 2, 320, 64
    Lq = 200
    q = normal((B, Lq, H, D), 320).to(dev())
    kc = normal((B, H, n_vis * L, D), 321).to(dev())
    vc = normal((B, H, n_vis * L, D), 322).to(dev())
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 2, p)
    for h in range(H):
        _check_selection(r, 0, h, n_vis, Ck, L, p, 1.0 / np.sqrt(D))
        _check_slots(r, 0, h, Lq)
        if p < 1e-3:
            assert ((r["sel"][0, h] >= 0).sum(-1).cpu() <= 1).all()
    q64, k64, v64, got = f64(q), f64(kc), f64(vc), f64(r["out"])
    for h in range(H):
        qperm, qoff = r["qperm"][0, h].cpu().numpy(), r["qoff"][0, h].cpu().numpy()
        groups = [(qperm[qoff[i]:qoff[i + 1]],
                   r["lists"][0, h, i, :int(r["llen"][0, h, i])].cpu().numpy().astype(np.int64))
                  for i in range(Cq) if qoff[i + 1] > qoff[i]]
        o_ref, _ = svg2.attn(q64[0, :, h], k64[0, h], v64[0, h], groups)
        assert_attn_close(got[0, :, h], o_ref, f"plan extremes h{h}")


def test_svg2_call_replays_from_a_hip_graph():
    # the whole denoising call (k-means of the own slot's keys and of the
    # queries on two streams, plan, attention) captured once and replayed:
    # each replay, started from the same centroids as an eager call, gives
    # the eager call's output bit for bit (no memset nodes: the kernels
    # clear their own counters)
    B, H, D, L, n_vis, Cq, Ck, p = 1, 2, 128, 320, 3, 4, 8, 0.6
    q = normal((B, L, H, D), 330).to(dev())
    kc = normal((B, H, n_vis * L, D), 331).to(dev())
    vc = normal((B, H, n_vis * L, D), 332).to(dev())
    r = _pipeline(q, kc, vc, L, n_vis, Cq, Ck, 2, p, splits=2)
    kcent, kperm, koff = r["kcent"], r["kperm"], r["koff"]
    qcent, qperm, qoff = r["qcent"], r["qperm"], r["qoff"]
    own = n_vis - 1
    ws_k = _ws(max(crattn.svg2_kmeans_workspace_bytes(B, H, L, Ck),
                   crattn.svg2_kmeans_workspace_bytes(B, H, L, Cq)))
    ws_q = _ws(crattn.svg2_kmeans_workspace_bytes(B, H, L, Cq))
    ks = kc[:, :, own * L:(own + 1) * L]
    out = torch.empty_like(q)
    side = torch.cuda.Stream(device=dev())

    def call():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        crattn.svg2_kmeans(q.permute(0, 2, 1, 3), Cq, 1, False, qcent, qperm, qoff, ws_q,
                           stream=side)
        crattn.svg2_kmeans(ks, Ck, 1, False, kcent[:, :, own], kperm[:, :, own],
                           koff[:, :, own], ws_k)
        main.wait_stream(side)
        crattn.svg2_plan(qcent, qoff, kcent, koff, kperm, n_vis, L, p, r["sel"], r["lists"],
                         r["llen"], r["slots"])
        crattn.svg2_attn(q, kc, vc, qperm, r["slots"], r["lists"], r["llen"], out, None, 2,
                         r["wsa"])

    state = [t.clone() for t in (kcent, qcent)]

    def restore():
        kcent.copy_(state[0])
        qcent.copy_(state[1])

    restore()
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out.zero_()
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        # eager work between the replays
        restore()
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


@pytest.mark.parametrize("D,from_tokens", [(128, True), (128, False), (64, True)])
def test_kmeans2_equals_two_single_calls(D, from_tokens):
    """svg2_kmeans2 launches both problems together (one chunk slot's keys,
    64 clusters, and the queries, 20 clusters, of different lengths); each
    result equals svg2_kmeans on that problem alone, bit for bit."""
    B, H = 1, 3
    kc = normal((B, H, 3000, D), 11).to(dev())
    q = normal((B, 777, H, D), 12).to(dev())
    probs = [(kc[:, :, 1000:2000], 64), (q.permute(0, 2, 1, 3), 20)]
    init = [normal((B, H, C, D), 13 + i, torch.float32).to(dev())
            for i, (_, C) in enumerate(probs)]
    outs = []
    for fused in (False, True):
        bufs = []
        for (x, C), c0 in zip(probs, init):
            n = x.shape[2]
            perm = torch.full((B, H, n), -7, dtype=torch.int32, device=dev())
            off = torch.full((B, H, C + 1), -7, dtype=torch.int32, device=dev())
            ws = _ws(crattn.svg2_kmeans_workspace_bytes(B, H, n, C))
            bufs.append((x, C, c0.clone(), perm, off, ws))
        if fused:
            crattn.svg2_kmeans2(bufs[0], bufs[1], 2, from_tokens)
        else:
            for b in bufs:
                crattn.svg2_kmeans(b[0], b[1], 2, from_tokens, *b[2:])
        torch.cuda.synchronize()
        outs.append([(b[2].cpu(), b[3].cpu(), b[4].cpu()) for b in bufs])
    for single, pair in zip(outs[0], outs[1]):
        for u, v in zip(single, pair):
            assert torch.equal(u, v)
    # the clusterings are real ones: offsets end at n, perm is a permutation
    for (x, C), (_, perm, off) in zip(probs, outs[1]):
        n = x.shape[2]
        assert int(off[..., -1].min()) == n == int(off[..., -1].max())
        assert torch.equal(perm.sort(dim=-1).values,
                           torch.arange(n, dtype=torch.int32).expand(B, H, n))
