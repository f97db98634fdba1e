"""GPU parity of qkv_rope_append (fused QKV projection + Causal-RoPE + cache
append) against the fp64 oracle.

Bar, per element, for the rotated Q' and K' (pair (a, b) before rotation,
S = sum_c |x_c||w_c| of each, C terms):
    |got - exact| <= ulp_bf16(exact) + 2 C 2^-24 (S_a + S_b) + 2^-22 (|a| + |b|)
i.e. one bf16 rounding, the fp32 accumulation bound of the products (bf16 x
bf16 products are exact in fp32), propagated through the rotation, and the
fp32 rotation error with the fp32 cos/sin table.  For V (no rotation):
    |got - exact| <= ulp_bf16(exact) + C 2^-24 S.
Cache rows outside [cache_pos, cache_pos + n) must be untouched.
"""
import numpy as np
import pytest
import torch

import autoregressive_video_diffusion_amd as crattn
import oracle
from gpu_helpers import bf16_ulp, dev, f64, table
from workloads import normal

pytestmark = pytest.mark.gpu


def _inputs(B, n, C, H, D, seed):
    x = normal((B, n, C), seed, torch.float32).to(torch.bfloat16)
    w = (normal((3 * H * D, C), seed + 1, torch.float32) / np.sqrt(C)).to(torch.bfloat16)
    return x, w


def _run(x, w, H, D, cap, cache_pos, t0, tok_off, gh, gw, with_q=True, fill=7.0):
    B, n, C = x.shape
    mt, mh, mw = t0 + (tok_off + n - 1) // (gh * gw) + 1, gh, gw
    tab = table(D, mt, mh, mw)
    xd, wd = x.to(dev()), w.to(dev())
    q = torch.empty(B, n, H, D, dtype=torch.bfloat16, device=dev()) if with_q else None
    kc = torch.full((B, H, cap, D), fill, dtype=torch.bfloat16, device=dev())
    vc = torch.full((B, H, cap, D), -fill, dtype=torch.bfloat16, device=dev())
    crattn.qkv_rope_append(xd, wd, q, kc, vc, cache_pos, tab, mt, mh, mw, t0, tok_off, gh, gw)
    torch.cuda.synchronize()
    return q, kc, vc


def _check(got, exact, s_abs, pre, C, rotated, what):
    """got, exact, s_abs, pre: [..., D] fp64 (pre = the projection before rotation)."""
    err = np.abs(got - exact)
    if rotated:
        pair_s = s_abs[..., 0::2] + s_abs[..., 1::2]
        pair_x = np.abs(pre[..., 0::2]) + np.abs(pre[..., 1::2])
        extra = np.repeat(2 * C * 2.0 ** -24 * pair_s + 2.0 ** -22 * pair_x, 2, axis=-1)
    else:
        extra = C * 2.0 ** -24 * s_abs
    tol = np.maximum(bf16_ulp(exact), 2.0 ** -126) + extra
    bad = err > tol
    frac1 = float((err <= bf16_ulp(exact)).mean())
    print(f"  {what}: max err {err.max():.3e}, worst {float((err / tol).max()):.2f}x bound, "
          f"{100 * frac1:.3f}% within 1 ulp", flush=True)
    assert not bad.any(), (what, int(bad.sum()), bad.size)


def _expected(x, w, H, D, t0, tok_off, gh, gw):
    xe, we = f64(x), f64(w)
    q, k, v = oracle.qkv_rope(xe, we, H, D, t0, tok_off, gh, gw)
    q0, k0, _ = oracle.qkv_project(xe, we, H, D)
    aq, ak, av = oracle.qkv_abs(xe, we, H, D)
    return (q, k, v), (q0, k0), (aq, ak, av)


@pytest.mark.parametrize("B,n,C,H,D,gh,gw,t0,cap,pos", [
    (1, 64, 128, 2, 64, 8, 8, 3, 256, 192),     # one 8x8 frame, one token tile
    (2, 200, 192, 2, 64, 10, 20, 5, 260, 40),   # ragged tokens, 3 C stages, 384 features
    (1, 330, 320, 3, 128, 11, 15, 2, 400, 64),  # 1152 features (4.5 tiles), 2 frames
])
def test_small_shapes_every_element(B, n, C, H, D, gh, gw, t0, cap, pos):
    x, w = _inputs(B, n, C, H, D, 300 + n)
    q, kc, vc = _run(x, w, H, D, cap, pos, t0, 0, gh, gw)
    (qe, ke, ve), (q0, k0), (aq, ak, av) = _expected(x, w, H, D, t0, 0, gh, gw)
    _check(f64(q), qe, aq, q0, C, True, "Q'")
    kg = f64(kc)[:, :, pos:pos + n].transpose(0, 2, 1, 3)
    vg = f64(vc)[:, :, pos:pos + n].transpose(0, 2, 1, 3)
    _check(kg, ke, ak, k0, C, True, "K'")
    _check(vg, ve, av, ve, C, False, "V")
    # every other cache row is untouched
    for c, fill in ((kc, 7.0), (vc, -7.0)):
        assert bool((c[:, :, :pos] == fill).all()) and bool((c[:, :, pos + n:] == fill).all())


def test_cache_update_without_q():
    B, n, C, H, D, gh, gw, t0, cap, pos = 1, 128, 64, 2, 64, 8, 16, 4, 128, 0
    x, w = _inputs(B, n, C, H, D, 77)
    _, kc, vc = _run(x, w, H, D, cap, pos, t0, 0, gh, gw, with_q=False)
    q1, kc1, vc1 = _run(x, w, H, D, cap, pos, t0, 0, gh, gw, with_q=True)
    assert torch.equal(kc, kc1) and torch.equal(vc, vc1)


def test_slice_equals_rows_of_whole_chunk():
    # a sequence-parallel rank's slice, projected from its global offset,
    # gives bit for bit the same rows as the whole-chunk call
    B, C, H, D, gh, gw, t0 = 1, 256, 4, 64, 12, 20, 7
    n_all, off, n = 2 * gh * gw, 170, 150
    x, w = _inputs(B, n_all, C, H, D, 91)
    q, kc, vc = _run(x, w, H, D, n_all, 0, t0, 0, gh, gw)
    qs, kcs, vcs = _run(x[:, off:off + n].contiguous(), w, H, D, n_all, off, t0, off, gh, gw)
    assert torch.equal(qs, q[:, off:off + n])
    assert torch.equal(kcs[:, :, off:off + n], kc[:, :, off:off + n])
    assert torch.equal(vcs[:, :, off:off + n], vc[:, :, off:off + n])


def test_480p_chunk_projection():
    # the 1.3B-shape chunk: 4680 tokens, C = 1536, 12 heads of 128, t0 = 18,
    # appended at slot 6 of a 7-chunk cache; every element checked
    B, n, C, H, D, gh, gw, t0 = 1, 4680, 1536, 12, 128, 30, 52, 18
    cap, pos = 7 * n, 6 * n
    x, w = _inputs(B, n, C, H, D, 4801)
    q, kc, vc = _run(x, w, H, D, cap, pos, t0, 0, gh, gw)
    (qe, ke, ve), (q0, k0), (aq, ak, av) = _expected(x, w, H, D, t0, 0, gh, gw)
    _check(f64(q), qe, aq, q0, C, True, "480P Q'")
    _check(f64(kc[:, :, pos:]).transpose(0, 2, 1, 3), ke, ak, k0, C, True, "480P K'")
    _check(f64(vc[:, :, pos:]).transpose(0, 2, 1, 3), ve, av, ve, C, False, "480P V")
    assert bool((kc[:, :, :pos] == 7.0).all()) and bool((vc[:, :, :pos] == -7.0).all())


@pytest.mark.parametrize("B,n,C", [
    (2, 3584, 256),   # 7168 tokens: 504 tiles of 256 x 256 fill two rounds of 256 CUs
    (1, 1000, 64),    # ragged token tail, one C stage
])
def test_large_token_counts_every_element(B, n, C):
    # shapes whose tile choice differs from the 480P chunk's; every element
    H, D, gh, gw, t0 = 12, 128, 28, 32, 1
    cap, pos = n + 64, 64
    x, w = _inputs(B, n, C, H, D, 5000 + n)
    q, kc, vc = _run(x, w, H, D, cap, pos, t0, 0, gh, gw)
    (qe, ke, ve), (q0, k0), (aq, ak, av) = _expected(x, w, H, D, t0, 0, gh, gw)
    _check(f64(q), qe, aq, q0, C, True, "Q'")
    _check(f64(kc[:, :, pos:]).transpose(0, 2, 1, 3), ke, ak, k0, C, True, "K'")
    _check(f64(vc[:, :, pos:]).transpose(0, 2, 1, 3), ve, av, ve, C, False, "V")
    assert bool((kc[:, :, :pos] == 7.0).all()) and bool((vc[:, :, :pos] == -7.0).all())


@pytest.mark.parametrize("B,n,C,H,D,with_q", [
    (1, 4000, 256, 23, 64, True),    # 4416 features: a ragged last feature tile
    (2, 3000, 192, 12, 128, False),  # cache update only: 3072 features, 6 C stages
])
def test_wide_tiles_every_element(B, n, C, H, D, with_q):
    # shapes whose 256 x 384 tiles fill the chip in one round while the
    # narrower tiles need two (the 480P chunk's choice too); every element
    gh, gw, t0 = 25, 40, 3
    cap, pos = n + 100, 100
    x, w = _inputs(B, n, C, H, D, 7000 + n)
    q, kc, vc = _run(x, w, H, D, cap, pos, t0, 0, gh, gw, with_q=with_q)
    (qe, ke, ve), (q0, k0), (aq, ak, av) = _expected(x, w, H, D, t0, 0, gh, gw)
    if with_q:
        _check(f64(q), qe, aq, q0, C, True, "Q'")
    _check(f64(kc[:, :, pos:pos + n]).transpose(0, 2, 1, 3), ke, ak, k0, C, True, "K'")
    _check(f64(vc[:, :, pos:pos + n]).transpose(0, 2, 1, 3), ve, av, ve, C, False, "V")
    for c, fill in ((kc, 7.0), (vc, -7.0)):
        assert bool((c[:, :, :pos] == fill).all()) and bool((c[:, :, pos + n:] == fill).all())


def test_wide_tile_table_at_its_lds_limit():
    # a 40 x 200 grid over two frames: the epilogue's table rows (2 x 22 of
    # axis t, 40 x 21 of h, 200 x 21 of w: 40.7 KB with the copies' tail) all
    # but fill the wide tile's LDS for them, each wavefront issues 40 of the
    # 159 256-byte copies, and the rows of axis w end where the table ends
    # (the copies read no entry past it); 256 x 384 tiles win the tie with
    # the narrower tiles here.  Every element.
    B, n, C, H, D, gh, gw, t0 = 1, 12000, 512, 4, 128, 40, 200, 5
    cap, pos = n + 64, 64
    x, w = _inputs(B, n, C, H, D, 7100)
    q, kc, vc = _run(x, w, H, D, cap, pos, t0, 0, gh, gw)
    (qe, ke, ve), (q0, k0), (aq, ak, av) = _expected(x, w, H, D, t0, 0, gh, gw)
    _check(f64(q), qe, aq, q0, C, True, "Q'")
    _check(f64(kc[:, :, pos:pos + n]).transpose(0, 2, 1, 3), ke, ak, k0, C, True, "K'")
    _check(f64(vc[:, :, pos:pos + n]).transpose(0, 2, 1, 3), ve, av, ve, C, False, "V")
    for c, fill in ((kc, 7.0), (vc, -7.0)):
        assert bool((c[:, :, :pos] == fill).all()) and bool((c[:, :, pos + n:] == fill).all())


def test_projection_replays_from_a_hip_graph():
    # the fused projection + rotation + append captured once and replayed:
    # every replay writes the eager call's Q' and cache rows bit for bit,
    # with eager calls between the replays
    B, n, C, H, D, gh, gw, t0, cap, pos = 1, 600, 512, 2, 128, 10, 20, 4, 1400, 500
    x, w = _inputs(B, n, C, H, D, 61)
    xd, wd = x.to(dev()), w.to(dev())
    mt, mh, mw = t0 + n // (gh * gw) + 2, gh, gw
    tab = table(D, mt, mh, mw)
    q = torch.empty(B, n, H, D, dtype=torch.bfloat16, device=dev())
    kc = torch.zeros(B, H, cap, D, dtype=torch.bfloat16, device=dev())
    vc = torch.zeros(B, H, cap, D, dtype=torch.bfloat16, device=dev())

    def call():
        crattn.qkv_rope_append(xd, wd, q, kc, vc, pos, tab, mt, mh, mw, t0, 0, gh, gw)

    call()
    torch.cuda.synchronize()
    ref = (q.clone(), kc.clone(), vc.clone())
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for t in (q, kc, vc):
            t.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, ref[0]), f"replay {rep}: q"
        assert torch.equal(kc[:, :, pos:pos + n], ref[1][:, :, pos:pos + n]), f"replay {rep}: k"
        assert torch.equal(vc[:, :, pos:pos + n], ref[2][:, :, pos:pos + n]), f"replay {rep}: v"
        # rows outside the appended range are not written
        assert (kc[:, :, :pos] == 7.0).all() and (vc[:, :, pos + n:] == 7.0).all()
        call()
        torch.cuda.synchronize()
        assert torch.equal(q, ref[0])
