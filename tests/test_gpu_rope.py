"""GPU parity of rope_precompute and rope_apply_append against the oracle.

fp32: within 1e-5 absolute; bf16: within one bf16 ulp of the exact (fp64)
rotation; V copied bit for bit; cache rows outside the appended range
untouched; a slice rotated from its global offsets equals the same rows of
the whole chunk, bit for bit.
"""
import numpy as np
import pytest
import torch

import autoregressive_video_diffusion_amd as crattn
import oracle
from gpu_helpers import ROPE_F32_ABS, assert_rope_bf16, dev, f64, table
from workloads import SP480, STEP480, TINY, WIN720, call_qkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,ext", [(64, (4, 8, 8)), (128, (21, 30, 52)), (128, (84, 45, 80)),
                                   (128, (2000, 3, 7))])
def test_table_within_one_fp32_ulp(D, ext):
    t = table(D, *ext)
    torch.cuda.synchronize()
    got = t.cpu().numpy().reshape(-1, 2).astype(np.float64)
    c, s = oracle.rope_table(D, *ext)
    for col, ref in ((0, c), (1, s)):
        ref32 = ref.astype(np.float32).astype(np.float64)
        err = np.abs(got[:, col] - ref32)
        assert (err <= np.spacing(np.abs(ref).astype(np.float32))).all()
        assert (err == 0).mean() > 0.99


def _caches(B, H, cap, D, dtype, fill=-3.0):
    kc = torch.full((B, H, cap, D), fill, dtype=dtype, device=dev())
    vc = torch.full((B, H, cap, D), fill, dtype=dtype, device=dev())
    return kc, vc


def _run(w, q, k, v, cap, cache_pos, n=None, tok_off=None, q_none=False, inplace=False):
    n = w.lq if n is None else n
    tok_off = w.tok_off if tok_off is None else tok_off
    mt, mh, mw = w.table_extents()
    tab = table(w.D, mt, mh, mw, w.theta)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    kc, vc = _caches(w.B, w.H, cap, w.D, k.dtype)
    if q_none:
        q_out = None
        qd = None
    elif inplace:
        q_out = qd
    else:
        q_out = torch.empty_like(qd)
    crattn.rope_apply_append(qd, q_out, kd, vd, kc, vc, cache_pos, tab, mt, mh, mw, w.t0, tok_off,
                             w.grid_h, w.grid_w)
    torch.cuda.synchronize()
    return q_out, kc, vc


def _check_cache(w, k, v, kc, vc, cache_pos, n, tok_off, bf16):
    k_ref = oracle.rope(f64(k), w.t0, tok_off, w.grid_h, w.grid_w, w.theta)
    got_k = f64(kc[:, :, cache_pos:cache_pos + n]).transpose(0, 2, 1, 3)
    if bf16:
        assert_rope_bf16(got_k, k_ref, f64(k))
    else:
        assert np.abs(got_k - k_ref).max() <= ROPE_F32_ABS
    np.testing.assert_array_equal(f64(vc[:, :, cache_pos:cache_pos + n]).transpose(0, 2, 1, 3),
                                  f64(v))
    # nothing outside the appended rows changed (checked on the device)
    for arr in (kc, vc):
        assert int((arr[:, :, :cache_pos] != -3.0).sum()) == 0
        assert int((arr[:, :, cache_pos + n:] != -3.0).sum()) == 0


def test_tiny_fp32_rope_append():
    w = TINY
    q, k, v = call_qkv(w, 0)
    q_out, kc, vc = _run(w, q, k, v, w.cap, w.cache_pos)
    q_ref = oracle.rope(f64(q), w.t0, w.tok_off, w.grid_h, w.grid_w, w.theta)
    err = np.abs(f64(q_out) - q_ref).max()
    print(f"  tiny fp32 rope max-abs {err:.2e}", flush=True)
    assert err <= ROPE_F32_ABS
    _check_cache(w, k, v, kc, vc, w.cache_pos, w.lq, w.tok_off, bf16=False)


def test_identity_at_origin_bitwise():
    w = TINY
    q, k, v = call_qkv(w, 5)
    import dataclasses

    w0 = dataclasses.replace(w, t0=0)
    q_out, kc, _ = _run(w0, q, k, v, w.cap, 0)
    np.testing.assert_array_equal(f64(q_out)[:, 0], f64(q)[:, 0])
    np.testing.assert_array_equal(f64(kc)[:, :, 0], f64(k)[:, 0])


def test_step480_bf16_rope_append():
    w = STEP480
    q, k, v = call_qkv(w, 0)
    q_out, kc, vc = _run(w, q, k, v, w.cap, w.cache_pos)
    q_ref = oracle.rope(f64(q), w.t0, w.tok_off, w.grid_h, w.grid_w, w.theta)
    assert_rope_bf16(f64(q_out), q_ref, f64(q))
    exact = (f64(q_out) == oracle.round_bf16(q_ref)).mean()
    print(f"  480P bf16 rope: {exact:.5f} equal to RNE of the exact value", flush=True)
    assert exact > 0.99
    _check_cache(w, k, v, kc, vc, w.cache_pos, w.lq, w.tok_off, bf16=True)


def test_sp_slice_equals_rows_of_whole_chunk_bitwise():
    w = STEP480
    q, k, v = call_qkv(w, 3)
    q_full, kc_full, vc_full = _run(w, q, k, v, w.cap, w.cache_pos)
    s = SP480
    sl = slice(s.tok_off, s.tok_off + s.lq)
    q_sl, kc_sl, vc_sl = _run(s, q[:, sl].contiguous(), k[:, sl].contiguous(),
                              v[:, sl].contiguous(), s.cap, s.cache_pos)
    assert torch.equal(q_sl, q_full[:, sl])
    rows = slice(s.cache_pos, s.cache_pos + s.lq)
    assert torch.equal(kc_sl[:, :, rows], kc_full[:, :, rows])
    assert torch.equal(vc_sl[:, :, rows], vc_full[:, :, rows])
    # and against the oracle at the slice's global positions
    q_ref = oracle.rope(f64(q[:, sl]), s.t0, s.tok_off, s.grid_h, s.grid_w, s.theta)
    assert_rope_bf16(f64(q_sl), q_ref, f64(q[:, sl]))


def test_cache_update_without_q_and_in_place_q():
    w = STEP480
    q, k, v = call_qkv(w, 4)
    _, kc, vc = _run(w, q, k, v, w.cap, w.cache_pos, q_none=True)
    _check_cache(w, k, v, kc, vc, w.cache_pos, w.lq, w.tok_off, bf16=True)
    q_in, _, _ = _run(w, q, k, v, w.cap, w.cache_pos, inplace=True)
    q_ref, _, _ = _run(w, q, k, v, w.cap, w.cache_pos)
    assert torch.equal(q_in, q_ref)


def test_batch2_ragged_grid_fp32_and_bf16():
    import dataclasses

    for dt in ("f32", "bf16"):
        w = dataclasses.replace(TINY, B=2, H=3, D=128, frames=2, grid_h=5, grid_w=7, t0=9,
                                lq=53, tok_off=11, dtype=dt)
        q, k, v = call_qkv(w, 7)
        cap, pos = 200, 77
        q_out, kc, vc = _run(w, q, k, v, cap, pos)
        q_ref = oracle.rope(f64(q), w.t0, w.tok_off, w.grid_h, w.grid_w, w.theta)
        if dt == "f32":
            assert np.abs(f64(q_out) - q_ref).max() <= ROPE_F32_ABS
        else:
            assert_rope_bf16(f64(q_out), q_ref, f64(q))
        _check_cache(w, k, v, kc, vc, pos, w.lq, w.tok_off, bf16=(dt == "bf16"))


def test_large_odd_divisors_bf16():
    # the pass finds a vector's row, head, batch, frame and grid row by
    # dividing by constants of the call (multiply-high division): a 37 x 199
    # grid, 9973 tokens from token 4999 (so frames 0..2), 5 heads, 3 batches,
    # head_dim 64 (8 vectors a row) checks them away from small powers of two
    import dataclasses

    w = dataclasses.replace(TINY, B=3, H=5, D=64, frames=3, grid_h=37, grid_w=199, t0=2,
                            lq=9973, tok_off=4999, dtype="bf16")
    q, k, v = call_qkv(w, 11)
    cap, pos = w.lq + 50, 31
    q_out, kc, vc = _run(w, q, k, v, cap, pos)
    q_ref = oracle.rope(f64(q), w.t0, w.tok_off, w.grid_h, w.grid_w, w.theta)
    assert_rope_bf16(f64(q_out), q_ref, f64(q))
    _check_cache(w, k, v, kc, vc, pos, w.lq, w.tok_off, bf16=True)


def test_win720_beyond_training_length():
    w = WIN720
    q, k, v = call_qkv(w, 0, n=1200)   # first 1200 tokens of the t0 = 81 chunk
    q_out, kc, vc = _run(w, q, k, v, w.cap, w.cache_pos, n=1200)
    q_ref = oracle.rope(f64(q), w.t0, 0, w.grid_h, w.grid_w, w.theta)
    assert_rope_bf16(f64(q_out), q_ref, f64(q))
    _check_cache(w, k, v, kc, vc, w.cache_pos, 1200, 0, bf16=True)


def test_fp32_large_time_index_accuracy():
    import dataclasses

    w = dataclasses.replace(TINY, t0=1900, H=1, lq=64)
    q, k, v = call_qkv(w, 8)
    q = q * 4.0
    q_out, _, _ = _run(w, q, k, v, 64, 0)
    q_ref = oracle.rope(f64(q), w.t0, 0, w.grid_h, w.grid_w, w.theta)
    err = np.abs(f64(q_out) - q_ref).max()
    print(f"  fp32 rope at t=1900, |x|<=~16: max-abs {err:.2e}", flush=True)
    assert err <= ROPE_F32_ABS
