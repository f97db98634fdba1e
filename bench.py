"""Benchmark of the chunk-causal Causal-RoPE attention step on one MI355X.

One step = the whole hot path for one denoising call of a 480P Wan-1.3B-shape
chunk: rope_apply_append (rotate Q and K of the 4680-token chunk at global
time index 18, write Q', append K' and V to cache slot 6) followed by
chunk_causal_attn (4680 queries x 32760 keys, 12 heads, head_dim 128, bf16).
The cos/sin table is built once before timing, as the method prescribes
(precomputed contiguous tables).

Inputs are synthetic N(0, 1) bf16 (seeded), resident in HBM before timing.
Eight complete buffer sets (inputs, outputs and KV cache, 273 MB each) are
used round-robin: between two uses of one set the others move ~600 MB through
HBM (the RoPE/append bursts alone, 86 MB per launch, move 7 x 86 MB), more
than the 256 MB Infinity Cache, so no launch finds its data there.  Before
the warm-up steps 64 untimed steps let the clock settle (it ramps over the
first ~30 ms of matrix work); the line records both counts.

Prints ONE JSON line.  Per-kernel times come from HIP events recorded on the
stream the library launches on (torch's current stream).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "chunk-causal attn TFLOP/s + ms/chunk (480P, 1.3B shape); % of bf16 MFMA peak"
COUNTERS = os.path.join(ROOT, "profiles", "attn_step480_hbm_counters.txt")
_CSRC = os.path.join(ROOT, "autoregressive_video_diffusion_amd", "csrc")
# the attention's device code: the kernel, its generated key loop, the planner
ATTN_SRC = tuple(os.path.join(_CSRC, f) for f in ("attn.hip", "attn_loop.inc", "plan.cpp"))


def attn_flops(B, H, Lq, visible_keys, D):
    """4*B*H*Lq*keys*D: two products (QK^T and PV), 2 flops per multiply-add.
    Masked pairs are not counted; softmax is not counted."""
    return 4 * B * H * Lq * visible_keys * D


def rope_bytes(B, n, H, D, elt=2, with_q=True):
    """Algorithmic HBM bytes of one fused RoPE/append call: read Q, K, V and
    write Q', K', V (6 tensors of B*n*H*D) -- 4 tensors without Q."""
    return (6 if with_q else 4) * B * n * H * D * elt


ROPE_SRC = os.path.join(ROOT, "autoregressive_video_diffusion_amd", "csrc", "rope.hip")
QKV_SRC = os.path.join(ROOT, "autoregressive_video_diffusion_amd", "csrc", "qkv.hip")


def qkv_flops(B, n, C, H, D):
    """2*B*n*C*3HD: the projection's multiply-adds (the rotation is not counted)."""
    return 2 * B * n * C * 3 * H * D


def qkv_bytes(B, n, C, H, D, elt=2):
    """Algorithmic HBM bytes of one fused projection call: read x and W, write
    Q', K', V (the cos/sin table, a few hundred KB, is not counted)."""
    return (B * n * C + 3 * H * D * C + 3 * B * n * H * D) * elt


def source_digest(path=ATTN_SRC) -> str:
    """sha256 (first 16 hex digits) of a source file, or of several in order."""
    h = hashlib.sha256()
    for p in (path,) if isinstance(path, str) else path:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel="attn"):
    """HBM bytes per launch of the attention ("attn"), RoPE/append ("rope") or
    fused projection ("qkv") kernel from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    for line in open(COUNTERS):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    src, key = {"attn": (ATTN_SRC, "traffic_bytes_per_launch"),
                "rope": (ROPE_SRC, "rope_traffic_bytes_per_launch"),
                "qkv": (QKV_SRC, "qkv_traffic_bytes_per_launch")}[kernel]
    if kv.get(f"{kernel}_source_sha256_16") != source_digest(src):
        return None
    try:
        return int(float(kv[key]))
    except (KeyError, ValueError):
        return None


_PRIOR = {}


class StepBuffers:
    def __init__(self, w, dev, seed_base):
        import torch

        from workloads import call_qkv, prior_cache

        q, k, v = call_qkv(w, seed_base)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        if w.name not in _PRIOR:   # the same prior cache contents in every set
            _PRIOR[w.name] = prior_cache(w)
        kc, vc = _PRIOR[w.name]
        self.kc, self.vc = kc.to(dev), vc.to(dev)
        self.q_out = torch.empty_like(self.q)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(w.B, w.H, w.lq, dtype=torch.float32, device=dev)


def make_table(w, dev):
    import torch

    import autoregressive_video_diffusion_amd as crattn

    mt, mh, mw = w.table_extents()
    t = torch.empty(crattn.rope_table_bytes(w.D, mt, mh, mw) // 4, dtype=torch.float32, device=dev)
    crattn.rope_precompute(t, w.D, mt, mh, mw, w.theta)
    return t, (mt, mh, mw)


def run_step(crattn, w, b, table, ext, ws):
    mt, mh, mw = ext
    crattn.rope_apply_append(b.q, b.q_out, b.k, b.v, b.kc, b.vc, w.cache_pos, table, mt, mh, mw,
                             w.t0, w.tok_off, w.grid_h, w.grid_w)
    crattn.chunk_causal_attn(b.q_out, b.kc, b.vc, w.kv_len, w.q_pos0, w.chunk_tokens, b.out,
                             b.lse, ws)


def time_attn_only(crattn, w, dev, reps=5):
    """Average attention time (ms) of one workload, events on the stream."""
    import torch

    from workloads import normal, prior_cache

    q = normal((w.B, w.lq, w.H, w.D), 1000 * w.index).to(dev)
    kc, vc = prior_cache(w)
    kc, vc = kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    wsb = crattn.chunk_causal_attn_workspace_bytes(w.B, w.H, w.lq, w.kv_len, w.q_pos0,
                                                   w.chunk_tokens, w.D)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=dev) if wsb else None
    for _ in range(2):
        crattn.chunk_causal_attn(q, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens, out, None, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        crattn.chunk_causal_attn(q, kc, vc, w.kv_len, w.q_pos0, w.chunk_tokens, out, None, ws)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def operand_sweep(crattn, w, dev, n=25):
    """The step attention on N(0, 1) operands and on constant K and V (same
    queries, same shapes, same kernel): per-launch ms of one burst of n
    launches after n warm-up launches, in that order.  The instruction stream
    is the same; on this chip the clock under matrix load depends on the
    operand data, so the gap between the two is the data's cost in clock."""
    import torch

    from workloads import normal, prior_cache

    q = normal((w.B, w.lq, w.H, w.D), 1000 * w.index).to(dev)
    kc, vc = prior_cache(w)
    kc, vc = kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    res = {}
    for name, (k_, v_) in (("normal", (kc, vc)),
                           ("const_kv", (torch.full_like(kc, 0.5), torch.full_like(vc, 0.5)))):
        def call(i, k_=k_, v_=v_):
            crattn.chunk_causal_attn(q, k_, v_, w.kv_len, w.q_pos0, w.chunk_tokens, out, None,
                                     None)
        burst_ms(call, 1, n)
        res[name] = round(burst_ms(call, 1, n)[0], 4)
    return {"attn_ms_normal_operands": res["normal"], "attn_ms_const_kv": res["const_kv"]}


def burst_ms(call, bursts, n):
    """Per-launch time (ms) of `bursts` bursts of n back-to-back calls, each
    burst between two events on the stream; sorted ascending."""
    import torch

    out = []
    for _ in range(bursts):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / n)
    return sorted(out)


def time_qkv(crattn, w, dev, table, ext, burst=20, bursts=5):
    """Fused QKV projection + RoPE + append of the chunk (hidden size H*D):
    per-launch time (ms) of bursts of back-to-back launches over four
    hidden-state sets; sorted ascending, one value per burst."""
    import torch

    from workloads import projection_inputs

    sets = [projection_inputs(w, i) for i in range(4)]
    xs = [x.to(dev) for x, _ in sets]
    wt = sets[0][1].to(dev)
    q_out = torch.empty(w.B, w.lq, w.H, w.D, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(w.B, w.H, w.cap, w.D, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)

    def call(i):
        crattn.qkv_rope_append(xs[i % 4], wt, q_out, kc, vc, w.cache_pos, table, *ext, w.t0,
                               w.tok_off, w.grid_h, w.grid_w)

    for i in range(2 * burst):
        call(i)
    torch.cuda.synchronize()
    return burst_ms(call, bursts, burst)


def qkv_matmul_us(w, dev, burst=20, bursts=5):
    """torch's bf16 matmul (hipBLASLt) of the same projection, x [n, C] times
    W^T [C, 3 H D], without the rotation or the append: per-launch µs of the
    median burst over the same four hidden-state sets (W^T made contiguous
    first)."""
    import torch

    from workloads import projection_inputs

    sets = [projection_inputs(w, i) for i in range(4)]
    xs = [x.to(dev).reshape(-1, x.shape[-1]) for x, _ in sets]
    wtt = sets[0][1].to(dev).t().contiguous()
    y = torch.empty(xs[0].shape[0], wtt.shape[1], dtype=torch.bfloat16, device=dev)
    for i in range(2 * burst):
        torch.matmul(xs[i % 4], wtt, out=y)
    torch.cuda.synchronize()
    ms = burst_ms(lambda i: torch.matmul(xs[i % 4], wtt, out=y), bursts, burst)[bursts // 2]
    return ms * 1e3


def time_hsa(crattn, w, b, kf=6, kb=32):
    """Hierarchical block-sparse attention on the step's chunk (rotated Q' and
    the 7-chunk cache of buffer set b): per-launch times of the key pooling
    of one appended chunk, of the selection (kf frames, kb blocks per
    256-row query block) and of the sparse attention; FLOPs counted over the
    keys each query block attends (own chunk + selected blocks)."""
    import torch

    per_frame = w.grid_h * w.grid_w
    L = w.chunk_tokens
    pool = torch.empty(crattn.hsa_pool_bytes(w.B, w.H, w.cap, w.D, per_frame) // 4,
                       dtype=torch.float32, device=b.q_out.device)
    crattn.hsa_pool_keys(b.kc, 0, w.cap, per_frame, pool)
    nqb = -(-w.lq // crattn.HSA_QBLOCK)
    sel = torch.empty(w.B, w.H, nqb, kb, dtype=torch.int32, device=pool.device)
    own0 = (w.q_pos0 // L) * L

    def pool_call(i):
        crattn.hsa_pool_keys(b.kc, own0, L, per_frame, pool)

    def select_call(i):
        crattn.hsa_select(b.q_out, pool, w.cap, w.kv_len, per_frame, w.q_pos0, L, kf, kb, sel)

    def attn_call(i):
        crattn.hsa_attn(b.q_out, b.kc, b.vc, w.kv_len, w.q_pos0, L, per_frame, sel, b.out, b.lse)

    for f in (pool_call, select_call, attn_call):
        for i in range(3):
            f(i)
    torch.cuda.synchronize()
    pool_ms = burst_ms(pool_call, 5, 20)[2]
    sel_ms = burst_ms(select_call, 5, 20)[2]
    attn_ms = burst_ms(attn_call, 5, 10)[2]
    # visible keys of each query block: the own chunk plus its blocks
    s = sel.cpu()
    nbf = -(-per_frame // crattn.HSA_KBLOCK)
    fl = 0
    for i in range(nqb):
        rows = min(crattn.HSA_QBLOCK, w.lq - i * crattn.HSA_QBLOCK)
        for h in range(w.H):
            ids = [int(x) for x in s[0, h, i] if int(x) >= 0]
            keys = L + sum(min(crattn.HSA_KBLOCK, per_frame - (x % nbf) * crattn.HSA_KBLOCK)
                           for x in ids)
            fl += 4 * rows * keys * w.D
    return pool_ms, sel_ms, attn_ms, fl


def time_svg2(crattn, w, q, kc, vc, out, lse, Cq=20, Ck=64, iters=2, p=0.9, splits=2):
    """Semantic-permutation sparse attention on one chunk's call: rotated
    queries q [B, lq, H, D] against the cache kc, vc.  The keys of every
    chunk slot are clustered first (Ck clusters, from tokens, 3 iterations:
    a stored chunk's clusters are made once).  A denoising call then runs
    k-means of the own slot's keys and of the queries (both in one launch
    sequence, each started from the previous call's centroids, `iters`
    iterations; the same call with the two k-means on two streams is timed
    beside it), the
    plan (top-p selection, key lists, query tiles) and the attention over
    the lists.  Returns per-launch times (ms) of each part and of the whole
    call, and the FLOPs over the listed keys."""
    import torch

    dev = q.device
    B, H, D, L, Lq = w.B, w.H, w.D, w.chunk_tokens, w.lq
    S = w.cap // L
    n_vis = w.kv_len // L
    own = w.q_pos0 // L
    kcent = torch.empty(B, H, S, Ck, D, dtype=torch.float32, device=dev)
    kperm = torch.empty(B, H, S, L, dtype=torch.int32, device=dev)
    koff = torch.empty(B, H, S, Ck + 1, dtype=torch.int32, device=dev)
    wsk = torch.empty(crattn.svg2_kmeans_workspace_bytes(B, H, L, Ck) // 4 + 4,
                      dtype=torch.float32, device=dev)
    wsq = torch.empty(crattn.svg2_kmeans_workspace_bytes(B, H, Lq, Cq) // 4 + 4,
                      dtype=torch.float32, device=dev)
    for s in range(n_vis):
        crattn.svg2_kmeans(kc[:, :, s * L:(s + 1) * L], Ck, 3, True, kcent[:, :, s],
                           kperm[:, :, s], koff[:, :, s], wsk)
    qcent = torch.empty(B, H, Cq, D, dtype=torch.float32, device=dev)
    qperm = torch.empty(B, H, Lq, dtype=torch.int32, device=dev)
    qoff = torch.empty(B, H, Cq + 1, dtype=torch.int32, device=dev)
    qv = q.permute(0, 2, 1, 3)
    crattn.svg2_kmeans(qv, Cq, 3, True, qcent, qperm, qoff, wsq)
    cap_l = -(-n_vis * L // 64) * 64
    lists = torch.empty(B, H, Cq, cap_l, dtype=torch.int32, device=dev)
    llen = torch.empty(B, H, Cq, dtype=torch.int32, device=dev)
    ns = crattn.svg2_n_slots(Lq, Cq)
    slots = torch.empty(B, H, ns, 4, dtype=torch.int32, device=dev)
    sel = torch.empty(B, H, Cq, n_vis * Ck, dtype=torch.int32, device=dev)
    wsa = torch.empty(crattn.svg2_attn_workspace_bytes(B, H, Lq, D, ns, splits) // 4,
                      dtype=torch.float32, device=dev)
    ks = kc[:, :, own * L:(own + 1) * L]
    side = torch.cuda.Stream(device=dev)  # default priority
    main = torch.cuda.current_stream(dev)

    def key_call(i):
        crattn.svg2_kmeans(ks, Ck, iters, False, kcent[:, :, own], kperm[:, :, own],
                           koff[:, :, own], wsk)

    def query_call(i, stream=None):
        crattn.svg2_kmeans(qv, Cq, iters, False, qcent, qperm, qoff, wsq, stream=stream)

    def plan_call(i):
        crattn.svg2_plan(qcent, qoff, kcent, koff, kperm, n_vis, Lq, p, sel, lists, llen, slots)

    def attn_call(i):
        crattn.svg2_attn(q, kc, vc, qperm, slots, lists, llen, out, lse, splits, wsa)

    def whole_call_two_streams(i):
        # the query k-means on a second stream, overlapping the key k-means
        side.wait_stream(main)
        query_call(i, side)
        key_call(i)
        main.wait_stream(side)
        plan_call(i)
        attn_call(i)

    def whole_call(i):
        # both k-means in one launch sequence (svg2_kmeans2)
        crattn.svg2_kmeans2((ks, Ck, kcent[:, :, own], kperm[:, :, own], koff[:, :, own], wsk),
                            (qv, Cq, qcent, qperm, qoff, wsq), iters, False)
        plan_call(i)
        attn_call(i)

    def cold_call(i):
        crattn.svg2_kmeans(ks, Ck, 3, True, kcent[:, :, own], kperm[:, :, own],
                           koff[:, :, own], wsk)

    for f in (key_call, query_call, plan_call, attn_call, whole_call, whole_call_two_streams):
        for i in range(3):
            f(i)
    torch.cuda.synchronize()
    t = {"keys": burst_ms(key_call, 5, 10)[2], "queries": burst_ms(query_call, 5, 10)[2],
         "plan": burst_ms(plan_call, 5, 10)[2], "attn": burst_ms(attn_call, 5, 10)[2],
         "call": burst_ms(whole_call, 5, 10)[2], "keys_cold": burst_ms(cold_call, 3, 5)[1],
         "call_two_streams": burst_ms(whole_call_two_streams, 5, 10)[2]}
    # the same call captured once in a HIP graph and replayed (its ~15
    # launches then cost no host-side launch time)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        whole_call(0)
    for i in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t["call_graph"] = burst_ms(lambda i: graph.replay(), 5, 10)[2]
    del graph
    key_call(0)  # leave the own slot's clusters warm, as before the timed calls
    plan_call(0)
    torch.cuda.synchronize()
    sizes = (qoff[..., 1:] - qoff[..., :-1]).to(torch.int64).cpu()
    fl = int(4 * D * (sizes * llen.to(torch.int64).cpu()).sum())
    return t, fl


def svg2_extras(crattn, w, dev, dense_attn_ms, dense_flops, Cq=20, Ck=64, iters=2, p=0.9,
                splits=2):
    """The semantic-permutation call at the step's shape on two inputs:
    clustered queries and keys (the structure the method relies on) and the
    step's N(0, 1) inputs (attention nearly uniform, so density ~ p)."""
    import torch

    from workloads import clustered_qk, prior_cache

    res = {"Cq": Cq, "Ck_per_chunk": Ck, "kmeans_iters_per_call": iters, "p": p,
           "splits": splits}
    _, vc = prior_cache(w)
    vc = vc.to(dev)
    out = torch.empty(w.B, w.lq, w.H, w.D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.B, w.H, w.lq, dtype=torch.float32, device=dev)
    for tag in ("clustered", "normal"):
        if tag == "clustered":
            q, kc = clustered_qk(w)
        else:
            q = torch.randn(w.B, w.lq, w.H, w.D, generator=torch.Generator().manual_seed(77),
                            dtype=torch.float32).to(torch.bfloat16)
            kc, _ = prior_cache(w)
        q, kc = q.to(dev), kc.to(dev)
        t, sfl = time_svg2(crattn, w, q, kc, vc, out, lse, Cq, Ck, iters, p, splits)
        tf = sfl / (t["attn"] * 1e-3) / 1e12
        res[tag] = {
            "density": round(sfl / dense_flops, 4),
            "kmeans_own_keys_us": round(t["keys"] * 1e3, 1),
            "kmeans_own_keys_cold_3it_us": round(t["keys_cold"] * 1e3, 1),
            "kmeans_queries_us": round(t["queries"] * 1e3, 1),
            "plan_us": round(t["plan"] * 1e3, 1), "attn_us": round(t["attn"] * 1e3, 1),
            "call_us": round(t["call"] * 1e3, 1),
            "call_two_streams_us": round(t["call_two_streams"] * 1e3, 1),
            "call_graph_replay_us": round(t["call_graph"] * 1e3, 1), "listed_flops": sfl,
            "attn_tflops": round(tf, 1),
            "call_speedup_vs_dense_attn": (round(dense_attn_ms / t["call"], 2)
                                           if dense_attn_ms is not None else None),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}
        del q, kc
    del vc, out, lse
    torch.cuda.empty_cache()
    return res


def fused_step_ms(crattn, w, sets, table, ext, ws, reps=10, rounds=3):
    """The step with the query rotation folded into attention (the
    RoPE/append pass writes only K' and V, then chunk_causal_attn_rope
    rotates Q on load) against the plain step, timed in alternating blocks of
    reps steps in the same window so clock drift hits both alike.  Returns
    (plain ms, fused ms): the median block of each."""
    import torch

    def plain(i):
        run_step(crattn, w, sets[i % len(sets)], table, ext, ws)

    def fused(i):
        b = sets[i % len(sets)]
        crattn.rope_apply_append(None, None, b.k, b.v, b.kc, b.vc, w.cache_pos, table, *ext, w.t0,
                                 w.tok_off, w.grid_h, w.grid_w)
        crattn.chunk_causal_attn_rope(b.q, table, *ext, w.t0, w.grid_h, w.grid_w, b.kc, b.vc,
                                      w.kv_len, w.q_pos0, w.chunk_tokens, b.out, b.lse, ws)

    for i in range(4):
        plain(i)
        fused(i)
    torch.cuda.synchronize()
    tp, tf = [], []
    for _ in range(rounds):
        tp += burst_ms(plain, 1, reps)
        tf += burst_ms(fused, 1, reps)
    return sorted(tp)[len(tp) // 2], sorted(tf)[len(tf) // 2]


def rollout_ms(crattn, dev, reps=2, hsa=None):
    """Whole 480P rollout: 7 chunks x (4 denoising calls + 1 cache update),
    with dense or (hsa = (kf, kb)) block-sparse attention."""
    import torch

    from autoregressive_video_diffusion_amd.rollout import ChunkRollout
    from workloads import ROLLOUT480 as w

    ro = ChunkRollout(w.B, w.H, w.D, w.frames, w.grid_h, w.grid_w, window=7, max_chunks=7,
                      device=dev, hsa=hsa)
    n = w.chunk_tokens
    qkv = [tuple(torch.randn(w.B, n, w.H, w.D, device=dev).to(torch.bfloat16) for _ in range(3))
           for _ in range(5)]
    q_out = torch.empty_like(qkv[0][0])
    out = torch.empty_like(q_out)

    def once():
        for c in range(7):
            for j in range(4):
                ro.denoise(c, *qkv[j], q_out, out)
            ro.update(c, qkv[4][1], qkv[4][2])

    once()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    return (time.perf_counter() - t) * 1e3 / reps


def hsa_win720(crattn, dev, dense_ms, kf=6, kb=32):
    """HSA on the 720P window (t0 81, own chunk in slot 6 of the 7-slot
    ring): key pooling of the ring, selection (kf of 18 history frames, kb
    blocks per 256-row query block) and the sparse attention; FLOPs over the
    keys each query block attends."""
    import torch

    from workloads import WIN720 as w, normal, prior_cache

    per_frame, L, cap = w.grid_h * w.grid_w, w.chunk_tokens, w.cap
    q = normal((w.B, w.lq, w.H, w.D), 720).to(dev)
    kc, vc = (x.to(dev) for x in prior_cache(w))
    out = torch.empty_like(q)
    pool = torch.empty(crattn.hsa_pool_bytes(w.B, w.H, cap, w.D, per_frame) // 4,
                       dtype=torch.float32, device=dev)
    crattn.hsa_pool_keys(kc, 0, cap, per_frame, pool)
    nqb = -(-w.lq // crattn.HSA_QBLOCK)
    sel = torch.empty(w.B, w.H, nqb, kb, dtype=torch.int32, device=dev)
    own = w.slot * L

    def select_call(i):
        crattn.hsa_select(q, pool, cap, cap, per_frame, own, L, kf, kb, sel)

    def attn_call(i):
        crattn.hsa_attn(q, kc, vc, cap, own, L, per_frame, sel, out)

    def pool_call(i):
        crattn.hsa_pool_keys(kc, own, L, per_frame, pool)

    for f in (pool_call, select_call, attn_call):
        f(0)
        f(1)
    torch.cuda.synchronize()
    pool_ms = burst_ms(pool_call, 3, 5)[1]
    sel_ms = burst_ms(select_call, 3, 5)[1]
    attn_ms = burst_ms(attn_call, 3, 3)[1]
    s_ = sel.cpu()
    nbf = -(-per_frame // crattn.HSA_KBLOCK)
    fl = 0
    for i in range(nqb):
        rows = min(crattn.HSA_QBLOCK, w.lq - i * crattn.HSA_QBLOCK)
        for h in range(w.H):
            ids = [int(x) for x in s_[0, h, i] if int(x) >= 0]
            keys = L + sum(min(crattn.HSA_KBLOCK, per_frame - (x % nbf) * crattn.HSA_KBLOCK)
                           for x in ids)
            fl += 4 * rows * keys * w.D
    tf = fl / (attn_ms * 1e-3) / 1e12
    del q, kc, vc, out, pool
    torch.cuda.empty_cache()
    return {"kf": kf, "kb": kb, "pool_chunk_us": round(pool_ms * 1e3, 2),
            "select_us": round(sel_ms * 1e3, 2), "attn_ms": round(attn_ms, 4),
            "visible_flops": fl, "speedup_vs_dense_attn": round(dense_ms / attn_ms, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def rollout_breakdown(crattn, dev):
    """The 480P rollout (7 chunks x (4 denoising calls + 1 cache update)),
    every call bracketed by events: per chunk the mean RoPE/append and
    attention time of its denoising calls and the cache-update time, with
    their rates against the rooflines, and the totals."""
    import torch

    from autoregressive_video_diffusion_amd.rollout import ChunkRollout
    from workloads import ROLLOUT480 as w

    ro = ChunkRollout(w.B, w.H, w.D, w.frames, w.grid_h, w.grid_w, window=7, max_chunks=7,
                      device=dev)
    n = w.chunk_tokens
    g = torch.Generator(device="cpu").manual_seed(2024)
    qkv = [tuple(torch.randn(w.B, n, w.H, w.D, generator=g).to(torch.bfloat16).to(dev)
                 for _ in range(3)) for _ in range(5)]
    q_out = torch.empty_like(qkv[0][0])
    out = torch.empty_like(q_out)

    def once(ev=None):
        for c in range(7):
            for j in range(4):
                q, k, v = qkv[j]
                if ev is not None:
                    ev[c][j][0].record()
                ro.rope_append(c, q, q_out, k, v)
                if ev is not None:
                    ev[c][j][1].record()
                ro.attend(c, q_out, out)
                if ev is not None:
                    ev[c][j][2].record()
            if ev is not None:
                ev[c][4][0].record()
            ro.update(c, qkv[4][1], qkv[4][2])
            if ev is not None:
                ev[c][4][1].record()

    once()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[[mk() for _ in range(3)] for _ in range(5)] for _ in range(7)]
    t0 = time.perf_counter()
    once(ev)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    rb, ub = rope_bytes(w.B, n, w.H, w.D), rope_bytes(w.B, n, w.H, w.D, with_q=False)
    chunks, tot_a, tot_r, tot_u, tot_fl = [], 0.0, 0.0, 0.0, 0
    for c in range(7):
        a = [ev[c][j][1].elapsed_time(ev[c][j][2]) for j in range(4)]
        r = [ev[c][j][0].elapsed_time(ev[c][j][1]) for j in range(4)]
        u = ev[c][4][0].elapsed_time(ev[c][4][1])
        fl = attn_flops(w.B, w.H, n, (c + 1) * n, w.D)
        am = sum(a) / 4
        chunks.append({"chunk": c, "keys": (c + 1) * n, "attn_ms": round(am, 4),
                       "attn_tflops": round(fl / (am * 1e-3) / 1e12, 1),
                       "rope_append_us": round(sum(r) / 4 * 1e3, 2),
                       "cache_update_us": round(u * 1e3, 2)})
        tot_a += sum(a)
        tot_r += sum(r)
        tot_u += u
        tot_fl += 4 * fl
    a_tf = tot_fl / (tot_a * 1e-3) / 1e12
    r_gbs = (28 * rb + 7 * ub) / ((tot_r + tot_u) * 1e-3) / 1e9
    return {"calls": "7 chunks x (4 x (RoPE/append + attention) + cache update)",
            "wall_ms": round(wall, 3), "attn_ms_total": round(tot_a, 3),
            "rope_append_ms_total": round(tot_r + tot_u, 4), "per_chunk": chunks,
            "attn_roofline": {"bound": "mfma", "achieved": round(a_tf, 1),
                              "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(a_tf / PEAK_BF16_TFLOPS, 4), "flops": tot_fl},
            "rope_roofline": {"bound": "hbm", "achieved": round(r_gbs, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(r_gbs / PEAK_HBM_GBS, 4),
                              "bytes": 28 * rb + 7 * ub}}


def rope_append_rate(crattn, w, dev, sets=1, bursts=5, burst=10):
    """RoPE/append of one denoising call of workload w over `sets` buffer
    sets used round-robin: per-launch µs of the median burst, GB/s and the
    fraction of HBM peak (algorithmic bytes, 6 tensors)."""
    import torch

    from workloads import call_qkv

    mt, mh, mw = w.table_extents()
    table = torch.empty(crattn.rope_table_bytes(w.D, mt, mh, mw) // 4, dtype=torch.float32,
                        device=dev)
    crattn.rope_precompute(table, w.D, mt, mh, mw, w.theta)
    bufs = []
    for i in range(sets):
        q, k, v = (x.to(dev) for x in call_qkv(w, i))
        kc = torch.empty(w.B, w.H, w.cap, w.D, dtype=torch.bfloat16, device=dev)
        bufs.append((q, k, v, torch.empty_like(q), kc, torch.empty_like(kc)))

    def call(i):
        q, k, v, qo, kc, vc = bufs[i % sets]
        crattn.rope_apply_append(q, qo, k, v, kc, vc, w.cache_pos, table, mt, mh, mw, w.t0,
                                 w.tok_off, w.grid_h, w.grid_w)

    for i in range(2 * sets + 2):
        call(i)
    torch.cuda.synchronize()
    ms = burst_ms(call, bursts, max(burst, sets))[bursts // 2]
    b = rope_bytes(w.B, w.lq, w.H, w.D)
    gbs = b / (ms * 1e-3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return {"us": round(ms * 1e3, 2), "bytes_per_launch": b, "buffer_sets": sets,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def device_copy_us(nbytes, sets=8, bursts=7, burst=40):
    """torch's device-to-device copy of one nbytes buffer into another, over
    `sets` buffer pairs used round-robin (past the Infinity Cache, as the
    RoPE/append pass is timed): per-launch µs of the median burst.  The same
    bytes cross HBM as in a pass that reads nbytes and writes nbytes."""
    import torch

    n = nbytes // 2
    src = [torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_() for _ in range(sets)]
    dst = [torch.empty_like(x) for x in src]

    def call(i):
        dst[i % sets].copy_(src[i % sets])

    for i in range(2 * sets):
        call(i)
    torch.cuda.synchronize()
    ms = burst_ms(call, bursts, burst)[bursts // 2]
    del src, dst
    torch.cuda.empty_cache()
    return ms * 1e3


def matmul_tflops(n=8192, reps=20):
    """torch's bf16 matmul (hipBLASLt) of two n x n N(0,1) matrices on this
    box: a reference for what the matrix cores sustain on random operands
    under the same power limit (TFLOP/s of the median of five bursts)."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    ms = burst_ms(lambda i: torch.matmul(a, b, out=c), 5, reps)[2]
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def sample_rows(lq, per_frame, stride=16):
    """Every stride-th query row plus the first and last row of every frame."""
    import numpy as np

    rows = set(range(0, lq, stride))
    for f0 in range(0, lq, per_frame):
        rows |= {f0, min(lq, f0 + per_frame) - 1}
    return np.array(sorted(rows), dtype=np.int64)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_extras():
    """Host timings of the oracle on the other workloads: the SP-rank slice
    whole; the 480P rollout and the 720P window on a 1/16 row sample (every
    16th row plus the first and last row of every frame, all heads), scaled
    to all rows and labelled extrapolated."""
    import numpy as np

    import oracle
    from workloads import ROLLOUT480, SP480, WIN720

    threads = oracle.default_threads()
    rng = np.random.default_rng(11)
    res = {}

    def kv(w, cap):
        # data values do not change the oracle's cost: a random block tiled
        blk = rng.standard_normal((w.B, w.H, 4096, w.D))
        reps = -(-cap // 4096)
        k = np.ascontiguousarray(np.tile(blk, (1, 1, reps, 1))[:, :, :cap])
        return k, k * 0.5

    w = SP480
    q = rng.standard_normal((w.B, w.lq, w.H, w.D))
    k, v = kv(w, w.cap)
    t = time.perf_counter()
    oracle.attn(q, k, v, w.kv_len, w.q_pos0, w.chunk_tokens, threads=threads)
    dt = time.perf_counter() - t
    fl = attn_flops(w.B, w.H, w.lq, w.kv_len, w.D)
    res["sp480"] = {"s": round(dt, 2), "tflops": round(fl / dt / 1e12, 6), "rows": "all"}

    w = ROLLOUT480
    per_frame = w.grid_h * w.grid_w
    rows = sample_rows(w.lq, per_frame)
    q = rng.standard_normal((w.B, w.lq, w.H, w.D))
    k, v = kv(w, w.cap)
    dt, fl = 0.0, 0
    for c in range(7):
        t = time.perf_counter()
        oracle.attn(q, k, v, (c + 1) * w.lq, c * w.lq, w.chunk_tokens, rows=rows,
                    threads=threads)
        dt += time.perf_counter() - t
        fl += attn_flops(w.B, w.H, len(rows), (c + 1) * w.lq, w.D)
    scale = 4 * w.lq / len(rows)      # all rows, 4 denoising calls per chunk
    res["rollout480"] = {"s_extrapolated": round(dt * scale, 2),
                         "tflops": round(fl / dt / 1e12, 6),
                         "sample": f"{len(rows)} of {w.lq} rows, one call per chunk "
                                   f"({dt:.1f} s), scaled x{scale:.1f}"}
    del k, v

    w = WIN720
    rows = sample_rows(w.lq, w.grid_h * w.grid_w)
    q = rng.standard_normal((w.B, w.lq, w.H, w.D))
    k, v = kv(w, w.cap)
    t = time.perf_counter()
    oracle.attn(q, k, v, w.kv_len, w.q_pos0, w.chunk_tokens, rows=rows, threads=threads)
    dt = time.perf_counter() - t
    fl = attn_flops(w.B, w.H, len(rows), w.kv_len, w.D)
    res["win720"] = {"s_extrapolated": round(dt * w.lq / len(rows), 2),
                     "tflops": round(fl / dt / 1e12, 6),
                     "sample": f"{len(rows)} of {w.lq} rows ({dt:.1f} s), scaled "
                               f"x{w.lq / len(rows):.1f}"}
    res["threads"] = threads
    return res


def cpu_baseline(w, stride=1):
    """The oracle on the host cores: attention of every `stride`-th query row
    of the 480P chunk (all 12 heads, all 32760 keys), fp64.  The default is
    the whole chunk, about 10 s on 16 host threads."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(7)
    q = rng.standard_normal((w.B, w.lq, w.H, w.D))
    k = rng.standard_normal((w.B, w.H, w.cap, w.D))
    v = rng.standard_normal((w.B, w.H, w.cap, w.D))
    rows = np.arange(0, w.lq, stride)
    threads = oracle.default_threads()
    t = time.perf_counter()
    oracle.attn(q, k, v, w.kv_len, w.q_pos0, w.chunk_tokens, rows=rows, threads=threads)
    dt = time.perf_counter() - t
    fl = attn_flops(w.B, w.H, len(rows), w.kv_len, w.D)
    # one RoPE pass of the chunk's Q and K (fp64), for the append row
    x = rng.standard_normal((w.B, w.lq, w.H, w.D))
    t = time.perf_counter()
    oracle.rope(x, w.t0, w.tok_off, w.grid_h, w.grid_w)
    oracle.rope(x, w.t0, w.tok_off, w.grid_h, w.grid_w)
    dt_rope = time.perf_counter() - t
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": (f"attention of {len(rows)} of {w.lq} query rows (stride {stride}) x "
                       f"{w.H} heads vs {w.kv_len} keys, head_dim {w.D}, fp64, "
                       f"{dt:.1f} s on {threads} threads; RoPE of the chunk's Q and K "
                       f"{dt_rope * 1e3:.0f} ms")}


def copy_calibration():
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the attention launches keep speeding up over the first ~30 ms of work
    # (clock ramp); 40 warmup steps (~40 ms) reach the steady state
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--sets", type=int, default=8,
                    help="buffer sets used round-robin (8 x 273 MB: between two uses of a set "
                         "the others move ~600 MB, more than the 256 MB Infinity Cache)")
    ap.add_argument("--ramp-steps", type=int, default=64,
                    help="untimed steps before the warm-up ones: the chip's clock ramps over "
                         "its first ~30 ms of matrix work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--operand-sweep", action="store_true",
                    help="only the step attention on N(0,1) vs constant K/V (for a clock counter run)")
    ap.add_argument("--svg2-only", action="store_true",
                    help="only the semantic-permutation call (for profiling it)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU leg "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import autoregressive_video_diffusion_amd as crattn
    from workloads import SP480, STEP480, WIN720

    crattn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = STEP480
    if args.operand_sweep:
        print(json.dumps(operand_sweep(crattn, w, dev)))
        return
    if args.svg2_only:
        fl = attn_flops(w.B, w.H, w.lq, w.kv_len, w.D)
        print(json.dumps({"svg2_480": svg2_extras(crattn, w, dev, None, fl)}))
        return
    table, ext = make_table(w, dev)
    sets = [StepBuffers(w, dev, i) for i in range(args.sets)]
    wsb = crattn.chunk_causal_attn_workspace_bytes(w.B, w.H, w.lq, w.kv_len, w.q_pos0,
                                                   w.chunk_tokens, w.D)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=dev) if wsb else None
    torch.cuda.synchronize()

    for i in range(args.ramp_steps):
        run_step(crattn, w, sets[i % len(sets)], table, ext, ws)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        run_step(crattn, w, sets[i % len(sets)], table, ext, ws)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        b = sets[i % len(sets)]
        e = ev[i]
        e[0].record()
        crattn.rope_apply_append(b.q, b.q_out, b.k, b.v, b.kc, b.vc, w.cache_pos, table, *ext,
                                 w.t0, w.tok_off, w.grid_h, w.grid_w)
        e[1].record()
        crattn.chunk_causal_attn(b.q_out, b.kc, b.vc, w.kv_len, w.q_pos0, w.chunk_tokens, b.out,
                                 b.lse, ws)
        e[2].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / args.steps
    rope_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    attn_each = sorted(e[1].elapsed_time(e[2]) for e in ev)
    attn_ms = sum(attn_each) / args.steps
    pct = lambda f: attn_each[min(len(attn_each) - 1, int(f * len(attn_each)))]

    # RoPE/append alone: bursts of back-to-back launches over the rotated
    # buffer sets, each between two events, so event overhead does not
    # inflate the per-launch time of this ~15 us kernel; the median burst is
    # reported (the spread between bursts is a few percent)
    burst = max(4 * len(sets), 40)

    def rope_call(i):
        b = sets[i % len(sets)]
        crattn.rope_apply_append(b.q, b.q_out, b.k, b.v, b.kc, b.vc, w.cache_pos, table, *ext,
                                 w.t0, w.tok_off, w.grid_h, w.grid_w)

    rope_bursts = burst_ms(rope_call, 7, burst)
    rope_burst_ms = rope_bursts[len(rope_bursts) // 2]
    # the same bytes moved by torch's device copy (half read, half written)
    copy_us = device_copy_us(rope_bytes(w.B, w.lq, w.H, w.D) // 2)
    # the same box's bf16 matmul rate on random operands (power-limited)
    mm_tflops = matmul_tflops()

    # fused QKV projection (the next row of the path), timed on its own
    qkv_bursts = time_qkv(crattn, w, dev, table, ext)
    qkv_mm_us = qkv_matmul_us(w, dev)
    qkv_ms = qkv_bursts[len(qkv_bursts) // 2]
    C = w.H * w.D
    qkv_tflops = qkv_flops(w.B, w.lq, C, w.H, w.D) / (qkv_ms * 1e-3) / 1e12

    fl = attn_flops(w.B, w.H, w.lq, w.kv_len, w.D)
    rb = rope_bytes(w.B, w.lq, w.H, w.D)
    attn_tflops = fl / (attn_ms * 1e-3) / 1e12
    rope_gbs = rb / (rope_burst_ms * 1e-3) / 1e9
    value = fl / (ms_per_step * 1e-3) / 1e12

    extras = {}
    if not args.no_extras:
        extras["attn_operand_sweep"] = operand_sweep(crattn, w, dev)
        extras["sp480_attn_ms"] = round(time_attn_only(crattn, SP480, dev), 4)
        extras["sp480_attn_tflops"] = round(
            attn_flops(1, SP480.H, SP480.lq, SP480.kv_len, SP480.D)
            / (extras["sp480_attn_ms"] * 1e-3) / 1e12, 1)
        hp_ms, hs_ms, ha_ms, h_fl = time_hsa(crattn, w, sets[0])
        h_tf = h_fl / (ha_ms * 1e-3) / 1e12
        extras["hsa480"] = {
            "kf": 6, "kb": 32, "pool_chunk_us": round(hp_ms * 1e3, 2),
            "select_us": round(hs_ms * 1e3, 2), "attn_ms": round(ha_ms, 4),
            "visible_flops": h_fl, "attn_tflops": round(h_tf, 1),
            "speedup_vs_dense_attn": round(attn_ms / ha_ms, 2),
            "select_overhead_pct": round(100 * hs_ms / ha_ms, 2),
            "roofline": {"bound": "mfma", "achieved": round(h_tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(h_tf / PEAK_BF16_TFLOPS, 4)}}
        extras["svg2_480"] = svg2_extras(crattn, w, dev, attn_ms, fl)
        plain_ms, fused_ms = fused_step_ms(crattn, w, sets, table, ext, ws)
        extras["step_plain_vs_fused_qrot_ms"] = [round(plain_ms, 4), round(fused_ms, 4)]
        extras["rollout480"] = rollout_breakdown(crattn, dev)
        extras["rollout480_ms_total"] = extras["rollout480"]["wall_ms"]
        extras["rollout480_ms_per_chunk"] = round(extras["rollout480_ms_total"] / 7, 3)
        extras["rollout480_hsa_ms_total"] = round(rollout_ms(crattn, dev, hsa=(6, 32)), 3)
        extras["sp480_rope_append"] = rope_append_rate(crattn, SP480, dev, sets=8, burst=40)
        extras["sp480_rope_append"]["note"] = ("10.8 MB per launch: launch-bound, and its 8 "
                                               "sets fit the Infinity Cache; reported for context")
        torch.cuda.empty_cache()
        del sets
        torch.cuda.empty_cache()
        extras["win720_rope_append"] = rope_append_rate(crattn, WIN720, dev, sets=1)
        extras["win720_attn_ms"] = round(time_attn_only(crattn, WIN720, dev, reps=3), 3)
        extras["win720_attn_tflops"] = round(
            attn_flops(1, WIN720.H, WIN720.lq, WIN720.kv_len, WIN720.D)
            / (extras["win720_attn_ms"] * 1e-3) / 1e12, 1)
        extras["win720_hsa"] = hsa_win720(crattn, dev, extras["win720_attn_ms"])

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16, seeded; inputs resident in HBM",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "head_dim": w.D,
                   "chunk": f"{w.frames}x{w.grid_h}x{w.grid_w}", "queries": w.lq,
                   "keys": w.kv_len, "t0": w.t0, "buffer_sets": args.sets,
                   "clock_ramp_steps": args.ramp_steps},
        "ms_per_chunk": round(ms_per_step, 4),
        "attn_ms": round(attn_ms, 4),
        "attn_ms_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
        "attn_tflops": round(attn_tflops, 1),
        "pct_bf16_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "rope_append_us": round(rope_burst_ms * 1e3, 2),
        "rope_append_us_p10_p50_p90": [round(rope_bursts[0] * 1e3, 2),
                                       round(rope_burst_ms * 1e3, 2),
                                       round(rope_bursts[-1] * 1e3, 2)],
        "rope_append_in_step_us": round(rope_ms * 1e3, 2),
        "box_reference": {"torch_matmul_bf16_8192_tflops": round(mm_tflops, 1),
                          "attn_over_matmul": round(attn_tflops / mm_tflops, 4),
                          "note": "the same box's hipBLASLt GEMM on N(0,1) operands: what "
                                  "its matrix cores sustain under the power limit"},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic()},
        "rope_roofline": {"bound": "hbm", "achieved": round(rope_gbs, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(rope_gbs / PEAK_HBM_GBS, 4),
                          "bytes_per_launch": rb, "launches_timed": 7 * burst,
                          "traffic": read_traffic("rope"),
                          "device_copy_same_bytes_us": round(copy_us, 2),
                          "device_copy_frac": round(rb / (copy_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                                    4)},
        "qkv_rope_append": {"us": round(qkv_ms * 1e3, 2), "hidden": C,
                            "torch_matmul_same_shape_us": round(qkv_mm_us, 2),
                            "us_per_burst": [round(x * 1e3, 2) for x in qkv_bursts],
                            "roofline": {"bound": "mfma", "achieved": round(qkv_tflops, 1),
                                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                         "frac": round(qkv_tflops / PEAK_BF16_TFLOPS, 4),
                                         "flops_per_launch": qkv_flops(w.B, w.lq, C, w.H, w.D),
                                         "bytes_per_launch": qkv_bytes(w.B, w.lq, C, w.H, w.D),
                                         "traffic": read_traffic("qkv")}},
        "extras": extras,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
        if not args.no_extras:
            rec["cpu_baseline"]["other_workloads"] = oracle_extras()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
