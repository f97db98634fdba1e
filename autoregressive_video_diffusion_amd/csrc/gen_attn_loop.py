#!/usr/bin/env python3
"""Generate attn_loop.inc: the key loop of the dense chunk-causal attention
kernel for gfx950, as one block of hand-scheduled CDNA4 assembly.

    python gen_attn_loop.py [--out attn_loop.inc] [--report]

What the loop computes is the online-softmax flash attention of the kernel in
attn.hip (chunk-based causal attention, "Wave Forcing" abstract): for every
64-key tile, S^T = K Q^T on the matrix cores, p = 2^(s*c - m) with a lazily
raised running maximum m, O^T += V^T P^T, row sums of the bf16-rounded p.
This file only decides the instruction order and the registers.

Shape of the generated code (head_dim 128, 64-key tiles):
  * a workgroup of 4 wavefronts, one per SIMD, owns 256 query rows; each
    wavefront owns 64 rows as two 32-query blocks (qb = 0, 1), so every K
    and V fragment read from LDS feeds two products;
  * O (4 x 32 dims x 2 blocks, fp32) and Q (bf16) live in accumulation
    registers (a0..a191); scores, probabilities and fragments in v0..v235;
  * K/V tiles are copied global -> LDS (global_load_lds_dwordx4) into a ring
    of 4 stages, three tiles ahead, one barrier per tile;
  * a step handles tile t: S(t+1) = K(t+1) Q^T (32 products) while the
    exponentials of S(t) run, then O += P(t) V(t) (32 products) while the
    row maximum of S(t+1) runs; the copy of tile t+3 is issued in between.
    Four step variants (the ring stage and score buffer rotate) are unrolled.

Every MFMA is followed by a share of the other instructions; a scheduler
places them under each group's deadline, and a checker then walks every
control-flow path, inserting s_nop where a result would be read too soon
and s_waitcnt lgkmcnt before each product that reads a fragment.  The wait
states (MFMA result -> VALU read 12, VALU write -> MFMA operand 2, v_exp ->
VALU read 1, VALU write -> v_permlane32_swap 2) are those hipcc itself
inserts for the same pairs on gfx950; accumulation-register reads after an
MFMA get 18.
"""
from __future__ import annotations

import argparse
import os
import sys

# ------------------------------------------------------------------ geometry
D = 128
BN = 64
KP, VP = D // 8 + 1, D // 8 + 4     # padded LDS row pitches in 16-byte cells
K_CELLS, V_CELLS = BN * KP, BN * VP
STAGE = (K_CELLS + V_CELLS) * 16     # bytes of one ring stage (K then V)
V_LDS = K_CELLS * 16                 # V's offset inside a stage
NS = 4
NW = 4
K_INSTR, V_INSTR = K_CELLS // 64, V_CELLS // 64   # 17 and 20 copies of 1 KB
TILE_BYTES = BN * D * 2

# ------------------------------------------------------------------ registers
def S(buf, kb, qb):
    return ((buf * 2 + kb) * 2 + qb) * 16          # v[S .. S+15]


def P(qb, c):
    return 128 + (qb * 4 + c) * 4                  # v[P .. P+3]: packed bf16 pairs


def KF(f):
    return 160 + (f % 4) * 4                       # K fragment ring


def VF(g):
    return 176 + (g % 4) * 4                       # V^T fragment ring


VM = (192, 193)                  # running max per query block (base-2 units)
VTH = (236, 237)                 # rescale threshold per block: (m + 8) / c, in raw scores
VL = ((194, 195), (196, 197))    # row-sum chains per query block
VT = tuple(range(198, 206))      # temporaries
VONES = 206                      # bf16 (1, 1)
VKH8 = 207                       # 8 * (lane / 32)
VDMA = tuple(range(208, 218))    # copy offsets: 5 K slots, 5 V slots
VDMAL = tuple(range(218, 228))   # the same for the last tile (rows clamped)
VKB = tuple(range(228, 232))     # K fragment read base per stage
VVB = tuple(range(232, 236))     # V fragment read base per stage


def O(db, qb):
    return (db * 2 + qb) * 16                      # a[O .. O+15]


def Q(qb, ks):
    return 128 + (qb * 8 + ks) * 4                 # a[Q .. Q+3]


# scalar registers (inputs first, then scratch)
sKH, sVH, sT, sLAST, sREM, sC, sWB, sK5, sIC = 64, 66, 68, 69, 70, 71, 72, 73, 88
sTILE, sT3, sKA, sVA, sSB, sN0, sN1, sTMP = 74, 75, 76, 78, 80, 82, 84, 86
SCRATCH_S = tuple(range(74, 88))


def vr(base, n=1):
    return f"v{base}" if n == 1 else f"v[{base}:{base + n - 1}]"


def ar(base, n=1):
    return f"a{base}" if n == 1 else f"a[{base}:{base + n - 1}]"


def sr(base, n=1):
    return f"s{base}" if n == 1 else f"s[{base}:{base + n - 1}]"


def vset(base, n):
    return tuple(f"v{base + i}" for i in range(n))


def aset(base, n):
    return tuple(f"a{base + i}" for i in range(n))


# ------------------------------------------------------------------ instructions
class Ins:
    """One instruction: its text, its kind and the registers it writes and
    reads (reads of MFMA operands split into A/B and C)."""

    def __init__(self, text, kind, dst=(), src=(), srcc=(), lds_id=None):
        self.text, self.kind = text, kind
        self.dst, self.src, self.srcc = tuple(dst), tuple(src), tuple(srcc)
        self.lds_id = lds_id

    def __repr__(self):
        return self.text


def mfma(dst, a, b, c):
    """dst, c: 16-register ranges ('v', base) or ('a', base); c may be None
    (zero); a, b: 4-register ranges."""
    def rng(t, n):
        f = vset if t[0] == "v" else aset
        return f(t[1], n), (vr if t[0] == "v" else ar)(t[1], n)
    d_set, d_txt = rng(dst, 16)
    a_set, a_txt = rng(a, 4)
    b_set, b_txt = rng(b, 4)
    if c is None:
        c_set, c_txt = (), "0"
    else:
        c_set, c_txt = rng(c, 16)
    return Ins(f"v_mfma_f32_32x32x16_bf16 {d_txt}, {a_txt}, {b_txt}, {c_txt}", "mfma",
               d_set, a_set + b_set, c_set)


def valu(text, dst, src, kind="valu"):
    return Ins(text, kind, dst, src)


def salu(text):
    return Ins(text, "salu")


def label(name):
    return Ins(f"{name}:", "label")


def branch(text, target):
    i = Ins(text, "branch")
    i.target = target
    i.uncond = text.startswith("s_branch")
    return i


_lds_counter = [0]


def ds_read(text, dst):
    _lds_counter[0] += 1
    return Ins(text, "lds", dst, (), lds_id=_lds_counter[0])


# ------------------------------------------------------------------ building blocks
def k_read(f, stage):
    ks, kb = f // 2, f % 2
    off = kb * 32 * KP * 16 + ks * 32
    return [ds_read(f"ds_read_b128 {vr(KF(f), 4)}, {vr(VKB[stage])} offset:{off}",
                    vset(KF(f), 4))]


def v_read(g, stage):
    c, db = g // 4, g % 4
    off = c * 16 * VP * 16 + db * 64
    return [ds_read(f"ds_read_b64_tr_b16 {vr(VF(g), 2)}, {vr(VVB[stage])} offset:{off}",
                    vset(VF(g), 2)),
            ds_read(f"ds_read_b64_tr_b16 {vr(VF(g) + 2, 2)}, {vr(VVB[stage])} "
                    f"offset:{off + 4 * VP * 16}", vset(VF(g) + 2, 2))]


def dma(n, tile_reg_k, tile_reg_v):
    """Copy slot n (0..4 K, 5..9 V) of the tile whose global bases are in
    sKA / sVA into the stage whose per-wave base is in sSB."""
    if n < 4:
        m0 = f"s_add_u32 m0, {sr(sSB)}, {4 * n * 1024}"
        base = tile_reg_k
    elif n == 4:
        m0 = f"s_add_u32 m0, {sr(sSB)}, {sr(sK5)}"
        base = tile_reg_k
    else:
        m0 = f"s_add_u32 m0, {sr(sSB)}, {V_LDS + 4 * (n - 5) * 1024}"
        base = tile_reg_v
    return [Ins(m0, "salu", ("m0",)),
            Ins(f"global_load_lds_dwordx4 {vr(VDMA[n])}, {sr(base, 2)}", "vmem", (),
                (f"v{VDMA[n]}", "m0"))]


def tile_bases(tile_sreg, stage):
    """sKA/sVA = global bases of tile `tile_sreg`; sSB = stage base."""
    return [salu(f"s_lshl_b32 {sr(sTMP)}, {sr(tile_sreg)}, {TILE_BYTES.bit_length() - 1}"),
            salu(f"s_add_u32 {sr(sKA)}, {sr(sKH)}, {sr(sTMP)}"),
            salu(f"s_addc_u32 {sr(sKA + 1)}, {sr(sKH + 1)}, 0"),
            salu(f"s_add_u32 {sr(sVA)}, {sr(sVH)}, {sr(sTMP)}"),
            salu(f"s_addc_u32 {sr(sVA + 1)}, {sr(sVH + 1)}, 0"),
            salu(f"s_add_u32 {sr(sSB)}, {sr(sWB)}, {stage * STAGE}")]


def switch_to_last_offsets():
    return [valu(f"v_mov_b32 {vr(VDMA[i])}, {vr(VDMAL[i])}", (f"v{VDMA[i]}",),
                 (f"v{VDMAL[i]}",)) for i in range(10)]


def exp_group(buf, qb, c, half):
    """Exponentials of keys 8c' + 4*half .. +3 pairs: two packed pairs of
    P[qb][c] (c = 2 kb + c').  Two pairs interleaved so that every v_exp
    result has an instruction between it and its reader."""
    kb, cp = c // 2, c % 2
    base = S(buf, kb, qb) + cp * 8
    out = []
    pairs = [half * 2, half * 2 + 1]          # packed index inside the chunk (0..3)
    regs = [(base + 2 * j, base + 2 * j + 1) for j in pairs]
    for a, b in regs:
        for r in (a, b):
            out.append(valu(f"v_fma_f32 {vr(r)}, {vr(r)}, {sr(sC)}, -{vr(VM[qb])}",
                            (f"v{r}",), (f"v{r}", f"v{VM[qb]}")))
    for a, b in regs:
        for r in (a, b):
            out.append(valu(f"v_exp_f32 {vr(r)}, {vr(r)}", (f"v{r}",), (f"v{r}",), "trans"))
    for j, (a, b) in zip(pairs, regs):
        pr = P(qb, c) + j
        out.append(valu(f"v_cvt_pk_bf16_f32 {vr(pr)}, {vr(a)}, {vr(b)}", (f"v{pr}",),
                        (f"v{a}", f"v{b}")))
    for j in pairs:
        pr = P(qb, c) + j
        lr = VL[qb][j % 2]
        out.append(valu(f"v_dot2_f32_bf16 {vr(lr)}, {vr(pr)}, {vr(VONES)}, {vr(lr)}",
                        (f"v{lr}",), (f"v{pr}", f"v{VONES}", f"v{lr}")))
    return out


MAX_CHAINS = 4      # independent max3 chains per query block (1 or 4)
EXP_PAIRS = True    # interleave the exponential groups two by two
EXP_WEAVE = False   # within a pair, put a non-exponential instruction after each v_exp
MERGE_WAITS = False # fold an lgkmcnt wait into the one before it when possible
ABLATE = ()         # timing probes only: work left out of the main steps


def cross_max(tmp):
    """v[tmp] = max of v[tmp] over the lane and its partner (l ^ 32), the
    other half of the same query column (v[tmp+1] is clobbered)."""
    m, t2 = f"v{tmp}", f"v{tmp + 1}"
    return [valu(f"v_mov_b32 {t2}, {m}", (t2,), (m,)),
            valu(f"v_permlane32_swap_b32 {m}, {t2}", (m, t2), (m, t2), "perm"),
            valu(f"v_max_f32 {m}, {m}, {t2}", (m,), (m, t2))]


def max_ops(buf, qb, tmp, chain_tmps=(), cross=True):
    """Row maximum of S(buf)[*][qb] over this lane's 32 keys, then (cross)
    over the partner lane (l ^ 32), in raw score units: result in v[tmp]
    (v[tmp+1] is clobbered).  With MAX_CHAINS = 4 the 32 values are reduced
    in four independent chains (temporaries v[tmp], v[tmp+1] and chain_tmps)
    joined at the end, so consecutive max3 do not wait on each other.  The
    main steps take the lane's own maximum only: whether to rescale is
    decided per lane, and the rescale block itself takes the row's."""
    vals = [S(buf, kb, qb) + r for kb in range(2) for r in range(16)]
    m = f"v{tmp}"

    def chain(dst, vs):
        out = [valu(f"v_max3_f32 {dst}, {vr(vs[0])}, {vr(vs[1])}, {vr(vs[2])}", (dst,),
                    tuple(f"v{x}" for x in vs[:3]))]
        i = 3
        while i < len(vs):
            if i + 1 < len(vs):
                out.append(valu(f"v_max3_f32 {dst}, {dst}, {vr(vs[i])}, {vr(vs[i + 1])}", (dst,),
                                (dst, f"v{vs[i]}", f"v{vs[i + 1]}")))
                i += 2
            else:
                out.append(valu(f"v_max_f32 {dst}, {dst}, {vr(vs[i])}", (dst,),
                                (dst, f"v{vs[i]}")))
                i += 1
        return out

    if MAX_CHAINS == 1 or not chain_tmps:
        out = chain(m, vals)
    else:
        dsts = [m, f"v{tmp + 1}"] + [f"v{x}" for x in chain_tmps]
        parts = [chain(d, vals[8 * i:8 * i + 8]) for i, d in enumerate(dsts)]
        out = [ins for grp in zip(*parts) for ins in grp]          # round-robin
        out.append(valu(f"v_max3_f32 {m}, {dsts[0]}, {dsts[1]}, {dsts[2]}", (m,),
                        tuple(dsts[:3])))
        out.append(valu(f"v_max_f32 {m}, {m}, {dsts[3]}", (m,), (m, dsts[3])))
    if cross:
        out += cross_max(tmp)
    return out


def threshold(qb):
    """VTH[qb] = (m + 8) / c: a raw score above it would give p > 2^8."""
    t = VTH[qb]
    return [valu(f"v_add_f32 {vr(t)}, 0x41000000, {vr(VM[qb])}", (f"v{t}",), (f"v{VM[qb]}",)),
            valu(f"v_mul_f32 {vr(t)}, {sr(sIC)}, {vr(t)}", (f"v{t}",), (f"v{t}",))]


def rescale_block(cur_buf, tag):
    """Raise the running max where a row's new maximum exceeds it by more
    than 2^8 and rescale that row's sums and O (rare: early tiles).  The
    lanes' raw maxima are in VT[0] (qb 0) and VT[2] (qb 1); the row maxima
    and the per-lane decisions (sN0 / sN1) are taken here, so both halves of
    a row decide alike.  S(cur_buf) is free here and serves as the buffer
    for O."""
    out = [label(f"{tag}")]
    for qb in range(2):
        mc, need = VT[2 * qb], (sN0, sN1)[qb]
        mn, al = VT[4 + 2 * qb], VT[5 + 2 * qb]
        out += cross_max(mc)
        out.append(valu(f"v_cmp_gt_f32_e64 {sr(need, 2)}, {vr(mc)}, {vr(VTH[qb])}",
                        (f"s{need}",), (f"v{mc}", f"v{VTH[qb]}")))
        out += [valu(f"v_mul_f32 {vr(mc)}, {sr(sC)}, {vr(mc)}", (f"v{mc}",), (f"v{mc}",)),
                valu(f"v_cndmask_b32_e64 {vr(mn)}, {vr(VM[qb])}, {vr(mc)}, {sr(need, 2)}",
                     (f"v{mn}",), (f"v{VM[qb]}", f"v{mc}")),
                valu(f"v_sub_f32 {vr(al)}, {vr(VM[qb])}, {vr(mn)}", (f"v{al}",),
                     (f"v{VM[qb]}", f"v{mn}")),
                valu(f"v_exp_f32 {vr(al)}, {vr(al)}", (f"v{al}",), (f"v{al}",), "trans"),
                valu(f"v_mov_b32 {vr(VM[qb])}, {vr(mn)}", (f"v{VM[qb]}",), (f"v{mn}",))]
        out += threshold(qb)
        for ch in range(2):
            lr = VL[qb][ch]
            out.append(valu(f"v_mul_f32 {vr(lr)}, {vr(lr)}, {vr(al)}", (f"v{lr}",),
                            (f"v{lr}", f"v{al}")))
        tmp = S(cur_buf, 0, 0)   # 64 free registers
        regs = [(O(db, qb) + r) for db in range(4) for r in range(16)]
        for i, a in enumerate(regs):
            out.append(Ins(f"v_accvgpr_read_b32 v{tmp + i}, a{a}", "accr", (f"v{tmp + i}",),
                           (f"a{a}",)))
        for i in range(64):
            out.append(valu(f"v_mul_f32 v{tmp + i}, v{tmp + i}, {vr(al)}", (f"v{tmp + i}",),
                            (f"v{tmp + i}", f"v{al}")))
        for i, a in enumerate(regs):
            out.append(Ins(f"v_accvgpr_write_b32 a{a}, v{tmp + i}", "accw", (f"a{a}",),
                           (f"v{tmp + i}",)))
    return out


# ------------------------------------------------------------------ placement
def place(mfmas, items, head=()):
    """Interleave instructions between the MFMAs.  items: (target, Ins) with
    target a fractional gap number: gap g is the run of instructions just
    before MFMA g (gap len(mfmas) follows the last).  Each class of work is
    given targets spread evenly over the gaps where it may run, so every MFMA
    is followed by about the same amount of other work; ties keep list order."""
    n = len(mfmas)
    buckets = [[] for _ in range(n + 1)]
    for seq, (t, ins) in enumerate(items):
        g = min(n, max(0, int(t)))
        buckets[g].append((t, seq, ins))
    out = list(head)
    for g in range(n + 1):
        out += [ins for _, _, ins in sorted(buckets[g], key=lambda x: (x[0], x[1]))]
        if g < n:
            out.append(mfmas[g])
    return out


def spread(instrs, lo, hi):
    """Targets for a list of instructions spread evenly over gaps [lo, hi)."""
    k = len(instrs)
    return [(lo + (hi - lo) * i / k, ins) for i, ins in enumerate(instrs)]


# ------------------------------------------------------------------ program pieces
def qk_mfmas(buf):
    """S(buf) = K Q^T: k-step outer, so each K fragment feeds two
    consecutive products (qb 0, 1) and each accumulator is written every
    fourth product."""
    out = []
    for ks in range(8):
        for kb in range(2):
            for qb in range(2):
                f = ks * 2 + kb
                c = None if ks == 0 else ("v", S(buf, kb, qb))
                out.append(mfma(("v", S(buf, kb, qb)), ("v", KF(f)), ("a", Q(qb, ks)), c))
    return out


def pv_mfmas():
    """O += V^T P^T, chunk by chunk of 16 keys (the order the exponentials
    finish in); each V^T fragment feeds two consecutive products."""
    out = []
    for c in range(4):
        for db in range(4):
            for qb in range(2):
                g = c * 4 + db
                out.append(mfma(("a", O(db, qb)), ("v", VF(g)), ("v", P(qb, c)),
                                ("a", O(db, qb))))
    return out


def exp_chunk(cur, c):
    """The exponentials of chunk c of S(cur), both query blocks: 4 groups of
    12 instructions; with EXP_PAIRS two groups are merged stage by stage
    (fma, exp, cvt, dot2), doubling the distance between each instruction
    and the one that reads its result."""
    groups = [exp_group(cur, qb, c, half) for qb in range(2) for half in range(2)]
    if not EXP_PAIRS:
        return [i for g in groups for i in g]
    out = []
    for a, b in ((groups[0], groups[1]), (groups[2], groups[3])):
        if EXP_WEAVE:
            # fma a | exp a with fma b | exp b with cvt/dot2 a | cvt/dot2 b
            out += a[0:4]
            for k in range(4):
                out += [a[4 + k], b[k]]
            x = a[8:12]
            for k in range(4):
                out += [b[4 + k], x[k]]
            out += b[8:12]
        else:
            for lo, hi in ((0, 4), (4, 8), (8, 10), (10, 12)):
                out += a[lo:hi] + b[lo:hi]
    return out


def exp_items(cur, lo, hi):
    """The exponentials of S(cur), chunk by chunk (chunk c is read by the PV
    products base + 8c + qb), spread over gaps [lo, hi)."""
    instrs = []
    for c in range(4):
        instrs += exp_chunk(cur, c)
    return spread(instrs, lo, hi)


def exp_items_due(cur):
    """The same when the PV products start at once (the last tile): chunk 0
    before the first product, chunk c spread over the 8 products of chunk
    c - 1."""
    out = []
    for c in range(4):
        instrs = exp_chunk(cur, c)
        out += [(0, i) for i in instrs] if c == 0 else spread(instrs, 8 * c - 8, 8 * c - 1)
    return out


KR_AHEAD = 2.5      # gaps between a K fragment's read and its first product
VR_AHEAD = 3.0      # the same for V^T fragments (ring of 4: at most 6)


def k_read_items(stage, frags):
    """K fragment f feeds QK products 2f and 2f+1; its ring slot was last read
    by product 2f - 7, so it can be read up to six products ahead."""
    return [(2 * f - KR_AHEAD, ins) for f in frags for ins in k_read(f, stage)]


def v_read_items(stage, base):
    """V^T fragment g feeds PV products base + 2g and base + 2g + 1; its ring
    slot was last read by product base + 2g - 7."""
    out = []
    for g in range(16):
        for j, ins in enumerate(v_read(g, stage)):
            out.append((base + 2 * g - VR_AHEAD + 0.1 * j, ins))
    return out


def _ablate(items):
    """Drop classes of work from a step's items (timing probes: the results
    are wrong, every access stays where it was)."""
    def drop(i):
        t = i.text
        return (("exp" in ABLATE and (t.startswith("v_fma_f32") or t.startswith("v_exp_f32") or
                                      t.startswith("v_cvt_pk") or t.startswith("v_dot2"))) or
                ("max" in ABLATE and (t.startswith("v_max") or "permlane" in t or
                                      (t.startswith("v_mov_b32") and i.kind == "valu"))) or
                ("lds" in ABLATE and i.kind == "lds") or
                ("dma" in ABLATE and (i.kind == "vmem" or t.startswith("s_add_u32 m0"))) or
                ("barrier" in ABLATE and (i.kind == "barrier" or t.startswith("s_waitcnt vmcnt"))))
    return [(t, i) for t, i in items if not drop(i)]


def step(phi):
    """Main step of phase phi: tile t in the loop counter sT."""
    cur, nxt = phi % 2, 1 - phi % 2
    kst, vst, dst = (phi + 1) % NS, phi % NS, (phi + 3) % NS
    head = [label(f"crt_ph{phi}"),
            salu(f"s_cmp_ge_u32 {sr(sT)}, {sr(sLAST)}"),
            branch(f"s_cbranch_scc1 crt_last{phi}", f"crt_last{phi}"),
            salu(f"s_add_u32 {sr(sT3)}, {sr(sT)}, 3"),
            salu(f"s_min_u32 {sr(sTILE)}, {sr(sT3)}, {sr(sLAST)}"),
            salu(f"s_cmp_eq_u32 {sr(sTILE)}, {sr(sLAST)}"),
            branch(f"s_cbranch_scc1 crt_sw{phi}", f"crt_sw{phi}"),
            label(f"crt_swr{phi}")] + tile_bases(sTILE, dst)
    mf = qk_mfmas(nxt) + pv_mfmas()
    items = []
    # K fragments 0..3 of tile t+1 were read at the end of the previous step
    items += k_read_items(kst, range(4, 16))
    # the copy of tile t+3: one slot every second gap
    for n in range(10):
        for j, ins in enumerate(dma(n, sKA, sVA)):
            items.append((1 + 2 * n + 0.1 * j, ins))
    items += exp_items(cur, 0, 54)
    items += v_read_items(vst, 32)
    # row maximum of S(t+1) (its last products are 28..31)
    m0 = max_ops(nxt, 0, VT[0], (VT[4], VT[5]), cross=False)
    m1 = max_ops(nxt, 1, VT[2], (VT[6], VT[7]), cross=False)
    mx = [i for pair in zip(m0, m1) for i in pair]   # the two blocks interleaved
    items += spread(mx, 34, 63)
    # before the last two products: tile t+2 has landed and every wave is
    # past its reads of tile t's V; then tile t+2's first K fragments
    items += [(62.5, Ins("s_waitcnt lgkmcnt(0)", "wait")),
              (62.6, Ins("s_waitcnt vmcnt(10)", "wait")),
              (62.7, Ins("s_barrier", "barrier"))]
    nkst = (phi + 2) % NS
    items += [(62.8 + 0.01 * f, ins) for f in range(4) for ins in k_read(f, nkst)]
    if ABLATE:
        items = _ablate(items)
        if "mfma" in ABLATE:
            mf = mf[:1]
    body = place(mf, items, head)
    tail = []
    for qb in range(2):
        mc = VT[2 * qb]
        tail.append(valu(f"v_cmp_gt_f32_e64 {sr((sN0, sN1)[qb], 2)}, {vr(mc)}, {vr(VTH[qb])}",
                         (f"s{(sN0, sN1)[qb]}",), (f"v{mc}", f"v{VTH[qb]}")))
    tail += [salu(f"s_or_b64 {sr(sTMP, 2)}, {sr(sN0, 2)}, {sr(sN1, 2)}"),
             branch(f"s_cbranch_scc1 crt_resc{phi}", f"crt_resc{phi}"),
             label(f"crt_rescr{phi}"),
             salu(f"s_add_u32 {sr(sT)}, {sr(sT)}, 1")]
    if phi == NS - 1:
        tail.append(branch("s_branch crt_ph0", "crt_ph0"))
    cold = [label(f"crt_sw{phi}")] + switch_to_last_offsets() + \
        [branch(f"s_branch crt_swr{phi}", f"crt_swr{phi}")]
    cold += rescale_block(cur, f"crt_resc{phi}") + \
        [branch(f"s_branch crt_rescr{phi}", f"crt_rescr{phi}")]
    return body + tail, cold


def last_step(phi):
    """Tile t = last: exponentials of S(cur) (keys at or past the valid count
    masked when the tile is partial) and O += P V; no next tile."""
    cur, vst = phi % 2, phi % NS
    out = [label(f"crt_last{phi}"),
           salu(f"s_cmp_lt_u32 {sr(sREM)}, {BN}"),
           branch(f"s_cbranch_scc0 crt_nomask{phi}", f"crt_nomask{phi}"),
           valu(f"v_mov_b32 {vr(VT[7])}, 0xff800000", (f"v{VT[7]}",), ())]
    for kb in range(2):
        for r in range(16):
            key = kb * 32 + 16 * (r // 8) + r % 8
            t = VT[6]
            out += [valu(f"v_add_u32 {vr(t)}, {key}, {vr(VKH8)}", (f"v{t}",), (f"v{VKH8}",)),
                    valu(f"v_cmp_le_i32_e32 vcc, {sr(sREM)}, {vr(t)}", ("vcc",), (f"v{t}",))]
            for qb in range(2):
                x = S(cur, kb, qb) + r
                out.append(valu(f"v_cndmask_b32_e32 {vr(x)}, {vr(x)}, {vr(VT[7])}, vcc",
                                (f"v{x}",), (f"v{x}", f"v{VT[7]}", "vcc")))
    out.append(label(f"crt_nomask{phi}"))
    items = exp_items_due(cur) + v_read_items(vst, 0)
    body = place(pv_mfmas(), items, out)
    return body + [branch("s_branch crt_end", "crt_end")]


def prologue():
    out = [Ins("s_nop 7", "nop"),
           valu(f"v_mov_b32 {vr(VONES)}, 0x3f803f80", (f"v{VONES}",), ())]
    for qb in range(2):
        for ch in range(2):
            out.append(valu(f"v_mov_b32 {vr(VL[qb][ch])}, 0", (f"v{VL[qb][ch]}",), ()))
    # copies of tiles t, t+1, t+2 (clamped to the last) into stages 0, 1, 2
    for i in range(3):
        out += [salu(f"s_add_u32 {sr(sT3)}, {sr(sT)}, {i}"),
                salu(f"s_min_u32 {sr(sTILE)}, {sr(sT3)}, {sr(sLAST)}"),
                salu(f"s_cmp_eq_u32 {sr(sTILE)}, {sr(sLAST)}"),
                branch(f"s_cbranch_scc0 crt_pro{i}", f"crt_pro{i}")]
        out += switch_to_last_offsets()
        out.append(label(f"crt_pro{i}"))
        out += tile_bases(sTILE, i)
        for n in range(10):
            out += dma(n, sKA, sVA)
    out += [Ins("s_waitcnt vmcnt(20)", "wait"), Ins("s_barrier", "barrier")]
    # S of the first tile into buffer 0, then its row maximum
    out = place(qk_mfmas(0), k_read_items(0, range(16)), out)
    for qb in range(2):
        out += max_ops(0, qb, VT[2 * qb])
        out.append(valu(f"v_mul_f32 {vr(VM[qb])}, {sr(sC)}, {vr(VT[2 * qb])}", (f"v{VM[qb]}",),
                        (f"v{VT[2 * qb]}",)))
        out += threshold(qb)
    # tile t+1 has landed and is visible: its first K fragments
    out += [Ins("s_waitcnt vmcnt(10)", "wait"), Ins("s_barrier", "barrier")]
    for f in range(4):
        out += k_read(f, 1)
    return out


def check_p_ready(body):
    """Every PV product must come after the conversions that write all four
    registers of its P operand in the same step."""
    written = set()
    for ins in body:
        if ins.kind == "valu" and ins.text.startswith("v_cvt_pk_bf16_f32"):
            written |= set(ins.dst)
        if ins.kind == "mfma" and ins.dst[0].startswith("a"):
            p = [r for r in ins.src if r.startswith("v") and 128 <= int(r[1:]) < 160]
            missing = [r for r in p if r not in written]
            if missing:
                raise RuntimeError(f"{ins.text}: P registers {missing} not yet written")


def program():
    main, cold = [], []
    for phi in range(NS):
        b, c = step(phi)
        if "exp" not in ABLATE:
            check_p_ready(b)
        main += b
        cold += c
    lasts = []
    for phi in range(NS):
        b = last_step(phi)
        check_p_ready(b)
        lasts += b
    end = [label("crt_end"), Ins("s_waitcnt vmcnt(0) lgkmcnt(0)", "wait"),
           Ins("s_nop 7", "nop"), Ins("s_nop 7", "nop"), Ins("s_nop 7", "nop")]
    return prologue() + main + cold + lasts + end


# ------------------------------------------------------------------ hazard checker
def required_wait(wkind, r):
    """Wait states needed between a writer of kind wkind and reader r."""
    if wkind == "mfma":
        if r.kind == "mfma":
            return 0    # only same-accumulator chains through srcC occur here
        if r.kind in ("accr", "accw"):
            return 18
        return 12
    if wkind in ("valu", "perm", "trans", "accw"):
        if r.kind == "mfma":
            return 3 if wkind == "accw" else 2
        if r.kind == "perm":
            return 2
        if wkind == "trans":
            return 1
    return 0


def ws_of(i):
    if i.kind == "nop":
        return int(i.text.split()[1]) + 1
    return 0 if i.kind == "label" else 1


def _blocks(prog):
    """Basic blocks: (start, end) index ranges, successors by index."""
    starts = {0}
    for k, i in enumerate(prog):
        if i.kind == "label":
            starts.add(k)
        if i.kind == "branch" and k + 1 < len(prog):
            starts.add(k + 1)
    starts = sorted(starts)
    lab = {i.text[:-1]: k for k, i in enumerate(prog) if i.kind == "label"}
    blocks = []
    for j, s in enumerate(starts):
        e = starts[j + 1] if j + 1 < len(starts) else len(prog)
        succ = []
        last = prog[e - 1]
        if last.kind == "branch":
            succ.append(lab[last.target])
            if not last.uncond and e < len(prog):
                succ.append(e)
        elif e < len(prog):
            succ.append(e)
        blocks.append((s, e, succ))
    return blocks


def _merge(a, b):
    if a is None:
        return b
    if b is None:
        return a
    regs = {}
    for st in (a, b):
        for r, kinds in st[0].items():
            d = regs.setdefault(r, {})
            for k, ws in kinds.items():
                d[k] = min(ws, d.get(k, 10 ** 9))
    lds = dict(a[1])
    for x, n in b[1].items():
        lds[x] = min(n, lds.get(x, 10 ** 9))
    owner = dict(a[2])
    owner.update(b[2])
    return (regs, lds, owner)


def _run(prog, s, e, st, inserts):
    """Walk instructions [s, e) from state st; record needed waits."""
    regs = {r: dict(k) for r, k in st[0].items()}
    lds, owner = dict(st[1]), dict(st[2])
    for k in range(s, e):
        ins = prog[k]
        # outstanding LDS reads into registers this instruction touches
        need = [owner[r] for r in ins.src + ins.srcc + ins.dst if r in owner and owner[r] in lds]
        if need:
            n = min(15, min(lds[x] for x in need))
            inserts.setdefault(k, []).append(f"s_waitcnt lgkmcnt({n})")
            lds = {x: c for x, c in lds.items() if c < n}
        worst = 0
        for r in ins.src + ins.srcc:
            for kind, ws in regs.get(r, {}).items():
                worst = max(worst, required_wait(kind, ins) - ws)
        if worst > 0:
            inserts.setdefault(k, []).append(f"s_nop {worst - 1}")
            regs = {r: {kd: w + worst for kd, w in kinds.items()} for r, kinds in regs.items()}
        if ins.kind == "wait" and "lgkmcnt" in ins.text:
            n = int(ins.text.split("lgkmcnt(")[1].split(")")[0])
            lds = {x: c for x, c in lds.items() if c < n}
        w = ws_of(ins)
        if w:
            regs = {r: {kd: ws + w for kd, ws in kinds.items() if ws + w < 24}
                    for r, kinds in regs.items()}
            regs = {r: kinds for r, kinds in regs.items() if kinds}
        if ins.kind == "lds":
            lds = {x: c + 1 for x, c in lds.items()}
            lds[ins.lds_id] = 0
            for r in ins.dst:
                owner[r] = ins.lds_id
                regs.pop(r, None)
        else:
            for r in ins.dst:
                regs[r] = {ins.kind: 0}
                owner.pop(r, None)
    return (regs, lds, owner)


def fix(prog):
    """Insert s_nop and s_waitcnt lgkmcnt wherever some control-flow path
    needs them (data-flow over the basic blocks: per register the fewest
    wait states since a write of each kind, per outstanding LDS read the
    fewest LDS reads issued after it)."""
    for _ in range(20):
        blocks = _blocks(prog)
        index = {b[0]: j for j, b in enumerate(blocks)}
        entry = {0: ({}, {}, {})}
        for _it in range(12):
            changed = False
            for j, (s, e, succ) in enumerate(blocks):
                if s not in entry:
                    continue
                out = _run(prog, s, e, entry[s], {})
                for t in succ:
                    m = _merge(entry.get(t), out)
                    if entry.get(t) != m:
                        entry[t] = m
                        changed = True
            if not changed:
                break
        inserts = {}
        for s, e, succ in blocks:
            if s in entry:
                _run(prog, s, e, entry[s], inserts)
        if not inserts:
            return prog
        newp = []
        for k, ins in enumerate(prog):
            for txt in inserts.get(k, []):
                newp.append(Ins(txt, "nop" if txt.startswith("s_nop") else "wait"))
            newp.append(ins)
        prog = newp
    raise RuntimeError("hazard fixing did not converge")


def merge_waits(prog, window=12):
    """Fold an s_waitcnt lgkmcnt(n2) into an earlier lgkmcnt(n1) of the same
    straight-line run when at most `window` instructions lie between them:
    with k LDS reads issued in between, lgkmcnt(min(n1, n2 - k)) at the first
    point already guarantees the second (reads complete in order)."""
    out = list(prog)
    i = 0
    while i < len(out):
        a = out[i]
        if a.kind == "wait" and a.text.startswith("s_waitcnt lgkmcnt("):
            n1 = int(a.text.split("(")[1].split(")")[0])
            k = 0
            for j in range(i + 1, min(len(out), i + 1 + window)):
                b = out[j]
                if b.kind in ("label", "branch", "barrier"):
                    break
                if b.kind == "lds":
                    k += 1
                if b.kind == "wait" and b.text.startswith("s_waitcnt lgkmcnt("):
                    n2 = int(b.text.split("(")[1].split(")")[0])
                    if n2 - k >= 0:
                        out[i] = Ins(f"s_waitcnt lgkmcnt({min(n1, n2 - k)})", "wait")
                        del out[j]
                    break
        i += 1
    return out


def stats(prog):
    import collections
    c = collections.Counter(i.kind for i in prog)
    nops = sum(ws_of(i) for i in prog if i.kind == "nop")
    return dict(c), nops


def step_report(prog):
    """Instructions and nop wait states inside each phase's main step."""
    out = []
    for phi in range(NS):
        s = next(k for k, i in enumerate(prog) if i.text == f"crt_ph{phi}:")
        e = next(k for k, i in enumerate(prog) if i.text.startswith("s_add_u32 s68, s68, 1")
                 and k > s)
        seg = prog[s:e]
        n = sum(1 for i in seg if i.kind not in ("label",))
        nop = sum(ws_of(i) for i in seg if i.kind == "nop")
        waits = sum(1 for i in seg if i.kind == "wait")
        out.append((phi, n, nop, waits))
    return out


def render(prog):
    """Assembly lines.  Labels become numeric local labels (each number
    defined once per instance of the asm statement, references resolved
    forward or backward), so every instance has its own."""
    num, where = {}, {}
    for k, i in enumerate(prog):
        if i.kind == "label":
            num[i.text[:-1]] = 10 + len(num)
            where[i.text[:-1]] = k
    out = []
    for k, i in enumerate(prog):
        if i.kind == "label":
            out.append(f"{num[i.text[:-1]]}:")
        elif i.kind == "branch":
            op, tgt = i.text.split()
            out.append(f"  {op} {num[tgt]}{'f' if where[tgt] > k else 'b'}")
        else:
            out.append("  " + i.text)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                  "attn_loop.inc"))
    ap.add_argument("--report", action="store_true")
    ap.add_argument("--kr-ahead", type=float, default=None, help="K fragment read distance")
    ap.add_argument("--vr-ahead", type=float, default=None, help="V fragment read distance")
    ap.add_argument("--max-chains", type=int, default=None, choices=(1, 4))
    ap.add_argument("--exp-pairs", type=int, default=None, choices=(0, 1))
    ap.add_argument("--exp-weave", type=int, default=None, choices=(0, 1))
    ap.add_argument("--merge-waits", type=int, default=None, choices=(0, 1))
    ap.add_argument("--ablate", default="", help="timing probe: comma list of exp, max, lds, "
                    "dma, barrier, mfma left out of the main steps")
    args = ap.parse_args()
    global KR_AHEAD, VR_AHEAD, MAX_CHAINS, EXP_PAIRS, EXP_WEAVE, MERGE_WAITS, ABLATE
    if args.ablate:
        ABLATE = tuple(args.ablate.split(","))
    if args.exp_weave is not None:
        EXP_WEAVE = bool(args.exp_weave)
    if args.merge_waits is not None:
        MERGE_WAITS = bool(args.merge_waits)
    if args.max_chains is not None:
        MAX_CHAINS = args.max_chains
    if args.exp_pairs is not None:
        EXP_PAIRS = bool(args.exp_pairs)
    if args.kr_ahead is not None:
        KR_AHEAD = args.kr_ahead
    if args.vr_ahead is not None:
        VR_AHEAD = args.vr_ahead
    prog = fix(program())
    if MERGE_WAITS:
        prog = fix(merge_waits(prog))
    lines = render(prog)
    text = ("// Generated by gen_attn_loop.py; do not edit.  The key loop of the dense\n"
            "// chunk-causal attention kernel (head_dim 128) in CDNA4 assembly: one\n"
            "// string for an asm statement whose registers are fixed by its operands\n"
            "// and clobbers (see attn.hip).\n"
            "#define CRATTN_ATTN_LOOP_ASM \\\n" +
            " \\\n".join(f'  "{ln}\\n"' for ln in lines) + "\n")
    with open(args.out + ".tmp", "w") as f:
        f.write(text)
    os.replace(args.out + ".tmp", args.out)
    if args.report:
        print(stats(prog), len(prog), file=sys.stderr)
        for r in step_report(prog):
            print("phase %d: %d instructions, %d nop wait states, %d waits" % r, file=sys.stderr)


if __name__ == "__main__":
    main()
