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
    registers (a0..a191); scores, probabilities and fragments in v0..v239;
  * K and V tiles are copied global -> LDS (global_load_lds_dwordx4) into
    two rings of 4 stages (K three tiles ahead, V two), one barrier per tile;
  * a step handles tile t: O += P(t-1) V(t-1) (32 products), then
    S(t+1) = K(t+1) Q^T (32 products), while the exponentials of S(t) run
    beside both.  The product with V runs one tile behind the exponentials,
    so a tile's probabilities are known whole before any of them is used.

No row maximum is taken in the steps.  m starts at the first tile's exact
row maximum and p = 2^(s*c - m) is computed with it; the row sums are kept
in two alternating register sets (before and after each tile), and a step
ends by testing whether any lane's sums passed 2^31.  Until one does, every
p of the tile is below 2^31 and the fp32/bf16 arithmetic is as exact as with
the true maximum (scaling by 2^k changes no relative rounding).  When one
does (a row's scores rose far above m), a cold block takes the tile's row
maximum from its raw scores (the exponentials write to temporaries, so S(t)
is intact), raises m past it and past the mass already summed, rescales O
and the sums, and recomputes the tile's p.

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
K_STAGE, V_STAGE = K_CELLS * 16, V_CELLS * 16   # 17408, 20480 bytes
NS = 4
V_RING = NS * K_STAGE                # V ring after the K ring: 69632
NW = 4
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
# row-sum chains [set][qb][chain]: a step adds its tile to the set of its
# parity, starting from the other set (which keeps the sums before the tile)
VL = (((194, 195), (196, 197)), ((236, 237), (238, 239)))
VT = tuple(range(198, 206))      # exponential temporaries
VA = (240, 241)                  # rescale factors (cold block only)
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
sKH, sVH, sT, sLAST, sREM, sC, sWB, sK5 = 64, 66, 68, 69, 70, 71, 72, 73
sTILE, sTV, sKA, sVA, sSB, sSBV, sN0, sT3, sTMP, sLIM = 74, 75, 76, 78, 80, 81, 82, 84, 85, 86
SUM_LIMIT = 0x4F000000           # 2^31: a lane's row sum above it calls the rescale

# List mode (the block-sparse instance): tile j is the key rows [first_j,
# first_j + rows_j) from a table of (first row, rows) in LDS (at byte sTAB,
# padded with four copies of the last entry), not rows [64j, 64j + 64).
# Entries travel through a queue of four scalar slots (tile j in slot j mod
# 4), read one step ahead; a ragged tile's copies re-read its last row (its
# offsets clamped from the full ones kept in VDMAL) and its scores past the
# valid rows are masked.
LIST = False
sTAB, sCL = 88, 89               # table address; bit 0 / 1: K / V copy offsets clamped
sQK = (90, 91, 92, 93)           # first key row of the tile in each slot
sQR = (94, 95, 96, 97)           # its valid rows (1..64)
VTAB = (242, 243)                # the next entry, read a step ahead
VTA = 244                        # its LDS address

# Gather mode (the semantic-permutation instance): tile j is key rows
# list[64j .. 64j + 63] of a list of row indices in global memory, not rows
# [64j, 64j + 64).  Each step loads the 64 indices of tile t+4 (one per
# lane, lanes past a short final tile clamped to its last entry) into
# VIDX[(j - first) mod 4]; a loaded vector is shifted to byte offsets
# (x 256) once, and a copy slot's per-lane offset is the index of the
# lane's row, fetched across lanes with ds_bpermute_b32 (address VDMAL[n]
# = row * 4), or-ed with the lane's column bytes (byte n % 4 of VCOL[n / 4]).
GATHER = False
VIDX = (242, 243, 244, 245)      # index vectors of four consecutive tiles
VLANE4 = 246                     # lane * 4
VGT = 247                        # address of the index load
VCOL = (248, 249, 250)           # column bytes of the ten copy slots
sLST, sLA, sILIM, sTL, sRL4 = 88, 90, 92, 93, 94   # list base, load address, lane clamp,
                                                     # loaded tile, (rows of last - 1) * 4
sCAPM1 = 95                      # last row of the cache: indices are clamped to it


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


def dma(n):
    """Copy slot n (0..4 K, 5..9 V) of the tiles whose global bases are in
    sKA / sVA into the stages whose per-wave bases are in sSB / sSBV."""
    if n < 4:
        m0 = f"s_add_u32 m0, {sr(sSB)}, {4 * n * 1024}"
        base = sKA
    elif n == 4:
        m0 = f"s_add_u32 m0, {sr(sSB)}, {sr(sK5)}"
        base = sKA
    else:
        m0 = f"s_add_u32 m0, {sr(sSBV)}, {4 * (n - 5) * 1024}"
        base = sVA
    return [Ins(m0, "salu", ("m0",)),
            Ins(f"global_load_lds_dwordx4 {vr(VDMA[n])}, {sr(base, 2)}", "vmem", (),
                (f"v{VDMA[n]}", "m0"))]


def dma_k():
    return [i for n in range(5) for i in dma(n)]


def dma_v():
    return [i for n in range(5, 10) for i in dma(n)]


def k_bases(tile_sreg, stage):
    """sKA = global base of K tile `tile_sreg`; sSB = its stage's base."""
    return [salu(f"s_lshl_b32 {sr(sTMP)}, {sr(tile_sreg)}, {TILE_BYTES.bit_length() - 1}"),
            salu(f"s_add_u32 {sr(sKA)}, {sr(sKH)}, {sr(sTMP)}"),
            salu(f"s_addc_u32 {sr(sKA + 1)}, {sr(sKH + 1)}, 0"),
            salu(f"s_add_u32 {sr(sSB)}, {sr(sWB)}, {stage * K_STAGE}")]


def v_bases(tile_sreg, stage):
    """sVA = global base of V tile `tile_sreg`; sSBV = its stage's base."""
    return [salu(f"s_lshl_b32 {sr(sTMP)}, {sr(tile_sreg)}, {TILE_BYTES.bit_length() - 1}"),
            salu(f"s_add_u32 {sr(sVA)}, {sr(sVH)}, {sr(sTMP)}"),
            salu(f"s_addc_u32 {sr(sVA + 1)}, {sr(sVH + 1)}, 0"),
            salu(f"s_add_u32 {sr(sSBV)}, {sr(sWB)}, {V_RING + stage * V_STAGE}")]


def clamp_offsets(slots):
    """Copy rows clamped to the last valid key (the final tile)."""
    return [valu(f"v_mov_b32 {vr(VDMA[i])}, {vr(VDMAL[i])}", (f"v{VDMA[i]}",),
                 (f"v{VDMAL[i]}",)) for i in slots]


def tile_index(dst, ahead):
    """dst = min(t + ahead, last); SCC = (dst == last)."""
    return [salu(f"s_add_u32 {sr(sT3)}, {sr(sT)}, {ahead}"),
            salu(f"s_min_u32 {sr(dst)}, {sr(sT3)}, {sr(sLAST)}"),
            salu(f"s_cmp_eq_u32 {sr(dst)}, {sr(sLAST)}")]


def exp_group(buf, qb, c, half, lset, tmp):
    """Exponentials of keys 8c' + 4*half .. +3 pairs of chunk c (c = 2 kb +
    c') for query block qb: p = 2^(s*c - m) in four temporaries (S stays
    intact), two packed bf16 pairs of P[qb][c], and their row sums added to
    chain set lset (the first chunk starts from the other set)."""
    kb, cp = c // 2, c % 2
    base = S(buf, kb, qb) + cp * 8
    out = []
    pairs = [half * 2, half * 2 + 1]
    srcs = [base + 2 * j + e for j in pairs for e in range(2)]
    for s_, t in zip(srcs, tmp):
        out.append(valu(f"v_fma_f32 {vr(t)}, {vr(s_)}, {sr(sC)}, -{vr(VM[qb])}",
                        (f"v{t}",), (f"v{s_}", f"v{VM[qb]}")))
    for t in tmp:
        out.append(valu(f"v_exp_f32 {vr(t)}, {vr(t)}", (f"v{t}",), (f"v{t}",), "trans"))
    for k, j in enumerate(pairs):
        pr = P(qb, c) + j
        a, b = tmp[2 * k], tmp[2 * k + 1]
        out.append(valu(f"v_cvt_pk_bf16_f32 {vr(pr)}, {vr(a)}, {vr(b)}", (f"v{pr}",),
                        (f"v{a}", f"v{b}")))
    for j in pairs:
        pr = P(qb, c) + j
        lr = VL[lset][qb][j % 2]
        src = VL[1 - lset][qb][j % 2] if (c == 0 and half == 0) else lr
        out.append(valu(f"v_dot2_f32_bf16 {vr(lr)}, {vr(pr)}, {vr(VONES)}, {vr(src)}",
                        (f"v{lr}",), (f"v{pr}", f"v{VONES}", f"v{src}")))
    return out


def exp_chunk(buf, c, lset):
    """The exponentials of chunk c of S(buf), both query blocks: the two
    halves of a block merged stage by stage (fma, exp, cvt, dot2), each with
    its own four temporaries."""
    out = []
    for qb in range(2):
        a = exp_group(buf, qb, c, 0, lset, VT[0:4])
        b = exp_group(buf, qb, c, 1, lset, VT[4:8])
        for lo, hi in ((0, 4), (4, 8), (8, 10), (10, 12)):
            out += a[lo:hi] + b[lo:hi]
    return out


def max_ops(buf, qb, tmp, chain_tmps):
    """Row maximum of S(buf)[*][qb] over the lane's 32 keys (four chains of
    8 joined), then over the partner lane (l ^ 32), in raw score units:
    result in v[tmp] (v[tmp+1] and chain_tmps clobbered)."""
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

    dsts = [m, f"v{tmp + 1}"] + [f"v{x}" for x in chain_tmps]
    parts = [chain(d, vals[8 * i:8 * i + 8]) for i, d in enumerate(dsts)]
    out = [ins for grp in zip(*parts) for ins in grp]
    out.append(valu(f"v_max3_f32 {m}, {dsts[0]}, {dsts[1]}, {dsts[2]}", (m,), tuple(dsts[:3])))
    out.append(valu(f"v_max_f32 {m}, {m}, {dsts[3]}", (m,), (m, dsts[3])))
    out += cross_max(tmp)
    return out


def cross_max(tmp):
    """v[tmp] = max of v[tmp] over the lane and its partner (l ^ 32), the
    other half of the same query column (v[tmp+1] is clobbered)."""
    m, t2 = f"v{tmp}", f"v{tmp + 1}"
    return [valu(f"v_mov_b32 {t2}, {m}", (t2,), (m,)),
            valu(f"v_permlane32_swap_b32 {m}, {t2}", (m, t2), (m, t2), "perm"),
            valu(f"v_max_f32 {m}, {m}, {t2}", (m,), (m, t2))]


def sum_check(lset, tag):
    """Branch to `tag` when any lane's row-sum chain of set lset passed 2^31
    (a NaN sum never does)."""
    (a, b), (c, d) = VL[lset]
    t = VT[0]
    return [valu(f"v_max3_f32 {vr(t)}, {vr(a)}, {vr(b)}, {vr(c)}", (f"v{t}",),
                 (f"v{a}", f"v{b}", f"v{c}")),
            valu(f"v_max_f32 {vr(t)}, {vr(t)}, {vr(d)}", (f"v{t}",), (f"v{t}", f"v{d}")),
            valu(f"v_cmp_lt_f32_e64 {sr(sN0, 2)}, {sr(sLIM)}, {vr(t)}", (f"s{sN0}",),
                 (f"v{t}",)),
            salu(f"s_cmp_lg_u64 {sr(sN0, 2)}, 0"),
            branch(f"s_cbranch_scc1 {tag}", tag)]


def rescale_block(buf, lset, tag, back):
    """A tile whose probabilities summed past 2^31 in some lane: per query
    block, m' = max(m, c * rowmax(S(buf)), m + log2(row sum before the tile)
    - 8) (taken across the lane pair, so both halves of a row agree), the
    sums before the tile and O scaled by 2^(m - m'), and the tile's
    probabilities and sums recomputed with m'.  Afterwards every p of the
    tile is <= 1 and the sums are below 2^8 + 64.  S(buf) is then free and
    buffers O."""
    out = [label(tag)]
    prev = 1 - lset
    for qb in range(2):
        mx, t1, t2, t3, al = VT[0], VT[1], VT[2], VT[3], VT[4]
        out += max_ops(buf, qb, mx, (t2, t3))
        (la, lb) = VL[prev][qb]
        out += [valu(f"v_mul_f32 {vr(mx)}, {sr(sC)}, {vr(mx)}", (f"v{mx}",), (f"v{mx}",)),
                valu(f"v_max_f32 {vr(mx)}, {vr(mx)}, {vr(VM[qb])}", (f"v{mx}",),
                     (f"v{mx}", f"v{VM[qb]}")),
                valu(f"v_add_f32 {vr(t2)}, {vr(la)}, {vr(lb)}", (f"v{t2}",), (f"v{la}", f"v{lb}")),
                valu(f"v_log_f32 {vr(t2)}, {vr(t2)}", (f"v{t2}",), (f"v{t2}",), "trans"),
                valu(f"v_add_f32 {vr(t2)}, {vr(t2)}, {vr(VM[qb])}", (f"v{t2}",),
                     (f"v{t2}", f"v{VM[qb]}")),
                valu(f"v_add_f32 {vr(t2)}, 0xc1000000, {vr(t2)}", (f"v{t2}",), (f"v{t2}",)),
                valu(f"v_max_f32 {vr(mx)}, {vr(mx)}, {vr(t2)}", (f"v{mx}",), (f"v{mx}", f"v{t2}"))]
        out += cross_max(mx)
        out += [valu(f"v_sub_f32 {vr(al)}, {vr(VM[qb])}, {vr(mx)}", (f"v{al}",),
                     (f"v{VM[qb]}", f"v{mx}")),
                valu(f"v_exp_f32 {vr(al)}, {vr(al)}", (f"v{al}",), (f"v{al}",), "trans"),
                valu(f"v_mov_b32 {vr(VM[qb])}, {vr(mx)}", (f"v{VM[qb]}",), (f"v{mx}",)),
                valu(f"v_mul_f32 {vr(la)}, {vr(la)}, {vr(al)}", (f"v{la}",), (f"v{la}", f"v{al}")),
                valu(f"v_mul_f32 {vr(lb)}, {vr(lb)}, {vr(al)}", (f"v{lb}",), (f"v{lb}", f"v{al}"))]
        out.append(valu(f"v_mov_b32 {vr(VA[qb])}, {vr(al)}", (f"v{VA[qb]}",), (f"v{al}",)))
    # the tile's probabilities again, with the new maximum
    for c in range(4):
        out += exp_chunk(buf, c, lset)
    # O *= alpha, 64 accumulators at a time through S(buf)
    tmp = S(buf, 0, 0)
    for qb in range(2):
        al = VA[qb]
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
    out.append(branch(f"s_branch {back}", back))
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
    """O += V^T P^T, chunk by chunk of 16 keys; each V^T fragment feeds two
    consecutive products."""
    out = []
    for c in range(4):
        for db in range(4):
            for qb in range(2):
                g = c * 4 + db
                out.append(mfma(("a", O(db, qb)), ("v", VF(g)), ("v", P(qb, c)),
                                ("a", O(db, qb))))
    return out


KR_AHEAD = 2.5      # gaps between a K fragment's read and its first product
VR_AHEAD = 3.0      # the same for V^T fragments (ring of 4: at most 6)


def k_read_items(stage, base, frags):
    """K fragment f feeds QK products base + 2f and base + 2f + 1; its ring
    slot was last read by product base + 2f - 7."""
    return [(base + 2 * f - KR_AHEAD, ins) for f in frags for ins in k_read(f, stage)]


def v_read_items(stage, base, frags):
    """V^T fragment g feeds PV products base + 2g and base + 2g + 1; its
    ring slot was last read by product base + 2g - 7."""
    out = []
    for g in frags:
        for j, ins in enumerate(v_read(g, stage)):
            out.append((base + 2 * g - VR_AHEAD + 0.1 * j, ins))
    return out


def exp_items(buf, lset, windows):
    """The exponentials of S(buf), chunk c spread over windows[c]."""
    out = []
    for c in range(4):
        out += spread(exp_chunk(buf, c, lset), *windows[c])
    return out


# chunk c of the next tile's P may be written once the products reading the
# current P[c] (8c .. 8c+7) have issued
MID_EXP = [(8 + 14 * c, 22 + 14 * c) for c in range(4)]
LAST_EXP = [(8 * c + 6, 8 * c + 14) for c in range(4)]
FIRST_EXP = [(8 * c, 8 * c + 8) for c in range(4)]


def mask_body(buf, rows):
    """Scores of keys at or past `rows` (a scalar register) -> -inf."""
    out = [valu(f"v_mov_b32 {vr(VT[7])}, 0xff800000", (f"v{VT[7]}",), ())]
    for kb in range(2):
        for r in range(16):
            key = kb * 32 + 16 * (r // 8) + r % 8
            t = VT[6]
            out += [valu(f"v_add_u32 {vr(t)}, {key}, {vr(VKH8)}", (f"v{t}",), (f"v{VKH8}",)),
                    valu(f"v_cmp_le_i32_e32 vcc, {sr(rows)}, {vr(t)}", ("vcc",), (f"v{t}",))]
            for qb in range(2):
                x = S(buf, kb, qb) + r
                out.append(valu(f"v_cndmask_b32_e32 {vr(x)}, {vr(x)}, {vr(VT[7])}, vcc",
                                (f"v{x}",), (f"v{x}", f"v{VT[7]}", "vcc")))
    return out


def mask_check(buf, slot, tag):
    """List mode: branch to a cold mask of S(buf) when the tile in `slot`
    is ragged.  Returns (hot, cold)."""
    hot = [salu(f"s_cmp_lt_u32 {sr(sQR[slot])}, {BN}"),
           branch(f"s_cbranch_scc1 {tag}_mk", f"{tag}_mk"), label(f"{tag}_mkr")]
    cold = [label(f"{tag}_mk")] + mask_body(buf, sQR[slot]) + \
        [branch(f"s_branch {tag}_mkr", f"{tag}_mkr")]
    return hot, cold


def mask_tail(buf, tag):
    """Scores of keys at or past the valid count -> -inf (the final tile,
    when it is partial)."""
    tag = f"{tag}_nomask"
    out = [salu(f"s_cmp_lt_u32 {sr(sREM)}, {BN}"),
           branch(f"s_cbranch_scc0 {tag}", tag),
           valu(f"v_mov_b32 {vr(VT[7])}, 0xff800000", (f"v{VT[7]}",), ())]
    for kb in range(2):
        for r in range(16):
            key = kb * 32 + 16 * (r // 8) + r % 8
            t = VT[6]
            out += [valu(f"v_add_u32 {vr(t)}, {key}, {vr(VKH8)}", (f"v{t}",), (f"v{VKH8}",)),
                    valu(f"v_cmp_le_i32_e32 vcc, {sr(sREM)}, {vr(t)}", ("vcc",), (f"v{t}",))]
            for qb in range(2):
                x = S(buf, kb, qb) + r
                out.append(valu(f"v_cndmask_b32_e32 {vr(x)}, {vr(x)}, {vr(VT[7])}, vcc",
                                (f"v{x}",), (f"v{x}", f"v{VT[7]}", "vcc")))
    out.append(label(tag))
    return out


def step_head(tag, kstage, vstage):
    """Copy targets of the step: K tile min(t+3, last) and V tile min(t+2,
    last) (rows clamped once a tile is the last), their stage bases."""
    return (tile_index(sTILE, 3) +
            [branch(f"s_cbranch_scc1 {tag}_swk", f"{tag}_swk"), label(f"{tag}_swkr")] +
            tile_index(sTV, 2) +
            [branch(f"s_cbranch_scc1 {tag}_swv", f"{tag}_swv"), label(f"{tag}_swvr")] +
            k_bases(sTILE, kstage) + v_bases(sTV, vstage))


def head_cold(tag):
    return ([label(f"{tag}_swk")] + clamp_offsets(range(5)) +
            [branch(f"s_branch {tag}_swkr", f"{tag}_swkr"), label(f"{tag}_swv")] +
            clamp_offsets(range(5, 10)) + [branch(f"s_branch {tag}_swvr", f"{tag}_swvr")])


def tab_read():
    """List mode: read the next table entry (the address advances first)."""
    return [valu(f"v_add_u32 {vr(VTA)}, 8, {vr(VTA)}", (f"v{VTA}",), (f"v{VTA}",)),
            ds_read(f"ds_read_b64 {vr(VTAB[0], 2)}, {vr(VTA)}", vset(VTAB[0], 2))]


def tab_take(slot):
    """List mode: the entry read a step ahead into queue slot `slot` (five
    wait states before a scalar instruction reads what v_readfirstlane
    wrote)."""
    return [valu(f"v_readfirstlane_b32 {sr(sQK[slot])}, {vr(VTAB[0])}", (), (f"v{VTAB[0]}",)),
            valu(f"v_readfirstlane_b32 {sr(sQR[slot])}, {vr(VTAB[1])}", (), (f"v{VTAB[1]}",)),
            Ins("s_nop 4", "nop")]


def list_bases(slot, kind, stage):
    base, dst, sb, ring = ((sKH, sKA, sSB, 0) if kind == "k" else
                           (sVH, sVA, sSBV, V_RING))
    size = K_STAGE if kind == "k" else V_STAGE
    return [salu(f"s_lshl_b32 {sr(sTMP)}, {sr(sQK[slot])}, {(2 * D).bit_length() - 1}"),
            salu(f"s_add_u32 {sr(dst)}, {sr(base)}, {sr(sTMP)}"),
            salu(f"s_addc_u32 {sr(dst + 1)}, {sr(base + 1)}, 0"),
            salu(f"s_add_u32 {sr(sb)}, {sr(sWB)}, {ring + stage * size}")]


def list_clamp(slots, rows):
    """Copy offsets of `slots` from the full ones with rows clamped to
    rows - 1: offset = min(row, rows - 1) * 256 + column."""
    t, c = VT[6], VT[7]
    out = [salu(f"s_sub_u32 {sr(sTMP)}, {sr(rows)}, 1")]
    for i in slots:
        d, f = VDMA[i], VDMAL[i]
        out += [valu(f"v_lshrrev_b32 {vr(t)}, 8, {vr(f)}", (f"v{t}",), (f"v{f}",)),
                valu(f"v_min_u32 {vr(t)}, {sr(sTMP)}, {vr(t)}", (f"v{t}",), (f"v{t}",)),
                valu(f"v_and_b32 {vr(c)}, 0xff, {vr(f)}", (f"v{c}",), (f"v{f}",)),
                valu(f"v_lshl_or_b32 {vr(d)}, {vr(t)}, 8, {vr(c)}", (f"v{d}",),
                     (f"v{t}", f"v{c}"))]
    return out


def list_copy_check(tag, kind, slot):
    """List mode: the copy offsets of K (bit 0) or V (bit 1) follow the
    tile in `slot`: clamped when it is ragged, restored after one that
    was.  Returns (hot, cold)."""
    bit = 0 if kind == "k" else 1
    slots = range(5) if kind == "k" else range(5, 10)
    t = f"{tag}_{kind}"
    hot = [salu(f"s_cmp_lt_u32 {sr(sQR[slot])}, {BN}"),
           branch(f"s_cbranch_scc1 {t}c", f"{t}c"),
           salu(f"s_bitcmp1_b32 {sr(sCL)}, {bit}"),
           branch(f"s_cbranch_scc1 {t}u", f"{t}u"),
           label(f"{t}r")]
    cold = ([label(f"{t}c")] + list_clamp(slots, sQR[slot]) +
            [salu(f"s_bitset1_b32 {sr(sCL)}, {bit}"), branch(f"s_branch {t}r", f"{t}r"),
             label(f"{t}u")] + clamp_offsets(slots) +
            [salu(f"s_bitset0_b32 {sr(sCL)}, {bit}"), branch(f"s_branch {t}r", f"{t}r")])
    return hot, cold


def list_head(tag, phi, kstage, vstage, cur):
    """List mode step head: take the entry of tile t+3, bases and copy
    offsets of K(t+3) and V(t+2), mask S(t) if tile t is ragged."""
    ks, vs, ms = (phi + 3) % NS, (phi + 2) % NS, phi % NS
    hot = tab_take(ks)
    kh, kc = list_copy_check(tag, "k", ks)
    vh, vc = list_copy_check(tag, "v", vs)
    mh, mc = mask_check(cur, ms, tag)
    hot += kh + list_bases(ks, "k", kstage) + vh + list_bases(vs, "v", vstage) + mh
    return hot, kc + vc + mc


def gather_load(ahead, slot):
    """Gather mode: load the indices of tile min(t + ahead, last) into
    VIDX[slot], lanes past a short final tile clamped to its last row."""
    return tile_index(sTL, ahead) + [
        salu(f"s_cselect_b32 {sr(sILIM)}, {sr(sRL4)}, 0xfc"),   # (SCC: the last tile)
        salu(f"s_lshl_b32 {sr(sTMP)}, {sr(sTL)}, 8"),
        salu(f"s_add_u32 {sr(sLA)}, {sr(sLST)}, {sr(sTMP)}"),
        salu(f"s_addc_u32 {sr(sLA + 1)}, {sr(sLST + 1)}, 0"),
        valu(f"v_min_u32 {vr(VGT)}, {sr(sILIM)}, {vr(VLANE4)}", (f"v{VGT}",), (f"v{VLANE4}",)),
        Ins(f"global_load_dword {vr(VIDX[slot])}, {vr(VGT)}, {sr(sLA, 2)}", "vmem",
            (f"v{VIDX[slot]}",), (f"v{VGT}",))]


def gather_shift(slot):
    """Indices clamped to the cache's rows, then to byte offsets of rows."""
    x = vr(VIDX[slot])
    return [valu(f"v_min_u32 {x}, {sr(sCAPM1)}, {x}", (f"v{VIDX[slot]}",), (f"v{VIDX[slot]}",)),
            valu(f"v_lshlrev_b32 {x}, 8, {x}", (f"v{VIDX[slot]}",), (f"v{VIDX[slot]}",))]


def gather_offsets(slots, src):
    """Per-lane copy offsets of `slots` from the shifted index vector
    VIDX[src]: (bpermute, or) pairs, one pair per slot."""
    out = []
    for n in slots:
        out.append([ds_read(f"ds_bpermute_b32 {vr(VDMA[n])}, {vr(VDMAL[n])}, {vr(VIDX[src])}",
                            (f"v{VDMA[n]}",)),
                    valu(f"v_or_b32_sdwa {vr(VDMA[n])}, {vr(VDMA[n])}, {vr(VCOL[n // 4])} "
                         f"dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
                         f"src1_sel:BYTE_{n % 4}", (f"v{VDMA[n]}",),
                         (f"v{VDMA[n]}", f"v{VCOL[n // 4]}"))])
    return out


def gather_head(tag, phi, kstage, vstage):
    """Gather mode step head: the index load of tile t+4 (first of the
    step's vector-memory operations, so the step's closing vmcnt wait covers
    it), the shift of tile t+3's indices, the stage bases of K(t+3) and
    V(t+2).  The copy offsets follow as items (gather_items)."""
    return (gather_load(4, phi % NS) + gather_shift((phi + 3) % NS) +
            [salu(f"s_add_u32 {sr(sSB)}, {sr(sWB)}, {kstage * K_STAGE}"),
             salu(f"s_add_u32 {sr(sSBV)}, {sr(sWB)}, {V_RING + vstage * V_STAGE}")])


def gather_items(phi, lo):
    """The offsets of copy slot n placed two gaps before its copy (dma_items
    puts copy n at gap lo + 2n)."""
    items = []
    pairs = gather_offsets(range(5), (phi + 3) % NS) + gather_offsets(range(5, 10), (phi + 2) % NS)
    for n, (bp, orr) in enumerate(pairs):
        items += [(max(lo - 1, lo + 2 * n - 2) - 0.5, bp), (lo + 2 * n - 0.2, orr)]
    return items


def end_of_step(n_mf, vstage_next):
    """Before the last two products: every LDS read of the step is back,
    the tiles copied before this step have landed, every wave is past its
    reads; then the first V^T fragments of the next step's product."""
    items = [(n_mf - 1.5, Ins("s_waitcnt lgkmcnt(0)", "wait")),
             (n_mf - 1.4, Ins("s_waitcnt vmcnt(10)", "wait")),
             (n_mf - 1.3, Ins("s_barrier", "barrier"))]
    items += [(n_mf - 1.2 + 0.01 * g, ins) for g in range(2) for ins in v_read(g, vstage_next)]
    if LIST:   # before the fragment reads, so the next head waits for it alone
        items += [(n_mf - 1.25 + 0.01 * k, ins) for k, ins in enumerate(tab_read())]
    return items


def dma_items(lo, hi):
    ins = dma_k() + dma_v()
    return [(lo + (hi - lo) * (k // 2) / 10 + 0.01 * (k % 2), i) for k, i in enumerate(ins)]


def first_step():
    """t = first tile: S(t+1) = K(t+1) Q^T and the exponentials of S(t);
    no product with V yet."""
    tag = "crt_first"
    if LIST:
        hh, lcold = list_head(tag, 0, 3, 2, 0)
        head = [label(tag)] + hh
    elif GATHER:
        head = [label(tag)] + gather_head(tag, 0, 3, 2)
    else:
        head = [label(tag)] + step_head(tag, 3, 2)
    items = k_read_items(1, 0, range(16)) + dma_items(0, 20) + exp_items(0, 0, FIRST_EXP)
    if GATHER:
        items += gather_items(0, 0)
    items += end_of_step(32, 0)
    body = place(qk_mfmas(1), items, head)
    tail = sum_check(0, f"{tag}_resc") + [label(f"{tag}_rescr"),
                                         salu(f"s_add_u32 {sr(sT)}, {sr(sT)}, 1"),
                                         branch("s_branch crt_ph1", "crt_ph1")]
    cold = (lcold if LIST else [] if GATHER else head_cold(tag)) + \
        rescale_block(0, 0, f"{tag}_resc", f"{tag}_rescr")
    return body + tail, cold


def step(phi):
    """Main step of phase phi (tile t = first + phi mod 4): O += P(t-1)
    V(t-1), then S(t+1) = K(t+1) Q^T, the exponentials of S(t) beside
    both, the copies of K(t+3) and V(t+2)."""
    cur, nxt, lset = phi % 2, 1 - phi % 2, phi % 2
    tag = f"crt_ph{phi}"
    head = [label(tag), salu(f"s_cmp_ge_u32 {sr(sT)}, {sr(sLAST)}"),
            branch(f"s_cbranch_scc1 crt_last{phi}", f"crt_last{phi}")]
    if LIST:
        hh, lcold = list_head(tag, phi, (phi + 3) % NS, (phi + 2) % NS, cur)
        head += hh
    elif GATHER:
        head += gather_head(tag, phi, (phi + 3) % NS, (phi + 2) % NS)
    else:
        head += step_head(tag, (phi + 3) % NS, (phi + 2) % NS)
    mf = pv_mfmas() + qk_mfmas(nxt)
    items = v_read_items((phi + 3) % NS, 0, range(2, 16))
    items += k_read_items((phi + 1) % NS, 32, range(16))
    items += dma_items(1, 21)
    if GATHER:
        items += gather_items(phi, 1)
    items += exp_items(cur, lset, MID_EXP)
    items += end_of_step(64, phi % NS)
    body = place(mf, items, head)
    tail = sum_check(lset, f"{tag}_resc") + [label(f"{tag}_rescr"),
                                            salu(f"s_add_u32 {sr(sT)}, {sr(sT)}, 1")]
    if phi == NS - 1:
        tail.append(branch("s_branch crt_ph0", "crt_ph0"))
    cold = (lcold if LIST else [] if GATHER else head_cold(tag)) + \
        rescale_block(cur, lset, f"{tag}_resc", f"{tag}_rescr")
    return body + tail, cold


def drain(vstage, tag):
    """O += P(last) V(last): the products of the final tile."""
    body = place(pv_mfmas(), v_read_items(vstage, 0, range(16)), [label(tag)])
    return body + [branch("s_branch crt_end", "crt_end")]


def last_step(phi):
    """t = last (after the first): O += P(t-1) V(t-1) beside the
    exponentials of the (masked) final tile, then its own products."""
    cur, lset = phi % 2, phi % 2
    tag = f"crt_last{phi}"
    mcold = []
    if LIST:
        mh, mcold = mask_check(cur, phi % NS, tag)
        head = [label(tag)] + mh
    else:
        head = [label(tag)] + mask_tail(cur, tag)
    items = v_read_items((phi + 3) % NS, 0, range(2, 16)) + exp_items(cur, lset, LAST_EXP)
    body = place(pv_mfmas(), items, head)
    tail = sum_check(lset, f"{tag}_resc") + [label(f"{tag}_rescr")]
    if lset == 1:   # the row sums leave the loop in set 0
        for qb in range(2):
            for ch in range(2):
                d, s_ = VL[0][qb][ch], VL[1][qb][ch]
                tail.append(valu(f"v_mov_b32 {vr(d)}, {vr(s_)}", (f"v{d}",), (f"v{s_}",)))
    check_p_war(body, f"last {phi}")
    tail += drain(phi % NS, f"{tag}_drain")
    cold = mcold + rescale_block(cur, lset, f"{tag}_resc", f"{tag}_rescr")
    return body + tail, cold


def only_step():
    """The first tile is also the last: its exponentials, then its products."""
    tag = "crt_only"
    mcold = []
    if LIST:
        mh, mcold = mask_check(0, 0, tag)
        body = [label(tag)] + mh
    else:
        body = [label(tag)] + mask_tail(0, tag)
    for c in range(4):
        body += exp_chunk(0, c, 0)
    body += sum_check(0, f"{tag}_resc") + [label(f"{tag}_rescr")]
    body += drain(0, f"{tag}_drain")
    cold = mcold + rescale_block(0, 0, f"{tag}_resc", f"{tag}_rescr")
    return body, cold


def prologue():
    out = [Ins("s_nop 7", "nop"),
           valu(f"v_mov_b32 {vr(VONES)}, 0x3f803f80", (f"v{VONES}",), ()),
           salu(f"s_mov_b32 {sr(sLIM)}, {SUM_LIMIT:#x}")]
    for st in range(2):
        for qb in range(2):
            for ch in range(2):
                r = VL[st][qb][ch]
                out.append(valu(f"v_mov_b32 {vr(r)}, 0", (f"v{r}",), ()))
    # K(t), K(t+1), V(t), K(t+2), V(t+1) (tiles clamped to the last) into
    # K stages 0, 1, 2 and V stages 0, 1
    parts = [("k", 0, 0), ("k", 1, 1), ("v", 0, 0), ("k", 2, 2), ("v", 1, 1)]
    if LIST:
        # entries 0..2 into slots 0..2, entry 3 left in flight for the first step
        out.append(valu(f"v_mov_b32 {vr(VTA)}, {sr(sTAB)}", (f"v{VTA}",), ()))
        for j in range(3):
            if j:
                out += tab_read()
            else:
                out.append(ds_read(f"ds_read_b64 {vr(VTAB[0], 2)}, {vr(VTA)}", vset(VTAB[0], 2)))
            out += tab_take(j)
        out += tab_read()
        for kind, ahead, stage in parts:
            slots = range(5) if kind == "k" else range(5, 10)
            out += list_clamp(slots, sQR[ahead]) + list_bases(ahead, kind, stage)
            out += dma_k() if kind == "k" else dma_v()
        # clamped-offset flags after the last K part (tile 2) and V part (tile 1)
        out += [salu(f"s_cmp_lt_u32 {sr(sQR[2])}, {BN}"),
                salu(f"s_cselect_b32 {sr(sCL)}, 1, 0"),
                salu(f"s_cmp_lt_u32 {sr(sQR[1])}, {BN}"),
                salu(f"s_cselect_b32 {sr(sTMP)}, 2, 0"),
                salu(f"s_or_b32 {sr(sCL)}, {sr(sCL)}, {sr(sTMP)}")]
    if GATHER:
        # the copies read rows through their own offsets from the head bases;
        # the indices of tiles t .. t+2 shifted (t+3 is left for the first step)
        out += [salu(f"s_mov_b64 {sr(sKA, 2)}, {sr(sKH, 2)}"),
                salu(f"s_mov_b64 {sr(sVA, 2)}, {sr(sVH, 2)}"),
                salu(f"s_sub_u32 {sr(sRL4)}, {sr(sREM)}, 1"),
                salu(f"s_lshl_b32 {sr(sRL4)}, {sr(sRL4)}, 2")]
        # (the kernel loads the indices of tiles t .. t+3 into VIDX before
        # the loop, beside the queries)
        for j in range(3):
            out += gather_shift(j)
        for kind, ahead, stage in parts:
            slots = range(5) if kind == "k" else range(5, 10)
            pairs = gather_offsets(slots, ahead)
            out += [bp for bp, _ in pairs] + [orr for _, orr in pairs]
            if kind == "k":
                out.append(salu(f"s_add_u32 {sr(sSB)}, {sr(sWB)}, {stage * K_STAGE}"))
                out += dma_k()
            else:
                out.append(salu(f"s_add_u32 {sr(sSBV)}, {sr(sWB)}, {V_RING + stage * V_STAGE}"))
                out += dma_v()
    for i, (kind, ahead, stage) in enumerate(parts if not (LIST or GATHER) else []):
        dst = sTILE if kind == "k" else sTV
        out += tile_index(dst, ahead) + [branch(f"s_cbranch_scc0 crt_pro{i}", f"crt_pro{i}")]
        out += clamp_offsets(range(5) if kind == "k" else range(5, 10))
        out.append(label(f"crt_pro{i}"))
        out += (k_bases(dst, stage) + dma_k()) if kind == "k" else (v_bases(dst, stage) + dma_v())
    out += [Ins("s_waitcnt vmcnt(20)", "wait"), Ins("s_barrier", "barrier")]
    # S of the first tile into buffer 0, then its exact row maximum
    out = place(qk_mfmas(0), k_read_items(0, 0, range(16)), out)
    for qb in range(2):
        out += max_ops(0, qb, VT[2 * qb], (VT[4 + 2 * qb], VT[5 + 2 * qb]))
        out.append(valu(f"v_mul_f32 {vr(VM[qb])}, {sr(sC)}, {vr(VT[2 * qb])}", (f"v{VM[qb]}",),
                        (f"v{VT[2 * qb]}",)))
    # K(t+1) and V(t) have landed and are visible
    out += [Ins("s_waitcnt vmcnt(10)", "wait"), Ins("s_barrier", "barrier"),
            salu(f"s_cmp_ge_u32 {sr(sT)}, {sr(sLAST)}"),
            branch("s_cbranch_scc1 crt_only", "crt_only")]
    return out


def check_p_war(body, what):
    """No probability register may be rewritten before the products that
    read its previous value in the same block have issued."""
    written = set()
    for ins in body:
        if ins.kind == "valu" and ins.text.startswith("v_cvt_pk_bf16_f32"):
            written |= set(ins.dst)
        if ins.kind == "mfma" and ins.dst[0].startswith("a"):
            hit = [r for r in ins.src if r in written]
            if hit:
                raise RuntimeError(f"{what}: {ins.text} reads {hit} after they were rewritten")


def program():
    cold = []
    first, c = first_step()
    check_p_war(first, "first")
    cold += c
    main = []
    for phi in range(NS):
        b, c = step(phi)
        check_p_war(b, f"phase {phi}")
        main += b
        cold += c
    lasts = []
    for phi in range(NS):
        b, c = last_step(phi)
        lasts += b
        cold += c
    only, c = only_step()
    cold += c
    end = [label("crt_end"), Ins("s_waitcnt vmcnt(0) lgkmcnt(0)", "wait"),
           Ins("s_nop 7", "nop"), Ins("s_nop 7", "nop"), Ins("s_nop 7", "nop")]
    return prologue() + first + main + lasts + only + cold + end


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
        e = next(k for k, i in enumerate(prog) if i.text.startswith(f"s_add_u32 s{sT}, s{sT}, 1")
                 and k > s)
        seg = prog[s:e]
        n = sum(1 for i in seg if i.kind not in ("label",))
        nop = sum(ws_of(i) for i in seg if i.kind == "nop")
        waits = sum(1 for i in seg if i.kind == "wait")
        out.append((phi, n, nop, waits))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                  "attn_loop.inc"))
    ap.add_argument("--report", action="store_true")
    ap.add_argument("--kr-ahead", type=float, default=None, help="K fragment read distance")
    ap.add_argument("--vr-ahead", type=float, default=None, help="V fragment read distance")
    args = ap.parse_args()
    global KR_AHEAD, VR_AHEAD
    if args.kr_ahead is not None:
        KR_AHEAD = args.kr_ahead
    if args.vr_ahead is not None:
        VR_AHEAD = args.vr_ahead
    global LIST, GATHER
    text = ("// Generated by gen_attn_loop.py; do not edit.  The key loop of the\n"
            "// chunk-causal attention kernel (head_dim 128) in CDNA4 assembly, one\n"
            "// string each for an asm statement whose registers are fixed by its\n"
            "// operands and clobbers (see attn.hip): consecutive key tiles\n"
            "// (CRATTN_ATTN_LOOP_ASM), key tiles from a table of (first row, rows)\n"
            "// in LDS (CRATTN_ATTN_LOOP_LIST_ASM, the block-sparse instance) and key\n"
            "// rows from a list of row indices (CRATTN_ATTN_LOOP_GATHER_ASM, the\n"
            "// semantic-permutation instance).\n")
    progs = {}
    for LIST, GATHER, name in ((False, False, "CRATTN_ATTN_LOOP_ASM"),
                               (True, False, "CRATTN_ATTN_LOOP_LIST_ASM"),
                               (False, True, "CRATTN_ATTN_LOOP_GATHER_ASM")):
        prog = fix(program())
        progs[name] = prog
        lines = render(prog)
        text += (f"#define {name} \\\n" +
                 " \\\n".join(f'  "{ln}\\n"' for ln in lines) + "\n")
    prog = progs["CRATTN_ATTN_LOOP_ASM"]
    with open(args.out + ".tmp", "w") as f:
        f.write(text)
    os.replace(args.out + ".tmp", args.out)
    if args.report:
        print(stats(prog), len(prog), file=sys.stderr)
        for r in step_report(prog):
            print("phase %d: %d instructions, %d nop wait states, %d waits" % r, file=sys.stderr)


if __name__ == "__main__":
    main()
