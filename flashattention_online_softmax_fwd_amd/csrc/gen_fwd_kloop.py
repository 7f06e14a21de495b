#!/usr/bin/env python3
"""Generates fa_fwd_kloop.inc: the key loop of the 64-rows-per-wave forward as gfx950 assembly.

The forward of fa_fwd_w64.hip hands one wave 64 query rows (two 32-row blocks, rb 0 and 1) at
one wave per SIMD, so each K or V operand read from LDS feeds two matrix products.  The
whole per-workgroup computation after the setup is one inline-assembly statement built
here: the Q loads, the pipelined walk over 64-key tiles, the rare rescale of the output
accumulators, and the stores of O and LSE.  Writing it out lets the output accumulators
stay in AGPRs for the whole walk (only the rare rescale touches them outside the matrix
products) and lets every matrix product sit between the vector work of the softmax and
the LDS reads of the next operands.

The method is the pages' online softmax in base 2 with the kernel's lazy reference (see
fa_fwd_w64.hip).  Per 32-key half-tile h of a wave:
    S(h+1) = K Q^T        (the next half's scores, 16 products)
    O     += V^T P(h-1)   (the previous half's weighted values, 16 products)
    softmax(h) on the scores of this half: row max, lazy reference move, P = exp2(S c - m),
                          row sums, P rounded to the element type
The scores of half h+1 are therefore computed while half h's exponentials run, and the
values of half h-1 are added while half h's row maxima are formed.

Register plan (fixed, named by the clobber list of the statement):
    v0..v63     Q, rb * 32 + kk * 4 (kk = 16-dim step)
    v64..v127   S, two buffers of two row blocks
    v128..v159  P, two buffers, [rb][ks] (ks = 16-key step)
    v160..v175  K operand staging (4), v176..v191 V operand staging (4)
    v192..v199  m, l, alpha[parity][rb]
    v200..v223  temporaries
    a0..a127    O, [rb][db] (db = 32-dim block)
Everything the hardware does not interlock is spaced by this generator: it tracks the
producer of every register and inserts s_nop for the wait states the CDNA3/CDNA4 hazard
rules require (matrix result -> vector use, vector result -> matrix operand,
transcendental -> use, lane-mask write -> use, M0 write -> LDS DMA), and s_waitcnt
lgkmcnt for LDS reads still in flight when their destination is used.

Run:  python gen_fwd_kloop.py      (writes fa_fwd_kloop.inc next to this file)
"""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.environ.get("OUT_INC") or os.path.join(HERE, "fa_fwd_kloop.inc")

NEG_INF_BITS = "0xff800000"

# Head dimension of the variant being assembled (64 or 128); set by assemble().
D = 128


def KK():
    """16-dim steps of the score products (Q operand registers per row block / 4)."""
    return D // 16


def DB():
    """32-dim column blocks of O."""
    return D // 32


def ROWB():
    """Bytes of one K, V, Q or O row."""
    return 2 * D


def TILE():
    """Bytes of one 64-key K or V tile in LDS (buffers at 0, TILE, 2 TILE, 3 TILE)."""
    return 64 * ROWB()

# ---------------------------------------------------------------- registers

def vr(i):
    return "v%d" % i


def vrange(a, n):
    return "v[%d:%d]" % (a, a + n - 1)


# Register plan (see the module docstring).
PLAN = dict(Q0=0, S0=64, P0=128, KST0=160, VST0=176, M0=192)
TMP0 = 200           # v200..v223
NTMP = 24
NEGINF = 223         # holds -inf for lane-mask selects
NVCLOB = 224         # v0..v223 clobbered


def Qr(rb, kk):
    return PLAN["Q0"] + 4 * KK() * rb + 4 * kk


def Sr(buf, rb):
    return PLAN["S0"] + 32 * buf + 16 * rb


def Pr(buf, rb, ks):
    return PLAN["P0"] + 16 * buf + 8 * rb + 4 * ks


def KST(i):
    return PLAN["KST0"] + 4 * i


def VST(i):
    return PLAN["VST0"] + 4 * i


def Mr(rb):
    return PLAN["M0"] + rb


def Lr(rb):
    return PLAN["M0"] + 2 + rb


def ALr(par, rb):
    return PLAN["M0"] + 4 + 2 * par + rb


def Or(rb, db):
    """First AGPR of O's 32 x 32 block db of row block rb."""
    return 16 * DB() * rb + 16 * db


# Row sums: "valu" adds the fp32 P with vector adds (the default); "mfma16" adds the rounded
# P with one 16x16x32 product per 16 keys and row block, whose 0/1 A operand makes every
# lane's four results the sum over both lane halves of the lane's own row (see ones16), so l
# sits in AGPRs beside O.  Measured equal on the causal d = 128 workloads (64 vector adds per
# tile traded for 8 small products); an all-ones 32x32x16 product instead was 2-5% slower.
# Per head dimension (FA_GEN_ROWSUM for d = 128, FA_GEN_ROWSUM64 for d = 64).
ROWSUM_BY_D = {128: os.environ.get("FA_GEN_ROWSUM", "valu"), 64: os.environ.get("FA_GEN_ROWSUM64", "valu")}
for _r in ROWSUM_BY_D.values():
    if _r not in ("valu", "mfma16"):
        raise SystemExit("FA_GEN_ROWSUM and FA_GEN_ROWSUM64 must be valu or mfma16")
ROWSUM = ROWSUM_BY_D[128]
ONES = 216           # v216..v219: the 0/1 A operand of the row-sum products
MFMA_ROWSUM = ROWSUM == "mfma16"
LACC_REGS = 4


def Lacc(rb):
    """AGPRs of the row-sum product of row block rb (every register holds l of the lane's row)."""
    return 128 + LACC_REGS * rb


# ---------------------------------------------------------------- instructions

class Ins:
    """One instruction with the registers it reads and writes (for the hazard and
    waitcnt passes).  kind: mfma, valu, trans, perm, cmps (VALU writing an SGPR mask),
    accr, accw, salu, m0 (SALU writing M0), lds (LDS read), dma (LDS DMA load),
    vload, vstore, barrier, wait, nop, branch, label."""

    __slots__ = ("text", "kind", "defs", "uses", "srcc")

    def __init__(self, text, kind, defs=(), uses=(), srcc=None):
        self.text = text
        self.kind = kind
        self.defs = tuple(defs)
        self.uses = tuple(uses)
        self.srcc = srcc


def regs(a, n, prefix="v"):
    return ["%s%d" % (prefix, a + i) for i in range(n)]


class Skip:
    """A forward branch over ``body`` when the 64-bit SGPR operand ``flag`` is zero."""

    def __init__(self, flag, body, label):
        self.flag = flag
        self.body = body
        self.label = label


class Loop:
    """``body`` repeated while the SGPR operand ``counter`` (decremented at the end) is
    non-zero; entered only when it is non-zero."""

    def __init__(self, counter, body, label):
        self.counter = counter
        self.body = body
        self.label = label


class Cond:
    """``body`` run only when SCC (set by ``test``, a list of SALU texts) is 1."""

    def __init__(self, test, body, label):
        self.test = test
        self.body = body
        self.label = label


# ---------------------------------------------------------------- hazard rules

MFMA_WAIT = 20    # matrix result -> any other access of that register (>= passes + 3)


def required_wait(wkind, rkind, reg_role):
    """Wait states needed between a writer of kind ``wkind`` and a later instruction of
    kind ``rkind`` touching the same register in role ``reg_role`` ('use', 'def', 'srcc')."""
    if wkind == "mfma":
        if rkind == "mfma":
            return 0 if reg_role == "srcc" else MFMA_WAIT
        return MFMA_WAIT
    if rkind == "mfma":
        if wkind in ("valu", "trans", "perm", "accw", "cmps"):
            return 3
        return 0
    if wkind == "trans" and rkind in ("valu", "trans", "perm", "cmps", "accw", "vstore"):
        return 2
    if rkind == "perm" and wkind in ("valu", "trans", "cmps"):
        return 2
    if wkind == "perm" and rkind in ("valu", "trans", "cmps", "perm"):
        return 2
    if wkind == "cmps" and rkind in ("valu", "trans", "cmps"):
        return 2
    if wkind == "cmps" and rkind == "salu":
        return 4
    if wkind == "m0" and rkind == "dma":
        return 1
    if wkind == "accw" and rkind == "accr":
        return 1
    return 0


class State:
    def __init__(self):
        self.last = {}      # reg -> (position, kind)
        self.pos = 0        # wait states issued so far
        self.lds = []       # outstanding LDS reads: list of sets of destination regs (issue order)

    def copy(self):
        s = State()
        s.last = dict(self.last)
        s.pos = self.pos
        s.lds = [set(x) for x in self.lds]
        return s


def merge_states(a, b):
    """Join of two control-flow paths: the most recent writer of every register, and the
    LDS reads outstanding on either path (both paths must agree on LDS here)."""
    s = State()
    s.pos = max(a.pos, b.pos)
    for st in (a, b):
        for r, (p, k) in st.last.items():
            p2 = p + (s.pos - st.pos)
            if r not in s.last or p2 > s.last[r][0]:
                s.last[r] = (p2, k)
    s.lds = [set(x) for x in a.lds] if len(a.lds) >= len(b.lds) else [set(x) for x in b.lds]
    return s


def emit(ins, st, out):
    """Append ``ins`` to ``out`` after the waits it needs; update the state."""
    if ins.kind == "label":
        out.append(ins.text)
        return
    if ins.kind == "waitall":
        st.lds = []
    touched = [(r, "use") for r in ins.uses] + [(r, "def") for r in ins.defs]
    # LDS reads still in flight whose destination this instruction touches
    if st.lds:
        need = -1
        for i, dset in enumerate(st.lds):
            if any(r in dset for r, _ in touched):
                need = i
        if ins.kind in ("barrier",):
            need = len(st.lds) - 1
        if need >= 0:
            left = len(st.lds) - need - 1
            out.append("s_waitcnt lgkmcnt(%d)" % min(left, 15))
            st.pos += 1
            st.lds = st.lds[need + 1:]
    wait = 0
    for r, role in touched:
        if r not in st.last:
            continue
        p, k = st.last[r]
        rr = role
        if ins.kind == "mfma" and ins.srcc and r in ins.srcc:
            rr = "srcc"
        need = required_wait(k, ins.kind, rr)
        if need:
            wait = max(wait, need - (st.pos - p))
    while wait > 0:
        n = min(wait, 16)
        out.append("s_nop %d" % (n - 1))
        st.pos += n
        wait -= n
    out.append(ins.text)
    st.pos += 1
    if ins.kind == "lds":
        st.lds.append(set(ins.defs))
        if len(st.lds) > 15:
            raise RuntimeError("more than 15 LDS reads in flight")
    for r in ins.defs:
        st.last[r] = (st.pos - 1, ins.kind)


def lower(items, st, out, uid):
    """Lower a list of Ins / Skip / Loop / Cond into assembly lines."""
    for it in items:
        if isinstance(it, Ins):
            emit(it, st, out)
        elif isinstance(it, Skip):
            out.append("s_cmp_eq_u64 %s, 0" % it.flag)
            out.append("s_cbranch_scc1 %s_%s" % (it.label, uid))
            st.pos += 2
            before = st.copy()
            lower(it.body, st, out, uid)
            out.append("%s_%s:" % (it.label, uid))
            st2 = merge_states(before, st)
            st.last, st.pos, st.lds = st2.last, st2.pos, st2.lds
        elif isinstance(it, Cond):
            out.extend(it.test)
            out.append("s_cbranch_scc0 %s_%s" % (it.label, uid))
            st.pos += len(it.test) + 1
            before = st.copy()
            lower(it.body, st, out, uid)
            out.append("%s_%s:" % (it.label, uid))
            st2 = merge_states(before, st)
            st.last, st.pos, st.lds = st2.last, st2.pos, st2.lds
        elif isinstance(it, Loop):
            # the state at the loop head joins the entry with the end of the body: run the
            # body once to find its end state, then lower it for real from the join
            if st.lds:
                raise RuntimeError("LDS reads in flight at a loop head")
            trial = st.copy()
            lower(it.body, trial, [], uid)
            head = merge_states(st, trial)
            if head.lds:
                raise RuntimeError("LDS reads in flight at the end of a loop body")
            out.append("%s_%s:" % (it.label, uid))
            st.last, st.pos, st.lds = head.last, head.pos, head.lds
            lower(it.body, st, out, uid)
            out.append("s_sub_u32 %s, %s, 1" % (it.counter, it.counter))
            out.append("s_cmp_lg_u32 %s, 0" % it.counter)
            out.append("s_cbranch_scc1 %s_%s" % (it.label, uid))
            st.pos += 3
        else:
            raise TypeError(it)


# ---------------------------------------------------------------- building blocks

class Gen:
    def __init__(self, elem, causal):
        self.elem = elem            # "bf16" or "f16"
        self.kbuf = 0               # 1: operand reads go to the K / V buffer above the one
        self.vbuf = 0               #    %[koff] / %[voff] point at (the unrolled steady loop)
        self.causal = causal
        self.mfma_op = "v_mfma_f32_32x32x16_" + elem
        self.mfma16_op = "v_mfma_f32_16x16x32_" + elem
        # How far (log2 units) a row's maximum may rise above its reference before O, l
        # and the reference are rescaled.  P = exp2(S c - m) then stays below 2^slack: bf16
        # has float32's exponent range, so 2^48 is exact and O's float32 sums stay finite
        # while N * max|v| < 2^80; fp16 P must stay below 65504, hence 15.
        self.slack = "0x42400000" if elem == "bf16" else "0x41700000"     # 48.0, 15.0
        self.cvt_op = "v_cvt_pk_bf16_f32" if elem == "bf16" else "v_cvt_pk_f16_f32"

    # ---- operand reads from LDS
    def k_read(self, i, kk, t):
        """K operand for dims 16kk.. of keys 32t.. of the current K tile into staging i (the tile
        in the buffer %[koff] points at, or in the other one when self.kbuf is set)."""
        off = 32 * ROWB() * t + self.kbuf * TILE()
        return Ins("ds_read_b128 %s, %%[koff%d] offset:%d" % (vrange(KST(i), 4), kk, off), "lds",
                   defs=regs(KST(i), 4))

    def v_reads(self, i, db, ks, t):
        """V^T operand of dims 32db.. and keys 32t + 16ks.. (two transposing reads; self.vbuf as
        self.kbuf)."""
        off = 32 * ROWB() * t + 16 * ROWB() * ks + self.vbuf * TILE()
        return [Ins("ds_read_b64_tr_b16 %s, %%[voff%d] offset:%d" % (vrange(VST(i), 2), db, off), "lds",
                    defs=regs(VST(i), 2)),
                Ins("ds_read_b64_tr_b16 %s, %%[voff%d] offset:%d" % (vrange(VST(i) + 2, 2), DB() + db, off), "lds",
                    defs=regs(VST(i) + 2, 2))]

    def mfma_s(self, sbuf, rb, kk, st):
        d = Sr(sbuf, rb)
        src_c = "0" if kk == 0 else vrange(d, 16)
        uses = regs(KST(st), 4) + regs(Qr(rb, kk), 4) + ([] if kk == 0 else regs(d, 16))
        return Ins("%s %s, %s, %s, %s" % (self.mfma_op, vrange(d, 16), vrange(KST(st), 4), vrange(Qr(rb, kk), 4),
                                          src_c), "mfma", defs=regs(d, 16), uses=uses,
                   srcc=set(regs(d, 16)) if kk else None)

    def mfma_pv(self, pbuf, rb, db, ks, st):
        o = Or(rb, db)
        uses = regs(VST(st), 4) + regs(Pr(pbuf, rb, ks), 4) + regs(o, 16, "a")
        return Ins("%s a[%d:%d], %s, %s, a[%d:%d]" % (self.mfma_op, o, o + 15, vrange(VST(st), 4),
                                                      vrange(Pr(pbuf, rb, ks), 4), o, o + 15),
                   "mfma", defs=regs(o, 16, "a"), uses=uses, srcc=set(regs(o, 16, "a")))

    # ---- the product streams of one half: list of (reads, mfma) with staging slots
    def s_stream(self, sbuf, t, rbs):
        """S(h+1) into S buffer sbuf from K tile rows 32t..: per kk one K read feeding the
        products of every active row block."""
        out = []
        for kk in range(KK()):
            st = kk % 4
            prods = [self.mfma_s(sbuf, rb, kk, st) for rb in rbs]
            out.append(([self.k_read(st, kk, t)], prods))
        return out

    def mfma_l(self, pbuf, rb, ks):
        a = Lacc(rb)
        n = LACC_REGS
        op = self.mfma16_op
        uses = regs(ONES, 4) + regs(Pr(pbuf, rb, ks), 4) + regs(a, n, "a")
        return Ins("%s a[%d:%d], %s, %s, a[%d:%d]" % (op, a, a + n - 1, vrange(ONES, 4),
                                                      vrange(Pr(pbuf, rb, ks), 4), a, a + n - 1),
                   "mfma", defs=regs(a, n, "a"), uses=uses, srcc=set(regs(a, n, "a")))

    def pv_stream(self, pbuf, t, rbs):
        out = []
        n = 0
        for ks in range(2):
            for db in range(DB()):
                st = n % 4
                n += 1
                prods = [self.mfma_pv(pbuf, rb, db, ks, st) for rb in rbs]
                out.append((self.v_reads(st, db, ks, t), prods))
            if MFMA_ROWSUM:
                out.append(([], [self.mfma_l(pbuf, rb, ks) for rb in rbs]))
        return out


def t(n):
    if n >= NTMP - 1:
        raise ValueError("temporary register index")
    return TMP0 + n


MASK_SGPRS = {0: ["vcc", "%[mk1]", "%[mk2]", "%[mk3]"], 1: ["%[mk4]", "%[mk5]", "%[mk6]", "%[mk7]"]}


def mask_ops(s, m, mask_sgpr):
    """-inf into the scores S(s..s+15) of keys past the diagonal ("tri", threshold %[dmask]) or
    past the valid count ("lim", %[dlim]); nothing when m is None."""
    o = []
    if not m:
        return o
    thr = "%[dmask]" if m == "tri" else "%[dlim]"
    # key index within the half of register r of this lane, minus 4*hi: 8*(r>>2) + (r&3)
    seq = []
    for r in range(16):
        kc = 8 * (r >> 2) + (r & 3)
        mk = mask_sgpr[r % 4]
        if mk == "vcc":
            cmp_ = Ins("v_cmp_le_i32_e32 vcc, %d, %s" % (kc, thr), "cmps", defs=["vcc"])
            sel = Ins("v_cndmask_b32_e32 %s, %s, %s, vcc" % (vr(s + r), vr(NEGINF), vr(s + r)), "valu",
                      defs=[vr(s + r)], uses=[vr(s + r), vr(NEGINF), "vcc"])
        else:
            cmp_ = Ins("v_cmp_le_i32_e64 %s, %d, %s" % (mk, kc, thr), "cmps", defs=[mk])
            sel = Ins("v_cndmask_b32_e64 %s, %s, %s, %s" % (vr(s + r), vr(NEGINF), vr(s + r), mk), "valu",
                      defs=[vr(s + r)], uses=[vr(s + r), vr(NEGINF), mk])
        seq.append((cmp_, sel))
    for r in range(16):
        o.append(seq[r][0])
        if r >= 3:
            o.append(seq[r - 3][1])
    for r in range(13, 16):
        o.append(seq[r][1])
    return o


def interleave_streams(ops_dead, streams, live):
    out = list(ops_dead)
    ls = [streams[rb] for rb in live]
    i = 0
    while any(i < len(x) for x in ls):
        for x in ls:
            if i < len(x):
                out.append(x[i])
        i += 1
    return out


def softmax_fast(g, sbuf, pbuf, par, masks, dead):
    """The vector work of one half when every row's reference is finite, split in two.

    fast: the masks, then P = exp2(S c - m) against the current reference into temporaries
    (S stays as it is), P rounded for the PV product, the row sums in the four chains of
    softmax_ops, l_old = l, l += sum, and the wave's ballot %[ga<par>] of lanes whose partial
    sum exceeds 2^slack: some score may have outrun the reference.
    slow (run only when that ballot is set): l = l_old, then softmax_ops on the masked S,
    which moves the reference, recomputes P and sets %[ga<par>] to its own ballot.
    When no row's maximum outruns its reference by the slack, softmax_ops would keep the
    reference and use alpha = 1, so both paths give the same bits."""
    live = [rb for rb in (0, 1) if rb not in dead]
    ops_dead = []
    for rb in dead:
        for ks in range(2):
            for j in range(4):
                ops_dead.append(Ins("v_mov_b32 %s, 0" % vr(Pr(pbuf, rb, ks) + j), "valu", defs=[vr(Pr(pbuf, rb, ks) + j)]))
    limit = "0x57800000" if g.elem == "bf16" else "0x47000000"      # 2^48, 2^15: 2^slack
    streams = {rb: [] for rb in live}
    checks = []
    restore = []
    for idx, rb in enumerate(live):
        o = streams[rb]
        s = Sr(sbuf, rb)
        base = 9 * idx       # t(0..8) and t(9..17): the blocks' temporaries live side by side
        T = lambda n, base=base: vr(t(base + n))
        S = lambda r, s=s: vr(s + r)
        m = vr(Mr(rb))
        o.extend(mask_ops(s, masks.get(rb), MASK_SGPRS[rb]))
        adds_late = []
        for c in range(8):
            a, b = (T(0), T(1)) if c % 2 == 0 else (T(2), T(3))
            o.append(Ins("v_fma_f32 %s, %s, %%[c], -%s" % (a, S(2 * c), m), "valu", defs=[a], uses=[S(2 * c), m]))
            o.append(Ins("v_fma_f32 %s, %s, %%[c], -%s" % (b, S(2 * c + 1), m), "valu", defs=[b], uses=[S(2 * c + 1), m]))
            o.append(Ins("v_exp_f32_e32 %s, %s" % (a, a), "trans", defs=[a], uses=[a]))
            o.append(Ins("v_exp_f32_e32 %s, %s" % (b, b), "trans", defs=[b], uses=[b]))
            p = Pr(pbuf, rb, c // 4) + c % 4
            o.append(Ins("%s %s, %s, %s" % (g.cvt_op, vr(p), a, b), "valu", defs=[vr(p)], uses=[a, b]))
            if c < 4:
                # chains 0..3 start with elements (2c, 2c + 1), as in softmax_ops
                o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5 + c), a, b), "valu", defs=[T(5 + c)], uses=[a, b]))
            else:
                # element r >= 8 joins chain r % 4, in the order of softmax_ops
                for r, x in ((2 * c, a), (2 * c + 1, b)):
                    o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5 + r % 4), x, T(5 + r % 4)), "valu",
                                 defs=[T(5 + r % 4)], uses=[x, T(5 + r % 4)]))
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5), T(5), T(6)), "valu", defs=[T(5)], uses=[T(5), T(6)]))
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(7), T(7), T(8)), "valu", defs=[T(7)], uses=[T(7), T(8)]))
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5), T(5), T(7)), "valu", defs=[T(5)], uses=[T(5), T(7)]))
        L = vr(Lr(rb))
        o.append(Ins("v_mov_b32_e32 %s, %s" % (T(4), L), "valu", defs=[T(4)], uses=[L]))
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (L, L, T(5)), "valu", defs=[L], uses=[L, T(5)]))
        gb = "%%[g%d%d]" % (par, rb)
        checks += [Ins("v_cmp_lt_f32_e32 vcc, %s, %s" % (limit, T(5)), "cmps", defs=["vcc"], uses=[T(5)]),
                   Ins("s_mov_b64 %s, vcc" % gb, "salu", defs=[gb], uses=["vcc"])]
        restore.append(Ins("v_mov_b32_e32 %s, %s" % (L, T(4)), "valu", defs=[L], uses=[T(4)]))
    fast = interleave_streams(ops_dead, streams, live) + checks
    gs = ["%%[g%d%d]" % (par, rb) for rb in live]
    if len(gs) == 2:
        fast.append(Ins("s_or_b64 %%[ga%d], %s, %s" % (par, gs[0], gs[1]), "salu", defs=["%%[ga%d]" % par], uses=gs))
    else:
        fast.append(Ins("s_mov_b64 %%[ga%d], %s" % (par, gs[0]), "salu", defs=["%%[ga%d]" % par], uses=gs))
    slow = restore + softmax_ops(g, sbuf, pbuf, par, {}, False, dead)
    return fast, slow, par


def soft(g, sbuf, pbuf, par, masks, first, dead):
    """The softmax of a half: the two-path form once every reference is finite (and with the
    fp32 row sums), else softmax_ops."""
    if FAST and not first and not MFMA_ROWSUM:
        return softmax_fast(g, sbuf, pbuf, par, masks, dead)
    return softmax_ops(g, sbuf, pbuf, par, masks, first, dead)


def softmax_ops(g, sbuf, pbuf, par, masks, first, dead):
    """The vector work of one half.

    masks: dict rb -> None | "tri" | "lim"  (lim: keys past the valid count, threshold in
    %[dlim]); dead: row blocks whose keys are all masked in this half (P = 0, alpha = 1).
    first: the reference may still be -inf (first half, or a masked half of the first tile):
    use 0 as the exp reference while it is.
    """
    live = [rb for rb in (0, 1) if rb not in dead]
    streams = {rb: [] for rb in live}
    ops_dead = []
    for rb in dead:
        for ks in range(2):
            for j in range(4):
                ops_dead.append(Ins("v_mov_b32 %s, 0" % vr(Pr(pbuf, rb, ks) + j), "valu", defs=[vr(Pr(pbuf, rb, ks) + j)]))
        ops_dead.append(Ins("v_mov_b32 %s, 1.0" % vr(ALr(par, rb)), "valu", defs=[vr(ALr(par, rb))]))
    mask_sgprs = MASK_SGPRS
    for idx, rb in enumerate(live):
        mask_sgpr = mask_sgprs[rb]
        o = streams[rb]
        s = Sr(sbuf, rb)
        base = 8 * idx       # temporaries of this row block: t(base) .. t(base + 8)
        T = lambda n: vr(t(base + n))
        o.extend(mask_ops(s, masks.get(rb), mask_sgprs[rb]))
        # row max over this lane's 16 scores
        S = lambda r: vr(s + r)
        o.append(Ins("v_max3_f32 %s, %s, %s, %s" % (T(0), S(0), S(1), S(2)), "valu", defs=[T(0)], uses=[S(0), S(1), S(2)]))
        o.append(Ins("v_max3_f32 %s, %s, %s, %s" % (T(1), S(3), S(4), S(5)), "valu", defs=[T(1)], uses=[S(3), S(4), S(5)]))
        o.append(Ins("v_max3_f32 %s, %s, %s, %s" % (T(2), S(6), S(7), S(8)), "valu", defs=[T(2)], uses=[S(6), S(7), S(8)]))
        o.append(Ins("v_max3_f32 %s, %s, %s, %s" % (T(3), S(9), S(10), S(11)), "valu", defs=[T(3)], uses=[S(9), S(10), S(11)]))
        o.append(Ins("v_max3_f32 %s, %s, %s, %s" % (T(4), S(12), S(13), S(14)), "valu", defs=[T(4)], uses=[S(12), S(13), S(14)]))
        o.append(Ins("v_max3_f32 %s, %s, %s, %s" % (T(0), T(0), T(1), T(2)), "valu", defs=[T(0)], uses=[T(0), T(1), T(2)]))
        o.append(Ins("v_max3_f32 %s, %s, %s, %s" % (T(3), T(3), T(4), S(15)), "valu", defs=[T(3)], uses=[T(3), T(4), S(15)]))
        o.append(Ins("v_max_f32_e32 %s, %s, %s" % (T(0), T(0), T(3)), "valu", defs=[T(0)], uses=[T(0), T(3)]))
        # the other lane half holds the same row: exchange and take the larger
        o.append(Ins("v_mov_b32_e32 %s, %s" % (T(1), T(0)), "valu", defs=[T(1)], uses=[T(0)]))
        o.append(Ins("v_permlane32_swap_b32_e32 %s, %s" % (T(0), T(1)), "perm", defs=[T(0), T(1)], uses=[T(0), T(1)]))
        o.append(Ins("v_max_f32_e32 %s, %s, %s" % (T(0), T(0), T(1)), "valu", defs=[T(0)], uses=[T(0), T(1)]))
        # scaled max, lazy move of the reference (only past 2^8 of growth)
        o.append(Ins("v_mul_f32_e32 %s, %%[c], %s" % (T(0), T(0)), "valu", defs=[T(0)], uses=[T(0)]))
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(2), g.slack, vr(Mr(rb))), "valu", defs=[T(2)], uses=[vr(Mr(rb))]))
        gb = "%%[g%d%d]" % (par, rb)
        o.append(Ins("v_cmp_gt_f32_e64 %s, %s, %s" % (gb, T(0), T(2)), "cmps", defs=[gb], uses=[T(0), T(2)]))
        o.append(Ins("v_cndmask_b32_e64 %s, %s, %s, %s" % (T(3), vr(Mr(rb)), T(0), gb), "valu", defs=[T(3)],
                     uses=[vr(Mr(rb)), T(0), gb]))
        if first:
            # nothing finite yet on this row: 0 as the exp reference (P = 0, alpha = 0)
            gk = mask_sgpr[1]
            o.append(Ins("v_cmp_eq_f32_e64 %s, %s, %s" % (gk, vr(NEGINF), T(3)), "cmps", defs=[gk],
                         uses=[vr(NEGINF), T(3)]))
            o.append(Ins("v_cndmask_b32_e64 %s, %s, 0, %s" % (T(4), T(3), gk), "valu", defs=[T(4)],
                         uses=[T(3), gk]))
            ref = T(4)
        else:
            ref = T(3)
        o.append(Ins("v_sub_f32_e32 %s, %s, %s" % (T(2), vr(Mr(rb)), ref), "valu", defs=[T(2)], uses=[vr(Mr(rb)), ref]))
        o.append(Ins("v_exp_f32_e32 %s, %s" % (vr(ALr(par, rb)), T(2)), "trans", defs=[vr(ALr(par, rb))], uses=[T(2)]))
        o.append(Ins("v_mov_b32_e32 %s, %s" % (vr(Mr(rb)), T(3)), "valu", defs=[vr(Mr(rb))], uses=[T(3)]))
        # P = exp2(S c - m), in place; row sums in four chains; P rounded for the PV product
        pe = []
        for r in range(16):
            pe.append(Ins("v_fma_f32 %s, %s, %%[c], -%s" % (S(r), S(r), ref), "valu", defs=[S(r)], uses=[S(r), ref]))
            pe.append(Ins("v_exp_f32_e32 %s, %s" % (S(r), S(r)), "trans", defs=[S(r)], uses=[S(r)]))
        o.extend(pe)
        cvts = []
        for ks in range(2):
            for j in range(4):
                p = Pr(pbuf, rb, ks) + j
                cvts.append(Ins("%s %s, %s, %s" % (g.cvt_op, vr(p), S(8 * ks + 2 * j), S(8 * ks + 2 * j + 1)), "valu",
                                defs=[vr(p)], uses=[S(8 * ks + 2 * j), S(8 * ks + 2 * j + 1)]))
        if MFMA_ROWSUM:
            o.extend(cvts)
            continue
        sums = []
        for c in range(4):
            sums.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5 + c), S(2 * c), S(2 * c + 1)), "valu",
                            defs=[T(5 + c)], uses=[S(2 * c), S(2 * c + 1)]))
        for r in range(8, 16):
            c = r % 4
            sums.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5 + c), S(r), T(5 + c)), "valu", defs=[T(5 + c)],
                            uses=[S(r), T(5 + c)]))
        # interleave sums and conversions
        for a, b in zip(sums[:8], cvts):
            o.append(a)
            o.append(b)
        o.extend(sums[8:])
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5), T(5), T(6)), "valu", defs=[T(5)], uses=[T(5), T(6)]))
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(7), T(7), T(8)), "valu", defs=[T(7)], uses=[T(7), T(8)]))
        o.append(Ins("v_add_f32_e32 %s, %s, %s" % (T(5), T(5), T(7)), "valu", defs=[T(5)], uses=[T(5), T(7)]))
        o.append(Ins("v_fma_f32 %s, %s, %s, %s" % (vr(Lr(rb)), vr(Lr(rb)), vr(ALr(par, rb)), T(5)), "valu",
                     defs=[vr(Lr(rb))], uses=[vr(Lr(rb)), vr(ALr(par, rb)), T(5)]))
    # interleave the row blocks' streams
    out = interleave_streams(ops_dead, streams, live)
    # the wave's "any row moved its reference" ballot for this parity
    gs = ["%%[g%d%d]" % (par, rb) for rb in live]
    if len(gs) == 2:
        out.append(Ins("s_or_b64 %%[ga%d], %s, %s" % (par, gs[0], gs[1]), "salu", defs=["%%[ga%d]" % par], uses=gs))
    else:
        out.append(Ins("s_mov_b64 %%[ga%d], %s" % (par, gs[0]), "salu", defs=["%%[ga%d]" % par], uses=gs))
    return out


def rescale_block(par, rbs):
    """O *= alpha[par] on the row blocks rbs: read, multiply, write back, 8 at a time."""
    out = [Ins("s_nop 7", "nop")]
    regs_list = [(rb, Or(rb, db) + r) for rb in rbs for db in range(DB()) for r in range(16)]
    if MFMA_ROWSUM:
        regs_list += [(rb, Lacc(rb) + r) for rb in rbs for r in range(LACC_REGS)]
    for i in range(0, len(regs_list), 8):
        chunk = regs_list[i:i + 8]
        for j, (rb, a) in enumerate(chunk):
            out.append(Ins("v_accvgpr_read_b32 %s, a%d" % (vr(t(j)), a), "accr", defs=[vr(t(j))], uses=["a%d" % a]))
        for j, (rb, a) in enumerate(chunk):
            out.append(Ins("v_mul_f32_e32 %s, %s, %s" % (vr(t(j)), vr(ALr(par, rb)), vr(t(j))), "valu",
                           defs=[vr(t(j))], uses=[vr(t(j)), vr(ALr(par, rb))]))
        for j, (rb, a) in enumerate(chunk):
            out.append(Ins("v_accvgpr_write_b32 a%d, %s" % (a, vr(t(j))), "accw", defs=["a%d" % a], uses=[vr(t(j))]))
    return out


def merge_half(prod_streams, valu, extra, lead=2, preissued=0, head_valu=0, next_reads=()):
    """Interleave one half: the product streams (list of (reads, products) in order), the
    vector work and the extra instructions (DMA, toggles).  Each group's reads are issued
    ``lead`` groups ahead of its products; the vector and extra work is spread evenly over
    the products.  ``preissued``: the first groups whose reads the previous half already
    issued; ``head_valu``: vector instructions placed between the first reads and the first
    product (work that covers the read latency); ``next_reads``: the next half's first reads,
    issued after this half's last reads."""
    groups = []
    for stream in prod_streams:
        groups.extend(stream)
    nprod = sum(len(p) for _, p in groups)
    out = []
    for k in range(preissued, min(lead, len(groups))):
        out.extend(groups[k][0])
    vi = h0 = min(head_valu, len(valu))
    out.extend(valu[:vi])
    ei = 0
    done = 0
    pending_next = list(next_reads)
    for gi, (_, prods) in enumerate(groups):
        if gi + lead < len(groups):
            out.extend(groups[gi + lead][0])
        elif pending_next:
            out.extend(pending_next)
            pending_next = []
        for p in prods:
            out.append(p)
            done += 1
            vt = h0 + ((len(valu) - h0) * done + nprod - 1) // nprod if nprod else len(valu)
            et = (len(extra) * done + nprod - 1) // nprod if nprod else len(extra)
            while ei < et:
                out.append(extra[ei])
                ei += 1
            while vi < vt:
                out.append(valu[vi])
                vi += 1
    out.extend(pending_next)
    out.extend(extra[ei:])
    out.extend(valu[vi:])
    return out


# ---------------------------------------------------------------- tile loads (LDS DMA)

def dma_tile(which, nw):
    """This wave's share of one 64-key K or V tile (TILE / 1 KiB slices, slice ii = wave + nw*i)
    from %[<which>src] (byte offset of the tile in the head) into the buffer at %[<which>dst]
    (LDS address of this wave's first slice in the tile's buffer).  The lane's source offset
    within a slice depends on ii only through ii mod 4 (d = 128) or ii mod 2 (d = 64):
    %[dma0] (i even) and %[dma1] (i odd)."""
    out = []
    rs = "%[krs]" if which == "k" else "%[vrs]"
    for i in range(TILE() // 1024 // nw):
        out.append(Ins("s_add_u32 m0, %%[%sdst], %d" % (which, 1024 * nw * i), "m0", defs=["m0"]))
        out.append(Ins("s_add_u32 %%[soff], %%[%ssrc], %d" % (which, 1024 * nw * i), "salu", defs=["%[soff]"]))
        out.append(Ins("buffer_load_dwordx4 %%[dma%d], %s, %%[soff] offen lds" % (i & 1, rs), "dma",
                       uses=["m0", "%[soff]"]))
    return out


def advance_k():
    """Next K tile: source + one tile, LDS buffer toggled."""
    return [Ins("s_add_u32 %%[ksrc], %%[ksrc], %d" % TILE(), "salu", defs=["%[ksrc]"], uses=["%[ksrc]"]),
            Ins("s_xor_b32 %%[kdst], %%[kdst], %d" % TILE(), "salu", defs=["%[kdst]"], uses=["%[kdst]"])]


def advance_v():
    return [Ins("s_add_u32 %%[vsrc], %%[vsrc], %d" % TILE(), "salu", defs=["%[vsrc]"], uses=["%[vsrc]"]),
            Ins("s_xor_b32 %%[vdst], %%[vdst], %d" % TILE(), "salu", defs=["%[vdst]"], uses=["%[vdst]"])]


def toggle_reads():
    """Switch the K and V operand reads to the other buffer of each."""
    out = []
    for kk in range(KK()):
        out.append(Ins("v_xor_b32_e32 %%[koff%d], 0x%x, %%[koff%d]" % (kk, TILE(), kk), "valu",
                       defs=["%%[koff%d]" % kk], uses=["%%[koff%d]" % kk]))
    for i in range(2 * DB()):
        out.append(Ins("v_xor_b32_e32 %%[voff%d], 0x%x, %%[voff%d]" % (i, TILE(), i), "valu",
                       defs=["%%[voff%d]" % i], uses=["%%[voff%d]" % i]))
    return out


def barrier():
    """Every wave's tile loads have landed and its LDS reads have returned; then the barrier.
    (Loads that write LDS directly count in vmcnt, and a barrier does not wait for them.)"""
    return [Ins("s_waitcnt vmcnt(0) lgkmcnt(0)", "waitall"), Ins("s_barrier", "barrier")]


def nstores():
    """Vector memory stores of the epilogue (O and LSE), counted in the instructions it emits:
    an item's first barrier may leave exactly this many of the item before in flight."""
    return sum(1 for ins in epilogue(Gen("bf16", False)) if ins.kind == "vstore")


def q_vloads():
    """This wave's Q rows straight into the operand registers (rb 1 sits 32 rows on)."""
    out = [Ins("s_mov_b32 %%[soff], %d" % (32 * ROWB()), "salu", defs=["%[soff]"])]
    for rb in (0, 1):
        for kk in range(KK()):
            so = "0" if rb == 0 else "%[soff]"
            out.append(Ins("buffer_load_dwordx4 %s, %%[qoff], %%[qrs], %s offen offset:%d" % (vrange(Qr(rb, kk), 4), so, 32 * kk),
                           "vload", defs=regs(Qr(rb, kk), 4), uses=[] if rb == 0 else ["%[soff]"]))
    return out


def q_stage():
    """The next item's Q rows of this wave into its LDS staging area at %[qst] (LDS DMA):
    slice j = KK() rb + kk holds, at 16 lane bytes per lane, the operand registers of (rb,
    kk) exactly as q_vloads would load them, so that one ds_read_b128 per slice brings them
    back without bank conflicts."""
    out = []
    for rb in (0, 1):
        for kk in range(KK()):
            j = KK() * rb + kk
            out.append(Ins("s_add_u32 m0, %%[qst], %d" % (1024 * j), "m0", defs=["m0"]))
            out.append(Ins("s_mov_b32 %%[soff], %d" % (32 * ROWB() * rb + 32 * kk), "salu", defs=["%[soff]"]))
            out.append(Ins("buffer_load_dwordx4 %[nqoff], %[nqrs], %[soff] offen lds", "dma", uses=["m0", "%[soff]"]))
    return out


def q_unstage():
    """Q from the staging area at %[qlds] (this lane's 16 bytes of slice 0) into the operand
    registers."""
    out = []
    for rb in (0, 1):
        for kk in range(KK()):
            j = KK() * rb + kk
            out.append(Ins("ds_read_b128 %s, %%[qlds] offset:%d" % (vrange(Qr(rb, kk), 4), 1024 * j), "lds",
                           defs=regs(Qr(rb, kk), 4)))
            if j % 8 == 7:
                out.append(Ins("s_waitcnt lgkmcnt(0)", "waitall"))
    return out


def kv_prefetch(g, nw):
    """The next item's first tiles into the other LDS buffer set (%[nkdst]: its K buffer 0 plus
    this wave's slice): K tile 0 to K buffer 0, K tile 1 (when the next item has one) to K
    buffer 1, V tile 0 to V buffer 1, from the next head (%[nkrs], %[nvrs])."""
    def tile(dst, rs):
        out = []
        for i in range(TILE() // 1024 // nw):
            out.append(Ins("s_add_u32 m0, %%[nkdst], %d" % (dst + 1024 * nw * i), "m0", defs=["m0"]))
            out.append(Ins("s_mov_b32 %%[soff], %d" % (src_of[dst] + 1024 * nw * i), "salu", defs=["%[soff]"]))
            out.append(Ins("buffer_load_dwordx4 %%[dma%d], %s, %%[soff] offen lds" % (i & 1, rs), "dma",
                           uses=["m0", "%[soff]"]))
        return out
    src_of = {0: 0, TILE(): TILE(), 3 * TILE(): 0}
    out = tile(0, "%[nkrs]")
    out.append(Cond(["s_cmp_gt_u32 %[nnt], 1"], tile(TILE(), "%[nkrs]"), "L_pk1_%d" % len(g.labels)))
    g.labels.append(1)
    out.extend(tile(3 * TILE(), "%[nvrs]"))
    return out


def prefetch(g, nw, with_q):
    """The next item's loads, issued once per item by every wave in the same two steps: its
    first K/V tiles when %[kit] reaches %[pkv], its Q rows when %[kit] reaches %[pq] (a step
    no S product of this item follows; ~0 when there is no next item)."""
    out = [Cond(["s_cmp_eq_u32 %[kit], %[pkv]"], kv_prefetch(g, nw), "L_pkv%d" % len(g.labels))]
    g.labels.append(1)
    if with_q:
        out.append(Cond(["s_cmp_eq_u32 %[kit], %[pq]"], q_stage(), "L_pq%d" % len(g.labels)))
        g.labels.append(1)
    return out


# ---------------------------------------------------------------- the program

def half_groups(g, s_next, pv_prev):
    """The product groups of one half, S and PV alternating."""
    s_groups = g.s_stream(*s_next) if s_next else []
    pv_groups = g.pv_stream(*pv_prev) if pv_prev else []
    merged = []
    for i in range(max(len(s_groups), len(pv_groups))):
        if i < len(s_groups):
            merged.append(s_groups[i])
        if i < len(pv_groups):
            merged.append(pv_groups[i])
    return merged


LEAD = 2          # product groups a group's operand reads run ahead
FAST = os.environ.get("FA_GEN_FAST", "1") == "1"
HEAD_VALU = 12    # softmax instructions that cover the first reads of a half after a barrier


def first_reads(g, s_next, pv_prev):
    """The reads of a half's first LEAD groups (to be issued by the half before it)."""
    out = []
    for reads, _ in half_groups(g, s_next, pv_prev)[:LEAD]:
        out.extend(reads)
    return out


def half_interleaved(g, s_next, pv_prev, soft, rescale_par, extra=(), preissued=False, next_half=None,
                     after_barrier=False):
    """One half with the S and PV products alternating.  The rescale of O for the previous
    half's softmax, when any row moved its reference, comes before the first product.
    preissued: this half's first reads were issued by the previous half; next_half:
    (s_next, pv_prev) of the following half when no barrier separates them, whose first
    reads this half issues at its end; after_barrier: start with a few softmax
    instructions while the first reads are in flight."""
    merged = half_groups(g, s_next, pv_prev)
    out = []
    if pv_prev and rescale_par is not None:
        out.append(Skip("%%[ga%d]" % rescale_par, rescale_block(rescale_par, pv_prev[2]), "L_rs%d" % len(g.labels)))
        g.labels.append(1)
    nxt = first_reads(g, *next_half) if next_half else ()
    slow = None
    if isinstance(soft, tuple):
        soft, slow, par = soft
    out.extend(merge_half([merged], list(soft), list(extra), lead=LEAD, preissued=LEAD if preissued else 0,
                          head_valu=HEAD_VALU if after_barrier else 0, next_reads=nxt))
    if slow is not None:
        out.append(Skip("%%[ga%d]" % par, slow, "L_sl%d" % len(g.labels)))
        g.labels.append(1)
    return out


def build(elem, causal, nw):
    g = Gen(elem, causal)
    g.labels = []
    all_rb = (0, 1)
    prog = []
    # ---- setup: O = 0, m = -inf, l = 0, Q loads (sign folded), -inf constant
    prog.append(Ins("v_mov_b32 %s, %s" % (vr(NEGINF), NEG_INF_BITS), "valu", defs=[vr(NEGINF)]))
    for rb in all_rb:
        prog.append(Ins("v_mov_b32 %s, %s" % (vr(Mr(rb)), NEG_INF_BITS), "valu", defs=[vr(Mr(rb))]))
        prog.append(Ins("v_mov_b32 %s, 0" % vr(Lr(rb)), "valu", defs=[vr(Lr(rb))]))
    prog.append(Ins("s_mov_b32 %[kit], 1", "salu", defs=["%[kit]"]))
    # ---- Q and the first tiles: K(0), K(1) (if any), V(0).  The first item of a workgroup
    # loads them here (%[pf] = 0) and waits for them; a later one finds them prefetched by the
    # item before it (its K/V in this item's buffer set, its Q staged in LDS), waits only for
    # loads older than that item's epilogue stores, and reads Q back from the staging area.
    own = q_vloads() + dma_tile("k", nw) + advance_k()
    own.append(Cond(["s_cmp_gt_u32 %[nt], 1"], dma_tile("k", nw), "L_k1"))
    own.extend(advance_k() + dma_tile("v", nw) + advance_v())
    staged = [Ins("s_waitcnt vmcnt(%d)" % nstores(), "wait")] + q_unstage()
    staged.extend(advance_k() + advance_k() + advance_v())
    prog.append(Cond(["s_cmp_eq_u32 %[pf], 0"], own, "L_own"))
    prog.append(Cond(["s_cmp_lg_u32 %[pf], 0"], staged, "L_staged"))
    zero = list(range(32 * DB()))
    if MFMA_ROWSUM:
        zero += list(range(Lacc(0), Lacc(0) + 2 * LACC_REGS))
    for a in zero:
        prog.append(Ins("v_accvgpr_write_b32 a%d, 0" % a, "accw", defs=["a%d" % a]))
    if MFMA_ROWSUM:
        prog.extend(ones16(elem))
    prog.append(Cond(["s_cmp_eq_u32 %[pf], 0"], [Ins("s_waitcnt vmcnt(0)", "wait")], "L_ownw"))
    # every wave's share of the first tiles has landed (the stores of the item before, at most
    # nstores() younger vector memory operations, need not have)
    prog.append(Ins("s_waitcnt vmcnt(%d) lgkmcnt(0)" % nstores(), "waitall"))
    prog.append(Ins("s_barrier", "barrier"))
    for r in range(8 * KK()):
        prog.append(Ins("v_xor_b32_e32 v%d, %%[flip], v%d" % (r, r), "valu", defs=["v%d" % r], uses=["v%d" % r]))
    # S(0) alone
    prog.extend(merge_half([g.s_stream(0, 0, all_rb)], [], []))

    tri = "tri" if causal else "lim"
    maskA = {0: "tri"} if causal else {0: "lim", 1: "lim"}
    maskB = {1: "tri"} if causal else {0: "lim", 1: "lim"}
    deadB = (0,) if causal else ()
    rbB = (1,) if causal else all_rb
    lim_ops = lambda which: [] if causal else [
        Ins("v_sub_u32_e32 %%[dlim], %%[%s], %%[hi4]" % which, "valu", defs=["%[dlim]"])]

    # iteration k: barrier B_k, loads K(k+1) and V(k), halves 2k-1 and 2k
    def iter_head(cond_k, cond_v, toggle=True):
        out = toggle_reads() if toggle else []
        out.extend(barrier())
        ek = dma_tile("k", nw) + advance_k()
        ev = dma_tile("v", nw) + advance_v()
        if cond_k:
            ek = [Cond(["s_add_u32 %[soff], %[kit], 1", "s_cmp_lt_u32 %[soff], %[nt]"], ek, "L_ck%d" % len(g.labels))]
            g.labels.append(1)
        if cond_v:
            ev = [Cond(["s_cmp_lt_u32 %[kit], %[nt]"], ev, "L_cv%d" % len(g.labels))]
            g.labels.append(1)
        return out, ek + ev

    # ---- L >= 1 path: half 0 unmasked
    pathA = []
    pathA.extend(half_interleaved(g, (1, 1, all_rb), None,
                                  soft(g, 0, 0, 0, {}, True, ()), None))
    pathA.append(Ins("s_mov_b64 %[ga0], 0", "salu", defs=["%[ga0]"]))      # O is zero: no rescale
    # steady loop over k = 1 .. L-1.  K tile j lands in K buffer j % 2 and V tile j in V buffer
    # (j + 1) % 2; %[koff] and %[voff] start at buffer 0 of each and each toggling iteration
    # flips both before reading, so iteration k reads K buffer k % 2 (tile k) and V buffer
    # k % 2 (tile k - 1).  Pairs of iterations run with the buffer named by the reads' offsets
    # (no register toggles); an odd count ends with one iteration in the toggling form, which
    # leaves the registers as L - 1 toggles would.
    def iteration(toggle, kbuf=0, vbuf=0):
        g.kbuf, g.vbuf = kbuf, vbuf
        head, dmas = iter_head(False, False, toggle)
        out = list(head)
        out.extend(half_interleaved(g, (0, 0, all_rb), (0, 0, all_rb),
                                    soft(g, 1, 1, 1, {}, False, ()), 0, dmas,
                                    next_half=((1, 1, all_rb), (1, 1, all_rb)), after_barrier=True))
        out.extend(half_interleaved(g, (1, 1, all_rb), (1, 1, all_rb),
                                    soft(g, 0, 0, 0, {}, False, ()), 1, [], preissued=True))
        out.append(Ins("s_add_u32 %[kit], %[kit], 1", "salu", defs=["%[kit]"], uses=["%[kit]"]))
        g.kbuf = g.vbuf = 0
        return out

    pair = iteration(False, 1, 1) + iteration(False, 0, 0)
    pathA.append(Ins("s_sub_u32 %[cnt], %[last], 1", "salu", defs=["%[cnt]"]))
    pathA.append(Ins("s_lshr_b32 %[cnt], %[cnt], 1", "salu", defs=["%[cnt]"], uses=["%[cnt]"]))
    pathA.append(Cond(["s_cmp_lg_u32 %[cnt], 0"], [Loop("%[cnt]", pair, "L_loop")], "L_skiploop"))
    pathA.append(Cond(["s_bitcmp0_b32 %[last], 0"], iteration(True), "L_odd%d" % len(g.labels)))
    g.labels.append(1)
    # iteration L: half 2L-1 unmasked, half 2L masked A
    head, dmas = iter_head(True, False)
    pathA.extend(head)
    pathA.extend(prefetch(g, nw, False))
    pathA.extend(lim_ops("limA"))
    pathA.extend(half_interleaved(g, (0, 0, all_rb), (0, 0, all_rb),
                                  soft(g, 1, 1, 1, {}, False, ()), 0, dmas,
                                  next_half=((1, 1, rbB), (1, 1, all_rb)), after_barrier=True))
    pathA.extend(half_interleaved(g, (1, 1, rbB), (1, 1, all_rb),
                                  soft(g, 0, 0, 0, maskA, False, ()), 1, [], preissued=True))
    pathA.append(Ins("s_add_u32 %[kit], %[kit], 1", "salu", defs=["%[kit]"], uses=["%[kit]"]))
    pathA.append(Ins("s_branch L_tailB_%=", "branch"))
    # ---- L == 0 path: half 0 masked A
    pathB = []
    pathB.extend(lim_ops("limA"))
    pathB.extend(half_interleaved(g, (1, 1, rbB), None,
                                  soft(g, 0, 0, 0, maskA, True, ()), None))
    pathB.append(Ins("s_mov_b64 %[ga0], 0", "salu", defs=["%[ga0]"]))
    # ---- tail B (iteration L+1): half 2L+1 (PV(2L), softmax masked B), half 2L+2 (PV(2L+1))
    tail = []
    head, dmas = iter_head(True, True)
    tail.extend(head)
    tail.extend(prefetch(g, nw, True))
    tail.extend(lim_ops("limB"))
    tail.extend(half_interleaved(g, None, (0, 0, all_rb),
                                 soft(g, 1, 1, 1, maskB, False, deadB), 0, dmas,
                                 next_half=(None, (1, 1, rbB)), after_barrier=True))
    tail.extend(half_interleaved(g, None, (1, 1, rbB), [], 1, [], preissued=True))
    tail.append(Ins("s_add_u32 %[kit], %[kit], 1", "salu", defs=["%[kit]"], uses=["%[kit]"]))
    # the wave is done with its rows: store O and LSE
    tail.extend(epilogue(g))
    # the waves still walking tiles need this wave's share of the loads and its barriers
    duty = []
    head, dmas = iter_head(True, True)
    duty.extend(head)
    duty.extend(prefetch(g, nw, True))
    duty.extend(dmas)
    duty.append(Ins("s_add_u32 %[kit], %[kit], 1", "salu", defs=["%[kit]"], uses=["%[kit]"]))
    tail.append(Ins("s_sub_u32 %[cnt], %[nt], %[last]", "salu", defs=["%[cnt]"]))
    tail.append(Ins("s_sub_u32 %[cnt], %[cnt], 1", "salu", defs=["%[cnt]"]))
    # a wave that staged the next Q after its own stores waits for it here, so that the next
    # item's wait for loads older than its last nstores() operations covers it
    tail.append(Cond(["s_cmp_lg_u32 %[cnt], 0"], [Loop("%[cnt]", duty, "L_duty"), Ins("s_waitcnt vmcnt(0)", "wait")],
                     "L_skipduty"))
    tail.append(Ins("s_waitcnt lgkmcnt(0)", "wait"))
    return g, prog, pathA, pathB, tail


def ones16(elem):
    """The A operand of the 16x16x32 row-sum products.

    P of a row block sits as the B operand of a 32x32x16 product: lane L holds row L % 32 and
    8 keys.  Read as the B operand of a 16x16x32 product, lane L is column L % 16 in k-group
    L // 16, so column n gathers rows n (groups 0, 2) and n + 16 (groups 1, 3).  With
    A[m][k] = 1 exactly when the k-group's parity equals bit 2 of m, output row m sums the 16
    keys of row n + 16 * ((m >> 2) & 1); the 16x16 output puts rows 4 * (L // 16) + j in
    lane L, so every result of lane L is the sum over the keys of row L % 32, its own row.
    Lane L of A is row L % 16, k-group L // 16: one when bit 4 of L equals bit 2 of L."""
    one2 = "0x3f803f80" if elem == "bf16" else "0x3c003c00"
    a, b, c = vr(t(1)), vr(t(2)), vr(t(3))
    out = [Ins("v_mbcnt_lo_u32_b32 %s, -1, 0" % a, "valu", defs=[a]),
           Ins("v_mbcnt_hi_u32_b32 %s, -1, %s" % (a, a), "valu", defs=[a], uses=[a]),
           Ins("v_lshrrev_b32_e32 %s, 2, %s" % (b, a), "valu", defs=[b], uses=[a]),
           Ins("v_lshrrev_b32_e32 %s, 4, %s" % (a, a), "valu", defs=[a], uses=[a]),
           Ins("v_xor_b32_e32 %s, %s, %s" % (a, a, b), "valu", defs=[a], uses=[a, b]),
           Ins("v_and_b32_e32 %s, 1, %s" % (a, a), "valu", defs=[a], uses=[a]),
           Ins("v_mov_b32_e32 %s, %s" % (c, one2), "valu", defs=[c]),
           Ins("v_cmp_eq_u32_e32 vcc, 0, %s" % a, "cmps", defs=["vcc"], uses=[a])]
    for i in range(4):
        out.append(Ins("v_cndmask_b32_e32 %s, 0, %s, vcc" % (vr(ONES + i), c), "valu",
                       defs=[vr(ONES + i)], uses=[c, "vcc"]))
    return out


def epilogue(g):
    out = [Ins("s_nop 15", "nop"), Ins("s_nop 15", "nop")]
    for rb in (0, 1):
        L = vr(Lr(rb))
        if MFMA_ROWSUM:
            out.append(Ins("v_accvgpr_read_b32 %s, a%d" % (L, Lacc(rb)), "accr", defs=[L], uses=["a%d" % Lacc(rb)]))
        else:
            tl = vr(t(20))
            out.append(Ins("v_mov_b32_e32 %s, %s" % (tl, L), "valu", defs=[tl], uses=[L]))
            out.append(Ins("v_permlane32_swap_b32_e32 %s, %s" % (L, tl), "perm", defs=[L, tl], uses=[L, tl]))
            out.append(Ins("v_add_f32_e32 %s, %s, %s" % (L, L, tl), "valu", defs=[L], uses=[L, tl]))
        inv = vr(t(21))
        out.append(Ins("v_rcp_f32_e32 %s, %s" % (inv, L), "trans", defs=[inv], uses=[L]))
        lg = vr(t(22))
        out.append(Ins("v_log_f32_e32 %s, %s" % (lg, L), "trans", defs=[lg], uses=[L]))
        out.append(Ins("v_add_f32_e32 %s, %s, %s" % (lg, vr(Mr(rb)), lg), "valu", defs=[lg], uses=[lg, vr(Mr(rb))]))
        out.append(Ins("v_mul_f32_e32 %s, 0x3f317218, %s" % (lg, lg), "valu", defs=[lg], uses=[lg]))   # ln 2
        loff = "%[loff]" if rb == 0 else vr(t(19))
        if rb == 1:
            out.append(Ins("v_add_u32_e32 %s, 0x80, %%[loff]" % vr(t(19)), "valu", defs=[vr(t(19))]))
        out.append(Ins("buffer_store_dword %s, %s, %%[lrs], 0 offen" % (lg, loff), "vstore", uses=[lg, loff]))
        ooff = "%[ooff]" if rb == 0 else vr(t(18))
        if rb == 1:
            out.append(Ins("v_add_u32_e32 %s, 0x%x, %%[ooff]" % (vr(t(18)), 32 * ROWB()), "valu", defs=[vr(t(18))]))
        for db in range(DB()):
            for gq in range(4):
                a0 = Or(rb, db) + 4 * gq
                tv = [vr(t(j)) for j in range(4)]
                for j in range(4):
                    out.append(Ins("v_accvgpr_read_b32 %s, a%d" % (tv[j], a0 + j), "accr", defs=[tv[j]],
                                   uses=["a%d" % (a0 + j)]))
                for j in range(4):
                    out.append(Ins("v_mul_f32_e32 %s, %s, %s" % (tv[j], inv, tv[j]), "valu", defs=[tv[j]],
                                   uses=[tv[j], inv]))
                pk = vr(t(8 + 2 * gq))
                pk2 = vr(t(9 + 2 * gq))
                out.append(Ins("%s %s, %s, %s" % (g.cvt_op, pk, tv[0], tv[1]), "valu", defs=[pk], uses=tv[:2]))
                out.append(Ins("%s %s, %s, %s" % (g.cvt_op, pk2, tv[2], tv[3]), "valu", defs=[pk2], uses=tv[2:]))
                off = (32 * db + 8 * gq) * 2
                out.append(Ins("buffer_store_dwordx2 %s, %s, %%[ors], 0 offen offset:%d" % (
                    "v[%d:%d]" % (t(8 + 2 * gq), t(9 + 2 * gq)), ooff, off), "vstore",
                    uses=[pk, pk2, ooff]))
    return out


def assemble(elem, causal, nw, d=128):
    global D, ROWSUM, MFMA_ROWSUM
    D = d
    ROWSUM = ROWSUM_BY_D[d]
    MFMA_ROWSUM = ROWSUM == "mfma16"
    g, prog, pathA, pathB, tail = build(elem, causal, nw)
    st = State()
    out = []
    lower(prog, st, out, "%=")
    out.append("s_cmp_eq_u32 %[last], 0")
    out.append("s_cbranch_scc1 L_pathB_%=")
    st.pos += 2
    stB = st.copy()
    lower(pathA, st, out, "%=")
    out.append("L_pathB_%=:")
    lower(pathB, stB, out, "%=")
    out.append("L_tailB_%=:")
    st2 = merge_states(st, stB)
    lower(tail, st2, out, "%=")
    return out


def main():
    parts = ["// Generated by gen_fwd_kloop.py; do not edit.  The key loop of the 64-rows-per-wave\n"
             "// forward (fa_fwd_w64.hip) as gfx950 assembly, one string per element type, mask and\n"
             "// number of waves per workgroup (which share each tile's loads).\n"
             "#pragma once\n"]
    for d in (128, 64):
        for nw in (2, 4):
            for elem in ("bf16", "f16"):
                for causal in (False, True):
                    lines = assemble(elem, causal, nw, d)
                    name = "FA_KLOOP_%s_%s_W%d_D%d" % (elem.upper(), "CAUSAL" if causal else "FULL", nw, d)
                    parts.append("#define %s \\\n%s\n" % (name, " \\\n".join('    "%s\\n"' % l for l in lines)))
    text = "\n".join(parts)
    with open(OUT, "w") as f:
        f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
