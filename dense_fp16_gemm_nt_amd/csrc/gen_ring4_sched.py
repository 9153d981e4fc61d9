"""Generate the instruction schedule of the 4-wave ring kernel (ring4.hpp).

The k loop of that kernel is one inline-assembly block so that the order of
matrix-core instructions, LDS fragment reads, direct-to-LDS loads and the
exact wait counts is fixed by construction instead of by the compiler's
scheduler.  This script writes that block as a C string macro into
ring4_sched.inc; the kernel supplies the operands.  Run it after changing
the schedule parameters:

    python gen_ring4_sched.py            # writes ring4_sched.inc

Pipeline (the pages' software pipeline with a double-buffered operand ring,
"TIRx GEMM detailed technical notes", V4-V5, on gfx950 direct-to-LDS loads):

  * workgroup tile 256 x 256, 64-wide k steps, 2 LDS stages of 64 KiB
    (A rows at +0, B rows at +32 KiB; 128-byte rows, 16-byte chunk c of
    row r at chunk c ^ ((r / 2) mod 8)), 4 waves in a 2 x 2 grid, each wave
    owning 128 x 128 outputs = 8 x 8 blocks of v_mfma_f32_16x16x32_f16.
    Block (i, j) (A rows 16i.., B rows 16j..) accumulates in a[4B:4B+3],
    B = 8i + j (all 256 accumulation registers).  The 16x16x32 form is
    used because it holds a higher clock than 32x32x16 at the same work per
    cycle (it reads and writes half the accumulator bytes per FLOP);
  * a k step is 2 sub-steps of 32 k; a wave issues 16 loads per step (8 A,
    8 B row groups of 1 KiB) and 32 fragment reads (one 16-byte LDS read
    per block and sub-step);
  * each step has a release barrier, after the last reads of its stage
    (step j+2 may then refill it), and a publish barrier, after this wave's
    loads of step j+1 have landed (its fragment reads follow);
  * the prologue loads steps 0 and 1 (both stages are free); the last two
    steps issue no loads of their own and the last step has no barrier.

Two forms are generated.  The third form (generate3, macro
G16_RING4_KLOOP3, rung 8) places at most one instruction between two
MFMAs; the fourth (generate4, macro G16_RING4_KLOOP4, rung 10, the
library's choice) also issues each block's two sub-steps back to back
into its accumulator and takes a partial first step and a ring carried
from tile to tile (see their sections below).  The first two forms of the
ladder (one barrier per step, and the release/publish split with clumped
instructions) were removed once the third superseded them.

MFMA operand roles: the B block feeds srcA and the A block srcB, so lane l
of block (i, j) holds output row 16i + l%16 and the four consecutive output
columns 16j + 4*(l/16) + 0..3.

Operands expected by the block (see ring4.hpp): load offsets %[axQ],
%[bxQ] (the row groups' lane offsets less 1024*(Q mod 4), the instruction
offset the loads carry) (VGPR); fragment-read addresses %[raSK], %[rbSK]
for stage S and sub-step K (VGPR); buffer resources %[rsa], %[rsb]; the
wave's LDS load base %[lb] (the fourth form: %[lb0], %[lb1]); the byte
offsets %[ko] and %[kh] of the next two steps to load and the count
%[rem] of k steps (SGPR, all modified; %[kh] is scratch); and for the
epilogue the staging and store addresses %[ewJ], %[erQ], %[soQ], the
output resource %[rsd], the row-group stride %[gstr] and the scratch
%[sdo]; the fourth form also takes the head masks %[hm0], %[hm1].  The
accumulators a0..a255 and fragment buffers v128..v255 are fixed
registers of the block.
"""
from __future__ import annotations

import os
import sys

FRAG_BASE = 128
NB = 8           # 16-row blocks per wave tile side
NQ = NB * NB     # MFMAs per sub-step
KSUB = 2         # 32-wide sub-steps per 64-wide k step
NLOAD = 16       # direct-to-LDS loads per wave per k step


def freg(buf: int, op: str, idx: int) -> str:
    base = FRAG_BASE + 64 * buf + (0 if op == "a" else 32) + 4 * idx
    return f"v[{base}:{base + 3}]"


def areg(i: int, j: int) -> str:
    """Accumulator of block (i, j): a[4B:4B+3], B = 8i + j (the block owns
    fixed accumulation registers; they never leave the assembly block)."""
    b = NB * i + j
    return f"a[{4 * b}:{4 * b + 3}]"


# ---------------------------------------------------------------- epilogue
# In the last k step the output is written while the MFMAs of later rows
# still run.  Row group i (16 output rows, blocks (i, 0..7)) is final once
# its 8 MFMAs of the last sub-step are issued and the MFMA results are
# readable; it is then converted (v_accvgpr_read, v_cvt_pk_f16_f32: round to
# nearest even), staged in this wave's 4 KiB LDS buffer i % 2 (rows of 256
# bytes, 16-byte chunk c of row r at chunk c ^ (r mod 16)), read back as
# whole rows and stored with 16-byte buffer stores, four rows per
# instruction.  The stores are non-temporal: the output is not read again
# by the kernel, and streaming it out as it is written leaves less to write
# back when the kernel ends (1-2% faster at 4096^3 and 8192^3).  Temporaries live in the first fragment buffer (v128..v191),
# free once sub-step 0 is done.
EPI_T = 128   # v128..v159: converted blocks of a group
EPI_R = 160   # v160..v191: read-back rows, two groups


def epilogue_group(i: int, t_base: int = EPI_T, r_base: int = EPI_R) -> list[tuple[str, bool]]:
    """Instructions of row group i as (text, is_lds_op); t_base and r_base
    are the first of the 32 VGPRs for converted blocks and for read-back
    rows."""
    out: list[tuple[str, bool]] = []
    off = (i % 2) * 4096
    for j in range(NB):
        b = NB * i + j
        t = t_base + 4 * j
        for r in range(4):
            out.append((f"v_accvgpr_read_b32 v{t + r}, a{4 * b + r}", False))
        out.append((f"v_cvt_pk_f16_f32 v{t}, v{t}, v{t + 1}", False))
        out.append((f"v_cvt_pk_f16_f32 v{t + 1}, v{t + 2}, v{t + 3}", False))
        out.append((f"ds_write_b64 %[ew{j}], v[{t}:{t + 1}] offset:{off}", True))
    out.append(("s_waitcnt lgkmcnt(0)", False))
    rb = r_base + 16 * (i % 2)
    for q in range(4):
        out.append((f"ds_read_b128 v[{rb + 4 * q}:{rb + 4 * q + 3}], %[er{q}] offset:{off}", True))
    out.append(("s_waitcnt lgkmcnt(0)", False))
    for q in range(4):
        out.append((f"buffer_store_dwordx4 v[{rb + 4 * q}:{rb + 4 * q + 3}], %[so{q}], %[rsd], %[sdo] offen nt", False))
    out.append(("s_add_u32 %[sdo], %[sdo], %[gstr]", False))
    return out


class Emitter:
    def __init__(self) -> None:
        self.lines: list[str] = []
        self.lgkm: list[tuple] = []   # outstanding LDS reads, in issue order

    def op(self, s: str) -> None:
        self.lines.append(s)

    def label(self, s: str) -> None:
        self.lines.append(s + ":")

    # --- LDS fragment reads ------------------------------------------------
    def read(self, buf: int, op: str, idx: int, stage: int, kk: int) -> None:
        self.op(f"ds_read_b128 {freg(buf, op, idx)}, %[r{op}{stage}{kk}] offset:{2048 * idx}")
        self.lgkm.append((buf, op, idx))

    def wait_frag(self, *need: tuple) -> None:
        """lgkmcnt wait for the reads in `need` (LDS reads complete in
        order, so the count is the number issued after the newest one)."""
        pos = [self.lgkm.index(n) for n in need if n in self.lgkm]
        if not pos:
            return
        p = max(pos)
        after = len(self.lgkm) - 1 - p
        if after > 15:  # the counter field is 4 bits: wait for more
            p = len(self.lgkm) - 1 - 15
            after = 15
        self.op(f"s_waitcnt lgkmcnt({after})")
        del self.lgkm[: p + 1]

    def wait_all(self) -> None:
        self.op("s_waitcnt vmcnt(0) lgkmcnt(0)")
        self.lgkm.clear()

    # --- epilogue interleaved with the last sub-step -------------------------
    def epi_start(self, order: str) -> None:
        # row groups finish in row order only when the MFMAs go row by row
        assert order in ("ij", "snake"), "the interleaved epilogue needs a row-major MFMA order"
        self.op("s_mov_b32 %[sdo], 0")
        self.epi_q: list[tuple[str, bool]] = []
        self.epi_next = 0          # next row group to queue

    def epi_emit(self, text: str, lds: bool) -> None:
        self.op(text)
        if text == "s_waitcnt lgkmcnt(0)":
            self.lgkm.clear()
        elif lds:
            self.lgkm.append(("epi",))

    def epi_after_mfma(self, q: int, per_slot: int, delay: int) -> None:
        """After MFMA q of the last sub-step: queue the row groups whose
        MFMAs were all issued at least `delay` MFMAs ago, then emit up to
        per_slot queued instructions."""
        while self.epi_next < NB and q >= NB * self.epi_next + NB - 1 + delay:
            self.epi_q += epilogue_group(self.epi_next)
            self.epi_next += 1
        for _ in range(min(per_slot, len(self.epi_q))):
            self.epi_emit(*self.epi_q.pop(0))

    def epi_finish(self) -> None:
        """After the last MFMA: MFMA write -> accumulator read latency, then
        the remaining groups."""
        self.op("s_nop 7")
        self.op("s_nop 7")
        self.op("s_nop 7")
        while self.epi_next < NB:
            self.epi_q += epilogue_group(self.epi_next)
            self.epi_next += 1
        while self.epi_q:
            self.epi_emit(*self.epi_q.pop(0))

    # --- MFMA ----------------------------------------------------------------
    def mfma(self, buf: int, i: int, j: int, first: bool) -> None:
        self.wait_frag((buf, "a", i), (buf, "b", j))
        c = areg(i, j)
        self.op(f"v_mfma_f32_16x16x32_f16 {c}, {freg(buf, 'b', j)}, {freg(buf, 'a', i)}, {'0' if first else c}")


def mfma_block(q: int, order: str) -> tuple[int, int]:
    assert order in ("ij", "ji", "snake")
    """Block (i, j) of the q-th MFMA of a sub-step.  'ij': i outer (runs of
    8 MFMAs share an A fragment); 'ji': j outer; 'snake': i outer with j
    reversed on odd rows (the B fragment repeats across a row change)."""
    if order == "ji":
        return q % NB, q // NB
    i, j = q // NB, q % NB
    if order == "snake" and i % 2 == 1:
        j = NB - 1 - j
    return i, j


def read_order(order: str) -> list[tuple[str, int]]:
    """Fragment reads in the order the MFMAs first need them."""
    seen: list[tuple[str, int]] = []
    for q in range(NQ):
        i, j = mfma_block(q, order)
        for f in (("a", i), ("b", j)):
            if f not in seen:
                seen.append(f)
    return seen


# ------------------------------------------------------------ third form
# Release and publish barriers per k step, as in the second form, with at
# most one instruction besides the MFMA in each MFMA gap.
#
# With one wave per SIMD the wave issues about one instruction every four
# cycles and a 16x16x32 MFMA occupies the matrix core for 16: one other
# instruction fits between two MFMAs for free, and each further one delays
# the next MFMA.  This form places every instruction of a step in its own
# gap (gap g follows MFMA g of the step):
#
#   * gaps 0..15: the 16 fragment reads of sub-step 1 (this stage);
#   * gap rel-1: s_waitcnt lgkmcnt(0) (this wave is done reading the
#     stage), gap rel: the release barrier - the stage is free for step j+2;
#   * from gap rel+1, one every load_every gaps: the 16 loads of step j+2
#     into this stage; those beyond the step go out at the start of step
#     j+1.  Each 4 loads of an operand share one M0 value: load q lands at
#     M0 + 1024*(q mod 4) through the instruction offset, which also moves
#     the global address, so the lane offsets passed for it (%[axQ],
#     %[bxQ]) are the row-group offsets minus that amount.  This takes 12
#     of the 16 M0 writes and every s_nop out of the step;
#   * gap pub-1: s_waitcnt vmcnt(n) for step j+1's loads (n counts the
#     younger loads of step j+2), gap pub: the publish barrier;
#   * from gap max(pub+1, f0_start) (sub-step 0 is done with the first
#     fragment buffer): the 16 fragment reads of step j+1's sub-step 0 (the
#     other stage), one wait for them f0_lat gaps after the last;
#   * the step offsets, the step counter and the compare in the last gaps
#     before MFMA 127, the branches after it.
#
# A load has from its issue to the publish barrier of the next step to
# land: more than 1.5 steps for the first of a step, about half a step for
# the last, which covers operands streamed from HBM.


class Emitter3(Emitter):
    def load_imm(self, op: str, q: int, stage: int, koff: str = "ko") -> None:
        """Load q (0..7) of operand op into `stage` with the instruction
        offset; M0 must hold the base of q's group of 4.  koff: the SGPR
        with the step's byte offset along K."""
        imm = 1024 * (q % 4)
        off = f" offset:{imm}" if imm else ""
        self.op(f"buffer_load_dwordx4 %[{op}x{q}], %[rs{op}], %[{koff}] offen{off} lds")

    @staticmethod
    def m0_line(op: str, q: int, stage: int) -> str:
        base = stage * 65536 + (32768 if op == "b" else 0) + 4096 * (q // 4)
        return f"s_add_u32 m0, %[lb], {base}"


LOAD3 = [("a", q) for q in range(8)] + [("b", q) for q in range(8)]


def emit_step3(e: Emitter3, stage: int, first: bool, carried: bool, ahead: bool, has_next: bool, last: bool,
               tail: list[str], p: dict) -> None:
    """One 64-wide k step j reading `stage` in the third form.  carried:
    step j+1's late loads are issued in this step; ahead: this step starts
    the loads of step j+2; has_next: step j+1 exists (publish barrier, its
    fragment reads); last: the final step (epilogue).  %[ko] is the byte
    offset of step j+1 and %[kh] that of step j+2 during the step."""
    order = p.get("order", "snake")
    ro = read_order(order)
    ng = KSUB * NQ
    gaps: list[list[tuple]] = [[] for _ in range(ng)]

    def free(g: int) -> bool:
        return 0 <= g < ng and not gaps[g]

    def first_free(g: int) -> int:
        while not free(g):
            g += 1
            assert g < ng, "step too full"
        return g

    rel, pub, every = p["rel"], p["pub"], p["load_every"]
    slots = [rel + 1 + every * k for k in range(NLOAD)]          # step j+2's loads, step-j gaps
    limit = ng - 8                                               # the last gaps hold the tail
    own = [(k, s) for k, s in enumerate(slots) if s < limit] if ahead else []
    carry = [(k, max(0, s - ng)) for k, s in enumerate(slots) if s >= limit] if carried else []
    if not last:
        br = [t for t in tail if t.startswith(("s_cbranch", "s_branch"))]
        rest = [t for t in tail if t not in br]
        assert tail == rest + br, "branches close the tail"
        for k, t in enumerate(rest):
            gaps[ng - 1 - len(rest) + k].append(("text", t))
        for t in br:
            gaps[ng - 1].append(("text", t))
    for n, (op, idx) in enumerate(ro):
        gaps[p["f1_start"] + n * p["f1_every"]].append(("read", (1, op, idx, stage, 1)))
    assert rel - 1 > p["f1_start"] + (len(ro) - 1) * p["f1_every"]
    if ahead:
        gaps[rel - 1].append(("text", "s_waitcnt lgkmcnt(0)", "clear"))
        gaps[rel].append(("text", "s_barrier"))
    else:
        gaps[rel - 1].append(("text", "s_waitcnt lgkmcnt(0)", "clear"))
    if has_next:
        # the publish gaps are reserved before the loads are placed
        gaps[pub - 1].append(("publish_wait",))
        gaps[pub].append(("text", "s_barrier"))
    # loads in issue order: step j+1's carried loads (other stage, %[ko]),
    # then step j+2's own loads (this stage, %[kh]); an M0 write whenever
    # the group of 4 changes, in a free gap after the previous load
    seq = [(k, s, stage ^ 1, "ko") for (k, s) in carry] + [(k, s, stage, "kh") for (k, s) in own]
    prev, cur_m0 = -1, None
    placed = []
    for (k, s, st, koff) in seq:
        op, q = LOAD3[k]
        g = first_free(max(s, prev + 1))
        grp = (st, op, q // 4)
        if grp != cur_m0:
            m = next((x for x in range(g - 1, prev, -1) if free(x)), None)
            if m is None:
                m = first_free(prev + 1)
                g = first_free(m + 1)
            gaps[m].append(("text", Emitter3.m0_line(op, q, st)))
            cur_m0 = grp
        gaps[g].append(("load", op, q, st, koff))
        placed.append((g, koff))
        prev = g
    assert all(g < ng - 1 - 4 for g, _ in placed), "loads run into the tail"
    if has_next:
        # publish: step j+1's loads have landed in every wave; the own loads
        # of step j+2 issued so far are younger and need not wait
        n_young = sum(1 for g, koff in placed if koff == "kh" and g < pub - 1)
        assert not any(koff == "ko" and g >= pub - 1 for g, koff in placed), "carried load after the publish wait"
        gaps[pub - 1] = [("text", f"s_waitcnt vmcnt({n_young})")]
        g = max(p["f0_start"], pub + 1)
        lastr = g
        for (op, idx) in ro:
            g = first_free(g)
            gaps[g].append(("read", (0, op, idx, stage ^ 1, 0)))
            lastr = g
            g += p.get("f0_every", 1)
        gaps[first_free(lastr + p["f0_lat"])].append(("text", "s_waitcnt lgkmcnt(0)", "clear"))
    scc_writers = [g for g in range(ng) for it in gaps[g]
                   if it[0] == "text" and it[1].startswith(("s_add_u32", "s_sub_u32"))]
    cmp_at = [g for g in range(ng) for it in gaps[g] if it[0] == "text" and it[1].startswith("s_cmp")]
    assert not cmp_at or max(scc_writers, default=-1) < min(cmp_at), "SCC clobbered before the branch"

    for g in range(ng):
        kk, q = divmod(g, NQ)
        i, j = mfma_block(q, order)
        if last and kk == KSUB - 1 and q == 0:
            e.epi_start(order)
        e.mfma(kk, i, j, first and kk == 0)
        if last and kk == KSUB - 1:
            e.epi_after_mfma(q, p["epi_slot"], p["epi_delay"])
        for it in gaps[g]:
            if it[0] == "read":
                e.read(*it[1])
            elif it[0] == "load":
                e.load_imm(it[1], it[2], it[3], it[4])
            else:
                e.op(it[1])
                if len(it) > 2:
                    e.lgkm.clear()
    if last:
        e.epi_finish()
        for t in tail:
            e.op(t)


def generate3(p: dict) -> str:
    """The k loop in the third form.  During step j, %[ko] is the byte
    offset of step j+1 (its late loads) and %[kh] that of step j+2."""
    order = p.get("order", "snake")
    e = Emitter3()
    for stage in (0, 1):
        if stage:
            e.op("s_add_u32 %[ko], %[ko], 128")
        for (op, q) in LOAD3:
            if q % 4 == 0:
                e.op(Emitter3.m0_line(op, q, stage))
                e.op("s_nop 0")  # M0 write -> LDS-DMA read of M0
            e.load_imm(op, q, stage)
    e.op("s_add_u32 %[kh], %[ko], 128")
    e.op(f"s_waitcnt vmcnt({NLOAD})")
    e.op("s_barrier")
    for (op, idx) in read_order(order):
        e.read(0, op, idx, 0, 0)
    e.op("s_waitcnt lgkmcnt(0)")
    e.lgkm.clear()

    adv = ["s_add_u32 %[ko], %[ko], 128", "s_add_u32 %[kh], %[kh], 128"]
    sub = "s_sub_u32 %[rem], %[rem], 1"
    cmp2 = "s_cmp_eq_u32 %[rem], 2"

    def step(stage, first, carried, ahead, has_next, last, tail):
        e.lgkm = []
        emit_step3(e, stage, first, carried, ahead, has_next, last, tail, p)

    e.op(cmp2)
    e.op("s_cbranch_scc1 5f")
    step(0, True, False, True, True, False, adv + [sub, cmp2, "s_cbranch_scc1 6f"])
    e.label("1")
    step(1, False, True, True, True, False, adv + [sub, cmp2, "s_cbranch_scc1 8f"])
    step(0, False, True, True, True, False, adv + [sub, cmp2, "s_cbranch_scc1 6f", "s_branch 1b"])
    e.label("5")
    step(0, True, False, False, True, False, [sub, "s_branch 2f"])               # KT == 2
    e.label("6")
    step(1, False, True, False, True, False, [sub, "s_branch 3f"])                # step KT-2 in stage 1
    e.label("8")
    step(0, False, True, False, True, False, [sub])                               # step KT-2 in stage 0
    e.label("2")
    step(1, False, False, False, False, True, ["s_branch 4f"])                   # last step in stage 1
    e.label("3")
    step(0, False, False, False, False, True, [])                                 # last step in stage 0
    e.label("4")
    return "\n".join(e.lines)


DEFAULT3 = {
    "order": "snake",
    "f1_start": 0, "f1_every": 1,
    "rel": 24,                      # release barrier (its wait one gap earlier)
    "load_every": 8,                # step j+2's loads from gap rel + 1
    "pub": 88,                      # publish barrier (its wait one gap earlier)
    "f0_start": 64,
    "f0_lat": 12,
    "epi_slot": 8, "epi_delay": 2,
}


# ----------------------------------------------------------- fourth form
# The two sub-steps of a block back to back: for each block (i, j) of a
# row, the MFMA of sub-step 0 and then that of sub-step 1 into the same
# accumulator.  The second reads its accumulator straight from the first
# (a dependent 16x16x32 MFMA issues back to back without a stall), and the
# matrix core then spends less energy on accumulator traffic: a
# measurement of MFMA-only loops under the board's power limit ran 5%
# faster in this order.
#
# Both halves of a step's fragments are then live together, so the
# registers are laid out by what a row needs:
#   A(h, i) = v[64 + 32h + 4i]            A block i, sub-step h (one set);
#   B(p, h, j) = v[128 + 64p + 32h + 4j]  B block j, sub-step h, for the
#                                         steps of parity p (two sets).
# During step j the fragments of step j+1 are read from the other stage:
# its B blocks into the other set, its A blocks of row i once row i of step
# j is done (rows 6 and 7 at the start of step j+1).  Barriers: a release
# barrier at gap rel (this stage's last reads, the late A rows, are done;
# step j+2 may refill it) and a publish barrier at gap pub (step j+1's
# loads have landed; its fragment reads follow).  Loads and offsets are
# those of the third form, except step 0's (the head step below).
#
# K need not be a multiple of 64 here: the k origin moves back by
# 64 * steps - K elements so that step 0 is the partial one.  Its chunks
# that fall before a row's first element get offsets beyond the buffer's
# size (the head masks %[hm0], %[hm1], one per row-group parity, since the
# swizzle gives a lane a different chunk in even and odd row groups), so
# the hardware's range check returns zeros for them instead of reading
# memory; every later step is whole.

def a4(h: int, i: int) -> str:
    return f"v[{64 + 32 * h + 4 * i}:{64 + 32 * h + 4 * i + 3}]"


def b4(p: int, h: int, j: int) -> str:
    base = 128 + 64 * p + 32 * h + 4 * j
    return f"v[{base}:{base + 3}]"


def head_reg(op: str, q: int) -> int:
    """VGPR holding the head-step lane offset of load q of operand op."""
    return 64 + (8 if op == "b" else 0) + q


class Emitter4(Emitter3):
    @staticmethod
    def m0_line4(op: str, q: int, stage: int) -> str:
        """M0 for the group of 4 loads holding q, in logical stage `stage`
        (%[lb0], %[lb1]: the wave's load base in the physical stage that
        holds logical stage 0, 1 of this tile)."""
        return f"s_add_u32 m0, %[lb{stage}], {(32768 if op == 'b' else 0) + 4096 * (q // 4)}"

    def load_head(self, op: str, q: int) -> None:
        """Load q of operand op for step 0 (stage 0, %[ko] = 0) from the
        masked offset in head_reg(op, q), with the instruction offset."""
        imm = 1024 * (q % 4)
        off = f" offset:{imm}" if imm else ""
        self.op(f"buffer_load_dwordx4 v{head_reg(op, q)}, %[rs{op}], %[ko] offen{off} lds")

    @staticmethod
    def next_load(op: str, q: int) -> str:
        """Load q of operand op of the next tile's step 0 (its head step)
        from the masked offset in %[ht], soffset 0, with the instruction
        offset."""
        imm = 1024 * (q % 4)
        off = f" offset:{imm}" if imm else ""
        return f"buffer_load_dwordx4 %[ht], %[rs{op}n], 0 offen{off} lds"

    def read4(self, op: str, h: int, idx: int, stage: int, p: int) -> None:
        reg = a4(h, idx) if op == "a" else b4(p, h, idx)
        self.op(f"ds_read_b128 {reg}, %[r{op}{stage}{h}] offset:{2048 * idx}")
        self.lgkm.append((op, h, idx, p if op == "b" else None))

    def mfma4(self, p: int, h: int, i: int, j: int, first: bool) -> None:
        self.wait_frag(("a", h, i, None), ("b", h, j, p))
        c = areg(i, j)
        self.op(f"v_mfma_f32_16x16x32_f16 {c}, {b4(p, h, j)}, {a4(h, i)}, {'0' if first else c}")

    def epi_after4(self, g: int, per_slot: int, delay: int, t_base: int, r_base: int) -> None:
        """After MFMA g of the last step: queue the rows whose MFMAs were all
        issued at least `delay` MFMAs ago, emit up to per_slot queued
        instructions."""
        while self.epi_next < NB and g >= 2 * NB * self.epi_next + 2 * NB - 1 + delay:
            self.epi_q += epilogue_group(self.epi_next, t_base, r_base)
            self.epi_next += 1
        for _ in range(min(per_slot, len(self.epi_q))):
            self.epi_emit(*self.epi_q.pop(0))

    def epi_finish4(self, t_base: int, r_base: int) -> None:
        self.op("s_nop 7")
        self.op("s_nop 7")
        self.op("s_nop 7")
        while self.epi_next < NB:
            self.epi_q += epilogue_group(self.epi_next, t_base, r_base)
            self.epi_next += 1
        while self.epi_q:
            self.epi_emit(*self.epi_q.pop(0))


def late_rows4(p: dict) -> list[int]:
    """Rows whose A fragments of step j+1 are read at the start of step j+1
    (their row of step j ends too late in the step)."""
    return [i for i in range(NB) if 2 * NB * i + 2 * NB + p["a_delay"] >= p["read_limit"]]


def emit_step4(e: Emitter4, stage: int, first: bool, carried: bool, ahead: bool, has_next: bool, last: bool,
               tail: list[str], p: dict, nxt: bool = False) -> None:
    """One 64-wide k step j reading `stage` (B fragments in set stage) in
    the fourth form; flags as in emit_step3, and nxt: the last step also
    loads the next tile's step 0.  The late A rows of this step
    are read at its start unless `first` (the prologue read them)."""
    order = p.get("order", "snake")
    ng = KSUB * NQ
    par = stage                                  # B fragment set of this step
    gaps: list[list[tuple]] = [[] for _ in range(ng)]
    late = late_rows4(p)

    def free(g: int) -> bool:
        return 0 <= g < ng and not gaps[g]

    def first_free(g: int) -> int:
        while not free(g):
            g += 1
            assert g < ng, "step too full"
        return g

    rel, pub, every = p["rel"], p["pub"], p["load_every"]
    if not last:
        br = [t for t in tail if t.startswith(("s_cbranch", "s_branch"))]
        rest = [t for t in tail if t not in br]
        assert tail == rest + br, "branches close the tail"
        for k, t in enumerate(rest):
            gaps[ng - 1 - len(rest) + k].append(("text", t))
        for t in br:
            gaps[ng - 1].append(("text", t))
    # this step's late A rows (from this stage)
    g = 0
    if not first:
        for i in late:
            for h in range(KSUB):
                g = first_free(g)
                gaps[g].append(("read", ("a", h, i, stage, par)))
                g += 1
    if ahead:
        assert g < rel - 1, "late reads after the release"
        gaps[rel - 1].append(("text", "s_waitcnt lgkmcnt(0)", "clear"))
        gaps[rel].append(("text", "s_barrier"))
    if has_next:
        gaps[pub - 1].append(("publish_wait",))
        gaps[pub].append(("text", "s_barrier"))
    # loads: as in the third form
    slots = [rel + 1 + every * k for k in range(NLOAD)]
    limit = ng - 8
    own = [(k, s_) for k, s_ in enumerate(slots) if s_ < limit] if ahead else []
    carry = [(k, max(0, s_ - ng)) for k, s_ in enumerate(slots) if s_ >= limit] if carried else []
    seq = [(k, s_, stage ^ 1, "ko") for (k, s_) in carry] + [(k, s_, stage, "kh") for (k, s_) in own]
    prev, cur_m0 = -1, None
    placed = []
    for (k, s_, st, koff) in seq:
        op, q = LOAD3[k]
        gg = first_free(max(s_, prev + 1))
        grp = (st, op, q // 4)
        if grp != cur_m0:
            m = next((x for x in range(gg - 1, prev, -1) if free(x)), None)
            if m is None:
                m = first_free(prev + 1)
                gg = first_free(m + 1)
            gaps[m].append(("text", Emitter4.m0_line4(op, q, st)))
            cur_m0 = grp
        gaps[gg].append(("load", op, q, st, koff))
        placed.append((gg, koff))
        prev = gg
    assert all(gg < ng - 1 - 4 for gg, _ in placed), "loads run into the tail"
    if last and nxt:
        # the next tile's step 0 into the other stage (free since the
        # previous step's publish barrier: its reads were all waited for
        # there): M0, the masked offset and the load in gaps of their own,
        # one load every nxt_every gaps from nxt_start, ahead of most of the
        # epilogue's stores
        gl = p["nxt_start"] - p["nxt_every"]
        for k, (op, q) in enumerate(LOAD3):
            prev_load = gl
            gl = first_free(max(prev_load + p["nxt_every"], p["nxt_start"]))
            before = [x for x in range(gl - 1, prev_load, -1) if free(x)]
            need = 2 if q % 4 == 0 else 1
            assert len(before) >= need, "no room for the next-tile load's M0 and offset"
            gaps[before[0]].append(("text", f"v_or_b32 %[ht], %[{op}x{q}], %[hm{q % 2}]"))
            if q % 4 == 0:
                gaps[before[1]].append(("text", Emitter4.m0_line4(op, q, stage ^ 1)))
            gaps[gl].append(("text", Emitter4.next_load(op, q)))
        assert gl < ng - 8, "next-tile loads run into the end of the step"
    if has_next:
        n_young = sum(1 for gg, koff in placed if koff == "kh" and gg < pub - 1)
        assert not any(koff == "ko" and gg >= pub - 1 for gg, koff in placed), "carried load after the publish wait"
        # (the late A reads of this step, long done, are waited for too: no
        # barrier is crossed with LDS reads in flight)
        gaps[pub - 1] = [("text", f"s_waitcnt vmcnt({n_young}) lgkmcnt(0)", "clear")]
        # step j+1's fragments (other stage): A row 0, all B blocks, then
        # the other A rows as their rows of this step finish
        reads = [("a", h, 0, pub + 1) for h in range(KSUB) if 0 not in late]
        reads += [("b", h, j, pub + 1) for j in range(NB) for h in range(KSUB)]
        reads += [("a", h, i, max(pub + 1, 2 * NB * i + 2 * NB + p["a_delay"])) for i in range(1, NB)
                  if i not in late for h in range(KSUB)]
        reads.sort(key=lambda r: r[3])
        gg, lastr = pub + 1, pub + 1
        for (op, h, idx, earliest) in reads:
            gg = first_free(max(gg, earliest))
            assert gg < p["read_limit"], "next-step reads beyond the read limit"
            gaps[gg].append(("read", (op, h, idx, stage ^ 1, par ^ 1)))
            lastr = gg
            gg += p["read_every"]
        gaps[first_free(lastr + p["f0_lat"])].append(("text", "s_waitcnt lgkmcnt(0)", "clear"))
    scc_writers = [gg for gg in range(ng) for it in gaps[gg]
                   if it[0] == "text" and it[1].startswith(("s_add_u32", "s_sub_u32"))]
    cmp_at = [gg for gg in range(ng) for it in gaps[gg] if it[0] == "text" and it[1].startswith("s_cmp")]
    assert not cmp_at or max(scc_writers, default=-1) < min(cmp_at), "SCC clobbered before the branch"

    t_base = epi_set4(par)
    step_at = len(e.lines)
    for gg in range(ng):
        pq, h = divmod(gg, 2)
        i, j = mfma_block(pq, order)
        if last and gg == 0:
            e.epi_start(order)
        e.mfma4(par, h, i, j, first and gg < 2 * NQ and per_block_first(gg))
        if last:
            e.epi_after4(gg, p["epi_slot"], p["epi_delay"], t_base, t_base + 32)
        for it in gaps[gg]:
            if it[0] == "read":
                e.read4(*it[1])
            elif it[0] == "load":
                e.load_imm(it[1], it[2], it[3], it[4])
            else:
                e.op(it[1])
                if len(it) > 2:
                    e.lgkm.clear()
    if last:
        e.epi_finish4(t_base, t_base + 32)
        if nxt:
            # stores issued after the last next-tile load: the next tile
            # waits for its step 0 with them (and its step-1 loads) in flight
            lines = e.lines[step_at:]
            last_load = max(n for n, ln in enumerate(lines) if ln.startswith("buffer_load_dwordx4 %[ht]"))
            e.s_after.append(sum(1 for ln in lines[last_load:] if ln.startswith("buffer_store_dwordx4")))
        for t in tail:
            e.op(t)


def epi_set4(par: int) -> int:
    """First VGPR of the last step's epilogue temporaries: the B set of the
    other parity, idle in the last step."""
    return 128 + 64 * (par ^ 1)


def per_block_first(gg: int) -> bool:
    """In the first step, the sub-step-0 MFMA of each block starts it from 0."""
    return gg % 2 == 0


def generate4(p: dict) -> str:
    """The k loop in the fourth form (same branch structure and offsets as
    the third)."""
    order = p.get("order", "snake")
    e = Emitter4()
    e.s_after = []
    # step 0 may be a partial step (K not a multiple of 64): its lane
    # offsets are OR-ed with the head mask of the row group's parity, which
    # moves the chunks before the row's first element out of the buffer
    # (they land as zeros); the mask is 0 when K is a multiple of 64.  The
    # offsets go to v64..v79, free until step 0's fragment reads.  A tile
    # loads its own step 0 here when %[first] != 0; otherwise its step 0
    # was loaded during the last step of the tile before (that step ran
    # with %[hasn] != 0), ahead of that tile's output stores.
    e.op("s_cmp_eq_u32 %[first], 0")
    e.op("s_cbranch_scc1 11f")
    for (op, q) in LOAD3:
        e.op(f"v_or_b32 v{head_reg(op, q)}, %[{op}x{q}], %[hm{q % 2}]")
    for (op, q) in LOAD3:
        if q % 4 == 0:
            e.op(Emitter4.m0_line4(op, q, 0))
            e.op("s_nop 0")  # M0 write -> LDS-DMA read of M0
        e.load_head(op, q)
    e.label("11")
    e.op("s_add_u32 %[ko], %[ko], 128")
    for (op, q) in LOAD3:
        if q % 4 == 0:
            e.op(Emitter4.m0_line4(op, q, 1))
            e.op("s_nop 0")
        e.load_imm(op, q, 1)
    e.op("s_add_u32 %[kh], %[ko], 128")
    e.op("s_cmp_eq_u32 %[first], 0")
    e.op("s_cbranch_scc1 12f")
    e.op(f"s_waitcnt vmcnt({NLOAD})")
    e.op("s_branch 13f")
    e.label("12")
    e.op("s_waitcnt vmcnt(@NEXT_WAIT@)")   # step-1 loads and the tile before's late stores
    e.label("13")
    e.op("s_barrier")
    # all fragments of step 0, in the order the first MFMAs need them
    e.read4("a", 0, 0, 0, 0)
    e.read4("a", 1, 0, 0, 0)
    for j in range(NB):
        for h in range(KSUB):
            e.read4("b", h, j, 0, 0)
    for i in range(1, NB):
        for h in range(KSUB):
            e.read4("a", h, i, 0, 0)
    pro = list(e.lgkm)

    adv = ["s_add_u32 %[ko], %[ko], 128", "s_add_u32 %[kh], %[kh], 128"]
    sub = "s_sub_u32 %[rem], %[rem], 1"
    cmp2 = "s_cmp_eq_u32 %[rem], 2"

    def step(stage, first, carried, ahead, has_next, last, tail, nxt=False):
        e.lgkm = list(pro) if first else []
        emit_step4(e, stage, first, carried, ahead, has_next, last, tail, p, nxt)

    e.op(cmp2)
    e.op("s_cbranch_scc1 5f")
    step(0, True, False, True, True, False, adv + [sub, cmp2, "s_cbranch_scc1 6f"])
    e.label("1")
    step(1, False, True, True, True, False, adv + [sub, cmp2, "s_cbranch_scc1 8f"])
    step(0, False, True, True, True, False, adv + [sub, cmp2, "s_cbranch_scc1 6f", "s_branch 1b"])
    e.label("5")
    step(0, True, False, False, True, False, [sub, "s_branch 2f"])               # KT == 2
    e.label("6")
    step(1, False, True, False, True, False, [sub, "s_branch 3f"])                # step KT-2 in stage 1
    e.label("8")
    step(0, False, True, False, True, False, [sub])                               # step KT-2 in stage 0
    # the last step, in either stage, with the next tile's step-0 loads
    # when %[hasn] != 0 and without them otherwise
    e.label("2")
    e.op("s_cmp_eq_u32 %[hasn], 0")
    e.op("s_cbranch_scc1 14f")
    step(1, False, False, False, False, True, ["s_branch 4f"], nxt=True)         # last step in stage 1
    e.label("14")
    step(1, False, False, False, False, True, ["s_branch 4f"])
    e.label("3")
    e.op("s_cmp_eq_u32 %[hasn], 0")
    e.op("s_cbranch_scc1 15f")
    step(0, False, False, False, False, True, ["s_branch 4f"], nxt=True)         # last step in stage 0
    e.label("15")
    step(0, False, False, False, False, True, [])
    e.label("4")
    assert len(set(e.s_after)) == 1, "both last-step copies leave the same stores after the next-tile loads"
    wait = NLOAD + e.s_after[0]
    assert wait < 64, "vmcnt is 6 bits"
    return "\n".join(e.lines).replace("@NEXT_WAIT@", str(wait))


DEFAULT4 = {
    "order": "snake",
    "rel": 12,                      # release barrier (its wait one gap earlier)
    "load_every": 8,                # step j+2's loads from gap rel + 1
    "pub": 64,                      # publish barrier (its wait one gap earlier)
    "a_delay": 1,                   # gaps between a row's last MFMA and the next step's read of its A
    "read_limit": 112,              # next-step reads end before this gap; later A rows move to the next step
    "read_every": 1,
    "f0_lat": 8,
    "epi_slot": 8, "epi_delay": 2,
    "nxt_start": 6,                 # the next tile's step-0 loads in the last step: from this gap ...
    "nxt_every": 4,                 # ... one every this many gaps
}


def as_macro(name: str, text: str) -> str:
    body = [f'    "{ln}\\n"' for ln in text.split("\n")]
    return f"#define {name} \\\n" + " \\\n".join(body) + "\n"


def params_line(p: dict) -> str:
    return ", ".join(f"{k}={v}" for k, v in p.items())


def main(argv: list[str]) -> int:
    here = os.path.dirname(os.path.abspath(__file__))
    out = os.path.join(here, "ring4_sched.inc")
    text3 = generate3(DEFAULT3)
    text4 = generate4(DEFAULT4)
    with open(out, "w") as f:
        f.write("// Generated by gen_ring4_sched.py.  Do not edit.\n")
        f.write("// G16_RING4_KLOOP3: release and publish barriers per k step, one instruction per MFMA gap; " + params_line(DEFAULT3) + ".\n")
        f.write(as_macro("G16_RING4_KLOOP3", text3))
        f.write("// G16_RING4_KLOOP4: each block's two sub-steps back to back, release and publish barriers; " + params_line(DEFAULT4) + ".\n")
        f.write(as_macro("G16_RING4_KLOOP4", text4))
    print(out, sum(len(t.split("\n")) for t in (text3, text4)), "lines")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
