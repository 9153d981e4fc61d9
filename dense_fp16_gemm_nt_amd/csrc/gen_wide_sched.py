"""Generate the k loop of the wide four-wave ring (ring_wide.hpp, rung 11).

The pages' last step before library parity grows the output tile that one
staged B tile feeds: two consumer warpgroups share each B tile ("GEMM III",
Step 9; "TIRx GEMM detailed technical notes", V9 "Why Share B?").  Here a
workgroup tile is 384 x 256: each 64-wide k step stages a 384-row A band and
a 256-row B band in LDS, and each B column block of 128 feeds two waves of
192 A rows, so operand bytes per FLOP (from L2 into LDS, and from LDS into
registers) drop by a sixth against the 256 x 256 tile of rung 10.

The gfx950 budget sets the form:
  * 4 waves in a 2 x 2 grid, each owning 192 x 128 outputs = 12 x 8 blocks
    of v_mfma_f32_16x16x32_f16: 384 accumulation registers, rows 0-7 in the
    256 AGPRs (block (i, j) at a[4(8i + j)]) and rows 8-11 in VGPRs
    (v[128 + 4(8(i - 8) + j)]);
  * the 128 VGPRs left hold one set of B fragments (B(h, j) at
    v[64 + 32h + 4j]), a ring of two A rows (A(slot, h) at v[48 + 8 slot +
    4h]) and, in v0-v47, the operands the compiler places;
  * LDS holds two stages of 80 KiB (A rows at +0, B rows at +48 KiB,
    128-byte rows swizzled as in rung 10), all 160 KiB: the epilogue stages
    its rows in the stage the last step does not read.

Schedule of one k step (192 MFMAs; gap g follows MFMA g):
  * rows in position order R (0..11; the last step 8..11, 0..7 so that the
    VGPR rows are written out first and free their registers for the
    AGPR rows' epilogue), each row's blocks in snake order that alternates
    with the stage parity, each block's two sub-steps back to back into its
    accumulator (rung 10's pairs);
  * during position p the A fragments of position p + 1 are read into the
    ring slot position p - 1 has finished with;
  * one barrier per step, after MFMA 175 (the last of position 10): it
    releases the stage (every read of the step has completed) and publishes
    the next step (this wave's loads of it have landed: vmcnt(0));
  * after it, the next step's B fragments are read as the last row frees
    them (the block the last row finishes last is read by the next step at
    its own start) and its first A row into the free ring slot; the loads
    of step j+2 go into the released stage, one every `load_every` gaps,
    the later ones carried into the next step.  Loads closer together
    than ~6 gaps queue at the XCD's L2 (every 2, 3, 4 gaps: 6.6%, 3.6%,
    1% slower than every 6 on 12288 x 4096 x 4096); further apart than ~8
    the last ones land after the barrier's wait (every 9: 3.8% slower).
"""
from __future__ import annotations

import os
import re
import sys

NBM, NBN, KSUB = 12, 8, 2
NG = NBM * NBN * KSUB            # MFMAs (gaps) per k step
A_LOADS, B_LOADS = 12, 8
STAGE = 81920                    # bytes per ring stage
B_OFF = 49152                    # B rows within a stage
LOADS = [("a", q) for q in range(A_LOADS)] + [("b", q) for q in range(B_LOADS)]
NLOAD = len(LOADS)
BAR_GAP = 16 * 11 - 1            # barrier after MFMA 175 (the last of position 10)


def acc(i: int, j: int) -> str:
    if i < 8:
        b = 4 * (NBN * i + j)
        return f"a[{b}:{b + 3}]"
    b = 128 + 4 * (NBN * (i - 8) + j)
    return f"v[{b}:{b + 3}]"


def acc_base(i: int, j: int) -> int:
    return 4 * (NBN * i + j) if i < 8 else 128 + 4 * (NBN * (i - 8) + j)


def breg(h: int, j: int) -> str:
    b = 64 + 32 * h + 4 * j
    return f"v[{b}:{b + 3}]"


def areg(slot: int, h: int) -> str:
    b = 48 + 8 * slot + 4 * h
    return f"v[{b}:{b + 3}]"


def rows_of(last: bool) -> list[int]:
    return [8, 9, 10, 11, 0, 1, 2, 3, 4, 5, 6, 7] if last else list(range(NBM))


def col_order(pos: int, stage: int) -> list[int]:
    """Block columns of the row at position `pos`: snake order whose start
    alternates with the stage parity, so that the last row of a step frees
    the B blocks in the order the next step's first row needs them."""
    return list(range(NBN)) if (pos + stage) % 2 == 0 else list(range(NBN - 1, -1, -1))


class Emitter:
    def __init__(self) -> None:
        self.lines: list[str] = []
        self.lgkm: list[str] = []        # destination register of each outstanding LDS read, in issue order

    def op(self, s: str) -> None:
        self.lines.append(s)

    def label(self, s: str) -> None:
        self.lines.append(s + ":")

    def read(self, reg: str, base: str, off: int) -> None:
        self.op(f"ds_read_b128 {reg}, %[{base}] offset:{off}")
        self.lgkm.append(reg)

    def read_a(self, stage: int, h: int, i: int, slot: int) -> None:
        self.read(areg(slot, h), f"ra{stage}{h}", 2048 * i)

    def read_b(self, stage: int, h: int, j: int) -> None:
        self.read(breg(h, j), f"rb{stage}{h}", 2048 * j)

    def wait_regs(self, *regs: str) -> None:
        """lgkmcnt wait for the newest reads into `regs` (LDS reads complete
        in issue order)."""
        pos = [max(k for k, r in enumerate(self.lgkm) if r == x) for x in regs if x in self.lgkm]
        if not pos:
            return
        p = max(pos)
        after = len(self.lgkm) - 1 - p
        if after > 15:
            p = len(self.lgkm) - 16
            after = 15
        self.op(f"s_waitcnt lgkmcnt({after})")
        del self.lgkm[: p + 1]

    def clear(self) -> None:
        self.lgkm.clear()

    def mfma(self, i: int, j: int, h: int, slot: int, zero: bool) -> None:
        self.wait_regs(areg(slot, h), breg(h, j))
        c = acc(i, j)
        self.op(f"v_mfma_f32_16x16x32_f16 {c}, {breg(h, j)}, {areg(slot, h)}, {'0' if zero else c}")


def m0_line(op: str, q: int, stage: int) -> str:
    base = stage * STAGE + 4096 * (q // 4)
    return f"s_add_u32 m0, %[lb{op}], {base}"


def load_line(op: str, q: int, koff: str) -> str:
    imm = 1024 * (q % 4)
    off = f" offset:{imm}" if imm else ""
    return f"buffer_load_dwordx4 %[{op}x{q}], %[rs{op}], %[{koff}] offen{off} lds"


# ------------------------------------------------------------- epilogue
# A finished row (16 output rows x 128 columns) is rounded to fp16 (round
# to nearest even), staged in the wave's 8 KiB of the idle stage (two 4 KiB
# buffers by position parity; rows of 256 bytes, 16-byte chunk c of row r
# at chunk c ^ (r mod 16)), read back as whole rows and written with
# non-temporal 16-byte stores, four rows per instruction.  VGPR rows are
# converted in place and read back into their own first 16 registers; AGPR
# rows go through the registers of rows 8-11 once those are written out.
# The generator tracks the registers every issued store reads and waits
# (vmcnt, counting the younger stores) before writing any of them again.
EPI_T = 128                                   # AGPR rows: converted blocks, v128..v159
EPI_R = [160, 176, 192, 208, 224, 240]        # AGPR rows: read-back rows, rotating over six sets


def epilogue_row(i: int, pos: int) -> list[tuple[str, str]]:
    """(text, kind) of row i's epilogue at position `pos` of the last step;
    kind is 'lds', 'store', 'valu' or 'wait'."""
    out: list[tuple[str, str]] = []
    off = (pos % 2) * 4096
    for j in range(NBN):
        if i >= 8:
            t = acc_base(i, j)
        else:
            t = EPI_T + 4 * j
            for r in range(4):
                out.append((f"v_accvgpr_read_b32 v{t + r}, a{acc_base(i, j) + r}", "valu"))
        out.append((f"v_cvt_pk_f16_f32 v{t}, v{t}, v{t + 1}", "valu"))
        out.append((f"v_cvt_pk_f16_f32 v{t + 1}, v{t + 2}, v{t + 3}", "valu"))
        out.append((f"ds_write_b64 %[ew{j}], v[{t}:{t + 1}] offset:{off}", "lds"))
    out.append(("s_waitcnt lgkmcnt(0)", "wait"))
    rb = acc_base(i, 0) if i >= 8 else EPI_R[(pos - 4) % len(EPI_R)]
    for q in range(4):
        out.append((f"ds_read_b128 v[{rb + 4 * q}:{rb + 4 * q + 3}], %[er{q}] offset:{off}", "lds"))
    out.append(("s_waitcnt lgkmcnt(0)", "wait"))
    out.append((f"s_mul_i32 %[sdo], %[gstr], {i}", "salu"))
    for q in range(4):
        out.append((f"buffer_store_dwordx4 v[{rb + 4 * q}:{rb + 4 * q + 3}], %[so{q}], %[rsd], %[sdo] offen nt", "store"))
    return out


def emit_step(e: Emitter, stage: int, first: bool, carried: bool, ahead: bool, has_next: bool, next_last: bool,
              last: bool, tail: list[str], p: dict) -> None:
    """One 64-wide k step j reading `stage`.  first: the prologue read this
    step's B fragments and first A row; carried: the loads of step j+1 that
    step j-1 did not issue go out here (%[ko]); ahead: this step loads step
    j+2 into its stage after the barrier (%[kh]); has_next: a step follows
    (barrier, its fragment reads); next_last: that step is the last (its
    rows start at 8); last: this is the last step (epilogue)."""
    gaps: list[list[tuple]] = [[] for _ in range(NG)]
    R = rows_of(last)
    seq = []                                    # (i, j, h, slot, pos) per MFMA
    for pos, i in enumerate(R):
        for j in col_order(pos, stage):
            for h in range(KSUB):
                seq.append((i, j, h, pos % 2, pos))

    # a gap holds at most one LDS read, one load and two other
    # instructions (measured on MI355X: up to three SALU or VALU
    # instructions between two 16x16x32 MFMAs cost no issue cycles, a
    # second LDS read or load does)
    cap = {"read": 1, "load": 1, "text": 2}

    def kind(it: tuple) -> str:
        return "read" if it[0].startswith("read") else ("load" if it[0] == "load" else "text")

    def free(g: int, k: str = "text") -> bool:
        return 0 <= g < NG and sum(1 for it in gaps[g] if kind(it) == k) < cap[k] and len(gaps[g]) < 3

    def first_free(g: int, k: str = "text") -> int:
        while not free(g, k):
            g += 1
            assert g < NG, "step too full"
        return g

    # the tail: step offsets, counter and compare, branches after MFMA NG-1
    if not last:
        br = [t for t in tail if t.startswith(("s_cbranch", "s_branch"))]
        rest = [t for t in tail if t not in br]
        assert tail == rest + br, "branches close the tail"
        for k, t in enumerate(rest):
            gaps[NG - 1 - len(rest) + k].append(("text", t))
        for t in br:
            gaps[NG - 1].append(("text", t))
    # this step's B block that the previous step's last row freed last
    g = 0
    if not first:
        prev_cols = col_order(NBM - 1, stage ^ 1)
        jl = prev_cols[-1]
        for h in range(KSUB):
            g = first_free(g, "read")
            gaps[g].append(("read_b", stage, h, jl))
            g += 1
    # A rows of positions 1..11 from this stage, each during the position before
    for pos in range(NBM - 1):
        gg = 16 * pos + p["a_delay"]
        for h in range(KSUB):
            gg = first_free(gg, "read")
            gaps[gg].append(("read_a", stage, h, R[pos + 1], (pos + 1) % 2))
            gg += 1
    if has_next:
        gaps[BAR_GAP - 1].append(("text", "s_waitcnt vmcnt(0) lgkmcnt(0)", "clear"))
        gaps[BAR_GAP].append(("text", "s_barrier"))
        # next step: the B blocks the last row frees (one gap after the
        # block's second MFMA; the last one is read by the next step itself)
        # its first row's A (ring slot 0, free since position 10 ended)
        i0 = rows_of(next_last)[0]
        gg = BAR_GAP + p["a_delay"]
        for h in range(KSUB):
            gg = first_free(gg, "read")
            gaps[gg].append(("read_a", stage ^ 1, h, i0, 0))
        cols = col_order(NBM - 1, stage)
        for t, j in enumerate(cols[:-1]):
            gg = BAR_GAP + 2 * t + 3          # one MFMA after the block's second MFMA
            for h in range(KSUB):
                gg = first_free(gg, "read")
                gaps[gg].append(("read_b", stage ^ 1, h, j))
    # loads: step j+1's carried loads (other stage, %[ko]) from gap 0, then
    # step j+2's own loads (this stage, %[kh]) after the barrier
    slots = [BAR_GAP + 1 + p["load_every"] * k for k in range(NLOAD)]
    limit = NG - 8
    own = [(k, s) for k, s in enumerate(slots) if s < limit] if ahead else []
    carry = [(k, 1 + max(0, s - NG)) for k, s in enumerate(slots) if s >= limit] if carried else []
    plan = [(k, s, stage ^ 1, "ko") for (k, s) in carry] + [(k, s, stage, "kh") for (k, s) in own]
    prev, cur_m0 = -1, None
    for (k, s, st, koff) in plan:
        op, q = LOADS[k]
        gg = first_free(max(s, prev + 1), "load")
        grp = (st, op, q // 4)
        if grp != cur_m0:
            m = next((x for x in range(gg - 1, prev, -1) if free(x)), None)
            if m is None:
                m = first_free(prev + 1)
                gg = first_free(m + 1, "load")
            gaps[m].append(("text", m0_line(op, q, st)))
            cur_m0 = grp
        gaps[gg].append(("load", op, q, koff))
        prev = gg
        assert gg < NG - 1 - 4, "loads run into the tail"
    assert not carried or all(s < BAR_GAP - 1 for (_, s, _, koff) in plan if koff == "ko"), "carried loads after the wait"
    scc_writers = [gg for gg in range(NG) for it in gaps[gg]
                   if it[0] == "text" and it[1].startswith(("s_add_u32", "s_sub_u32"))]
    cmp_at = [gg for gg in range(NG) for it in gaps[gg] if it[0] == "text" and it[1].startswith("s_cmp")]
    assert not cmp_at or max(scc_writers, default=-1) < min(cmp_at), "SCC clobbered before the branch"

    # emit, with the epilogue interleaved in the last step
    queue: list[tuple[str, str]] = []
    done_pos = 0
    stores_issued: list[set] = []               # registers each issued store reads, in order
    for gg, (i, j, h, slot, pos) in enumerate(seq):
        e.mfma(i, j, h, slot, first and per_block_first(gg, seq))
        if last:
            while done_pos < NBM and gg >= 16 * done_pos + 15 + p["epi_delay"]:
                queue += epilogue_row(R[done_pos], done_pos)
                done_pos += 1
            for _ in range(min(p["epi_slot"], len(queue))):
                emit_epi(e, queue.pop(0), stores_issued)
        # branches close their gap
        items = sorted(gaps[gg], key=lambda it: it[0] == "text" and it[1].startswith(("s_cbranch", "s_branch")))
        for it in items:
            if it[0] == "read_a":
                e.read_a(it[1], it[2], it[3], it[4])
            elif it[0] == "read_b":
                e.read_b(it[1], it[2], it[3])
            elif it[0] == "load":
                e.op(load_line(it[1], it[2], it[3]))
            else:
                e.op(it[1])
                if len(it) > 2:
                    e.clear()
    if last:
        e.op("s_nop 7")
        e.op("s_nop 7")
        e.op("s_nop 7")
        while done_pos < NBM:
            ri = R[done_pos]
            queue += epilogue_row(ri, done_pos)
            done_pos += 1
        while queue:
            emit_epi(e, queue.pop(0), stores_issued)
        for t in tail:
            e.op(t)


def vregs(spec: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return {int(spec[1:])}


def emit_epi(e: Emitter, item: tuple[str, str], stores_issued: list[set]) -> None:
    """Emit one epilogue instruction; before it writes a register that an
    issued store reads, wait until that store is done (the last step issues
    no loads, so vmcnt counts the younger stores only)."""
    text, kind = item
    dst = set()
    if text.startswith(("v_accvgpr_read_b32", "v_cvt_pk_f16_f32", "ds_read_b128")):
        dst = vregs(text.split()[1].rstrip(","))
    hit = [k for k, regs in enumerate(stores_issued) if regs & dst]
    if hit:
        younger = len(stores_issued) - 1 - max(hit)
        assert younger < 64, "vmcnt is 6 bits"
        e.op(f"s_waitcnt vmcnt({younger})")
        del stores_issued[: max(hit) + 1]
    e.op(text)
    if kind == "lds":
        e.lgkm.append("epi")
    elif kind == "wait":
        e.clear()
    elif kind == "store":
        stores_issued.append(vregs(text.split()[1].rstrip(",")))


def per_block_first(gg: int, seq) -> bool:
    return seq[gg][2] == 0


def generate(p: dict) -> str:
    """The k loop of rung 11 (same branch structure as the four-wave ring's
    third form): %[ko] is the byte offset of step j+1 and %[kh] that of step
    j+2 during step j."""
    e = Emitter()
    for stage in (0, 1):
        if stage:
            e.op("s_add_u32 %[ko], %[ko], 128")
        for (op, q) in LOADS:
            if q % 4 == 0:
                e.op(m0_line(op, q, stage))
                e.op("s_nop 0")  # M0 write -> LDS-DMA read of M0
            e.op(load_line(op, q, "ko"))
    e.op("s_add_u32 %[kh], %[ko], 128")
    e.op(f"s_waitcnt vmcnt({NLOAD})")
    e.op("s_barrier")
    # the first step's B fragments and first A row (the first step's rows
    # start at 0 unless it is also the last)
    for j in range(NBN):
        for h in range(KSUB):
            e.read_b(0, h, j)
    pro = list(e.lgkm)

    adv = ["s_add_u32 %[ko], %[ko], 128", "s_add_u32 %[kh], %[kh], 128"]
    sub = "s_sub_u32 %[rem], %[rem], 1"
    cmp2 = "s_cmp_eq_u32 %[rem], 2"

    # the LDS reads a step leaves in flight for the next one (its B blocks
    # and first A row), by the step's stage and whether the next is the
    # last: the next step's waits count them
    ends: dict[tuple, list] = {}

    def step(stage, first, carried, ahead, has_next, next_last, last, tail):
        if first:
            e.lgkm = list(pro)
            i0 = rows_of(last)[0]
            for h in range(KSUB):
                e.read_a(0, h, i0, 0)
        else:
            e.lgkm = list(ends[(stage ^ 1, last)])
        emit_step(e, stage, first, carried, ahead, has_next, next_last, last, tail, p)
        if has_next:
            key = (stage, next_last)
            assert ends.setdefault(key, list(e.lgkm)) == e.lgkm, "steps before one step leave different reads"

    e.op(cmp2)
    e.op("s_cbranch_scc1 5f")
    step(0, True, False, True, True, False, False, adv + [sub, cmp2, "s_cbranch_scc1 6f"])
    e.label("1")
    step(1, False, True, True, True, False, False, adv + [sub, cmp2, "s_cbranch_scc1 8f"])
    step(0, False, True, True, True, False, False, adv + [sub, cmp2, "s_cbranch_scc1 6f", "s_branch 1b"])
    e.label("5")
    step(0, True, False, False, True, True, False, [sub, "s_branch 2f"])        # KT == 2
    e.label("6")
    step(1, False, True, False, True, True, False, [sub, "s_branch 3f"])         # step KT-2 in stage 1
    e.label("8")
    step(0, False, True, False, True, True, False, [sub])                        # step KT-2 in stage 0
    e.label("2")
    step(1, False, False, False, False, False, True, ["s_branch 4f"])            # last step in stage 1
    e.label("3")
    step(0, False, False, False, False, False, True, [])                         # last step in stage 0
    e.label("4")
    return "\n".join(e.lines)


DEFAULT = {
    "a_delay": 1,          # gaps between a position's first MFMA and the reads of the next row's A
    "load_every": 6,       # step j+2's loads, one every this many gaps from the barrier
    "epi_slot": 8,         # epilogue instructions per MFMA gap of the last step
    "epi_delay": 5,        # MFMAs between a row's last MFMA and its epilogue (VGPR results: >= 19 wait states)
}


def as_macro(name: str, text: str) -> str:
    body = [f'    "{ln}\\n"' for ln in text.split("\n")]
    return f"#define {name} \\\n" + " \\\n".join(body) + "\n"


def params_line(p: dict) -> str:
    return ", ".join(f"{k}={v}" for k, v in p.items())


def main(argv: list[str]) -> int:
    here = os.path.dirname(os.path.abspath(__file__))
    out = os.path.join(here, "wide_sched.inc")
    text = generate(DEFAULT)
    with open(out, "w") as f:
        f.write("// Generated by gen_wide_sched.py.  Do not edit.\n")
        f.write("// G16_WIDE_KLOOP: 384 x 256 tiles, one barrier per k step; " + params_line(DEFAULT) + ".\n")
        f.write(as_macro("G16_WIDE_KLOOP", text))
        clob = ", ".join(f'"v{r}"' for r in range(48, 256)) + ", " + ", ".join(f'"a{r}"' for r in range(256))
        f.write("// Registers the block owns: v48..v255 and a0..a255.\n")
        f.write(f"#define G16_WIDE_CLOBBERS {clob}\n")
    print(out, len(text.split("\n")), "lines")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
