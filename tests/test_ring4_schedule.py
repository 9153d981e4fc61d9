"""Host checks of the generated k-loop schedule of the four-wave ring kernel.

The schedule (dense_fp16_gemm_nt_amd/csrc/ring4_sched.inc) is straight-line
assembly produced by gen_ring4_sched.py.  These tests execute its control
flow on the CPU for a range of k-step counts and check the ring protocol
("TIRx GEMM detailed technical notes", V5 "Software Pipeline with
Double-Buffered SMEM": a stage is refilled only after every consumer has
released it, and read only after its load has landed and been published):

  * every k step is loaded exactly once, into stage step % 2, and no load
    reaches beyond K;
  * a load into a stage is issued only after the barrier that follows the
    last read of the stage's previous contents, with no read of that stage
    since (the LDS write-after-read race across waves);
  * a fragment read sees a stage whose loads were waited for (vmcnt) and
    then published by a barrier, with no load into that stage in flight;
  * every MFMA consumes the fragments of its own k step, sub-step and
    block, after an lgkmcnt wait that covers their reads (LDS reads
    complete in issue order), and accumulates into the block's registers,
    starting from 0 in the first step;
  * the epilogue reads each accumulator once, after the MFMA that finished
    it and the MFMA-to-read latency, converts consecutive pairs, stages each
    16-row group in its own LDS buffer, reads it back only after the group's
    writes completed, and stores every row group once at its own offset;
  * all waves cross the same number of barriers, and the committed include
    is what the generator writes.

Both generated forms are checked: the third (generate3, rung 8) and the
fourth (generate4, rung 10, the library's choice), including the fourth
form's partial first step and its ring carried across tiles.

All four waves run the same instruction stream, so one stream stands for
all of them; the checks treat every barrier as the point where all waves'
earlier waited-for loads become visible.
"""
from __future__ import annotations

import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_fp16_gemm_nt_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_ring4_sched", os.path.join(CSRC, "gen_ring4_sched.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GEN = _gen()
NB = GEN.NB


def _regs(spec: str) -> int:
    """First register number of 'v[a:b]'."""
    return int(re.match(r"v\[(\d+):\d+\]", spec).group(1))


class Sim:
    """Executes one wave's stream of the generated block for KT k steps,
    for `tiles` consecutive tiles of one workgroup (the fourth form carries
    its ring from tile to tile; the others run one tile)."""

    def __init__(self, text: str, kt: int, tiles: int = 1, carry: bool = True):
        self.lines = text.split("\n")
        self.kt = kt
        self.tiles = tiles
        self.carry = carry      # the fourth form: each last step loads the next tile's step 0
        self.labels: dict[str, list[int]] = {}
        for i, ln in enumerate(self.lines):
            m = re.match(r"^(\d+):$", ln)
            if m:
                self.labels.setdefault(m.group(1), []).append(i)

    def target(self, ref: str, pc: int) -> int:
        n, d = ref[:-1], ref[-1]
        c = self.labels[n]
        return min(x for x in c if x > pc) if d == "f" else max(x for x in c if x < pc)

    def run(self) -> dict:
        kt = self.kt
        # across tiles: the vector-memory queue (loads and stores, issue
        # order), what each physical stage holds, barriers crossed
        vm: list[tuple] = []           # ("load", (tile, step), stage, n) | ("store",)
        landed: dict[int, dict] = {0: {}, 1: {}}    # stage -> {n: (tile, step)} waited for
        visible: dict[int, dict] = {0: {}, 1: {}}   # stage -> {n: (tile, step)} published
        reads_since_barrier = {0: 0, 1: 0}
        epoch = 0
        mfma = 0
        loaded_steps: dict[int, set] = {}
        par = 0                        # physical stage of the tile's logical stage 0
        first = 1
        for tile in range(self.tiles):
            has_next = tile + 1 < self.tiles
            hasn = int(has_next and self.carry)
            par_next = par ^ (kt & 1) if hasn else par
            rem, ko, kh, m0, scc = kt, 0, None, None, 0
            lgkm: list[tuple] = []         # outstanding reads (reg, content)
            frag: dict[int, tuple] = {}    # vgpr base -> (tile, step, kk, op, idx) once its read completed
            acc_started = set()
            per_block: dict[int, int] = {}  # MFMAs issued per accumulator block
            pc = 0
            final_at: dict[int, int] = {}          # block -> line of its last MFMA
            since_final: dict[int, int] = {}       # block -> wait states since
            acc_read: set = set()                  # accumulator registers read
            vreg: dict[int, tuple] = {}            # epilogue VGPR contents
            sdo = None
            head: dict = {}                        # VGPR or "ht" -> (op, q) of a step-0 lane offset
            staged: dict[int, tuple] = {}          # buf -> (group, set of j) completed
            stores: list = []

            def clobber(v: int) -> None:
                """A VALU write of v: a fragment held there is gone."""
                for base in [b for b in frag if b <= v < b + 4]:
                    del frag[base]

            while pc < len(self.lines):
                ln = self.lines[pc]
                if not ln.startswith("v_mfma"):
                    nop = re.match(r"s_nop (\d+)$", ln)
                    for b_ in since_final:
                        since_final[b_] += int(nop.group(1)) + 1 if nop else 1
                if ln.startswith("s_cmp_eq_u32 %[rem], "):
                    scc = int(rem == int(ln.split(",")[1]))
                elif ln == "s_cmp_eq_u32 %[first], 0":
                    scc = int(first == 0)
                elif ln == "s_cmp_eq_u32 %[hasn], 0":
                    scc = int(hasn == 0)
                elif ln.startswith("s_cbranch_scc1 "):
                    if scc:
                        pc = self.target(ln.split()[1], pc)
                        continue
                elif ln.startswith("s_branch "):
                    pc = self.target(ln.split()[1], pc)
                    continue
                elif ln.startswith("s_sub_u32 %[rem]"):
                    rem -= 1
                elif ln.startswith("s_add_u32 %[ko]"):
                    ko += 128
                elif ln == "s_add_u32 %[kh], %[ko], 128":
                    kh = ko + 128
                elif ln.startswith("s_add_u32 %[kh], %[kh], "):
                    kh += 128
                elif ln.startswith("s_add_u32 m0, %[lb], "):
                    m0 = int(ln.split(",")[2])
                elif ln.startswith("s_add_u32 m0, %[lb"):
                    m = re.match(r"s_add_u32 m0, %\[lb([01])\], (\d+)$", ln)
                    assert m, ln
                    m0 = (int(m.group(1)) ^ par) * 65536 + int(m.group(2))
                elif ln.startswith("v_or_b32"):
                    # a step-0 lane offset: row group q's reduced offsets
                    # with the head mask of q's parity
                    m = re.match(r"v_or_b32 (v\d+|%\[ht\]), %\[([ab])x(\d)\], %\[hm(\d)\]$", ln)
                    assert m, ln
                    dst, op, q, hp = m.group(1), m.group(2), int(m.group(3)), int(m.group(4))
                    assert hp == q % 2, f"row group {q} with the head mask of parity {hp}"
                    if dst.startswith("v"):
                        clobber(int(dst[1:]))
                        head[int(dst[1:])] = (op, q)
                    else:
                        head["ht"] = (op, q)
                elif ln.startswith("buffer_load_dwordx4"):
                    m = re.match(r"buffer_load_dwordx4 (?:%\[([ab])([ox])(\d)\]|v(\d+)|(%\[ht\])), %\[rs([ab])(n?)\], "
                                 r"(?:%\[(k[oh])\]|(0)) offen( offset:(\d+))? lds$", ln)
                    assert m, ln
                    rop, nxt, koff, imm = m.group(6), m.group(7) == "n", m.group(8), int(m.group(11) or 0)
                    if m.group(4) is not None or m.group(5) is not None:
                        key = int(m.group(4)) if m.group(4) is not None else "ht"
                        assert key in head, f"load from {key}, which holds no step-0 offset"
                        op, q = head[key]
                        kind = "x"
                    else:
                        op, kind, q = m.group(1), m.group(2), int(m.group(3))
                    assert op == rop, "lane offsets of one operand with the other's buffer"
                    if nxt:
                        # the next tile's step 0, from its own buffers, at k offset 0
                        assert kind == "x" and koff is None and m.group(5) is not None, "next-tile load form"
                        step, owner = 0, tile + 1
                    else:
                        assert koff is not None and m.group(5) is None
                        if m.group(4) is not None:
                            assert koff == "ko" and ko == 0, "a step-0 offset used after step 0"
                        # the immediate offset moves the global address and the
                        # LDS destination alike; the 'x' lane offsets of row
                        # group q are 1024 * (q mod 4) bytes short of the row
                        # group's
                        goff = (ko if koff == "ko" else kh) + imm - (1024 * (q % 4) if kind == "x" else 0)
                        assert goff % 128 == 0, f"global offset {goff} is not a k step"
                        step, owner = goff // 128, tile
                        assert 0 <= step < kt, f"load of step {step} beyond K (KT={kt})"
                    dst = m0 + imm
                    assert dst % 1024 == 0 and 0 <= dst < 2 * 65536, f"LDS destination {dst}"
                    st = dst // 65536
                    off = dst % 65536
                    n = 2 * ((off % 32768) // 1024) + (1 if off >= 32768 else 0)
                    assert (op == "a") == (n % 2 == 0), "A/B operand does not match the LDS region"
                    assert (off % 32768) // 1024 == q, f"row group {q} lands at row group {(off % 32768) // 1024}"
                    want = (par_next if nxt else par) ^ (step % 2)
                    assert st == want, f"step {step} of tile {owner} loaded into stage {st}, not {want}"
                    assert reads_since_barrier[st] == 0, "load into a stage read since the last barrier"
                    assert not nxt or hasn, "next-tile loads in a last step without a next tile"
                    vm.append(("load", (owner, step), st, n))
                    if owner == tile:
                        loaded_steps.setdefault(step, set()).add(n)
                elif ln.startswith("s_waitcnt"):
                    m = re.search(r"vmcnt\((\d+)\)", ln)
                    if m:
                        keep = int(m.group(1))
                        done, vm = (vm[: len(vm) - keep], vm[len(vm) - keep:]) if keep else (vm, [])
                        for op_ in done:
                            if op_[0] == "load":
                                landed[op_[2]][op_[3]] = op_[1]
                    m = re.search(r"lgkmcnt\((\d+)\)", ln)
                    if m:
                        keep = int(m.group(1))
                        done, lgkm = (lgkm[: len(lgkm) - keep], lgkm[len(lgkm) - keep:]) if keep else (lgkm, [])
                        for reg, content in done:
                            if content[0] == "epi_w":
                                buf, grp, j = content[1:]
                                st_ = staged.setdefault(buf, (grp, set()))
                                if st_[0] != grp:
                                    st_ = (grp, set())
                                st_[1].add(j)
                                staged[buf] = st_
                            elif content[0] == "epi_r":
                                vreg[reg] = content[1:]
                            else:
                                frag[reg] = content
                elif ln == "s_barrier":
                    assert not lgkm, "barrier with LDS reads in flight"
                    epoch += 1
                    reads_since_barrier = {0: 0, 1: 0}
                    for st in (0, 1):
                        for n, who in landed[st].items():
                            visible[st][n] = who
                        landed[st] = {}
                elif ln.startswith("ds_read_b128 ") and "%[er" in ln:
                    m = re.match(r"ds_read_b128 (v\[\d+:\d+\]), %\[er(\d)\] offset:(\d+)$", ln)
                    reg, q, buf = _regs(m.group(1)), int(m.group(2)), int(m.group(3)) // 4096
                    for v_ in range(reg, reg + 4):
                        clobber(v_)
                    grp, js = staged.get(buf, (None, set()))
                    assert js == set(range(NB)), f"read-back of buffer {buf} before all its writes completed"
                    lgkm.append((reg, ("epi_r", grp, q)))
                elif ln.startswith("ds_write_b64"):
                    m = re.match(r"ds_write_b64 %\[ew(\d)\], v\[(\d+):(\d+)\] offset:(\d+)$", ln)
                    j, r0, buf = int(m.group(1)), int(m.group(2)), int(m.group(4)) // 4096
                    lo, hi = vreg.get(r0), vreg.get(r0 + 1)
                    assert lo and hi and lo[0] == "pk" and hi[0] == "pk", "staging write of unconverted data"
                    b0 = lo[1] // 4
                    assert lo[1] == 4 * b0 and hi[1] == 4 * b0 + 2, "staging write of the wrong accumulator pairs"
                    grp, jj = b0 // NB, b0 % NB
                    assert jj == j and buf == grp % 2, f"block {b0} staged at column {j}, buffer {buf}"
                    if buf in staged and staged[buf][0] != grp:
                        del staged[buf]
                    lgkm.append((-1, ("epi_w", buf, grp, j)))
                elif ln.startswith("v_accvgpr_read_b32"):
                    m = re.match(r"v_accvgpr_read_b32 v(\d+), a(\d+)$", ln)
                    v, a = int(m.group(1)), int(m.group(2))
                    clobber(v)
                    blk = a // 4
                    assert blk in final_at and since_final[blk] >= 11, f"accumulator a{a} read too early"
                    assert a not in acc_read, f"a{a} read twice"
                    acc_read.add(a)
                    vreg[v] = ("acc", a)
                elif ln.startswith("v_cvt_pk_f16_f32"):
                    m = re.match(r"v_cvt_pk_f16_f32 v(\d+), v(\d+), v(\d+)$", ln)
                    d_, x, y = int(m.group(1)), int(m.group(2)), int(m.group(3))
                    clobber(d_)
                    cx, cy = vreg.get(x), vreg.get(y)
                    assert cx and cy and cx[0] == "acc" and cy[0] == "acc" and cy[1] == cx[1] + 1, "conversion pair"
                    vreg[d_] = ("pk", cx[1])
                elif ln == "s_mov_b32 %[sdo], 0":
                    sdo = 0
                elif ln == "s_add_u32 %[sdo], %[sdo], %[gstr]":
                    sdo += 1
                elif ln.startswith("buffer_store_dwordx4"):
                    m = re.match(r"buffer_store_dwordx4 (v\[\d+:\d+\]), %\[so(\d)\], %\[rsd\], %\[sdo\] offen( nt)?$", ln)
                    reg, q = _regs(m.group(1)), int(m.group(2))
                    assert vreg.get(reg) == (sdo, q), f"store of {vreg.get(reg)} at group {sdo}, rows {q}"
                    stores.append((sdo, q))
                    vm.append(("store",))
                elif ln.startswith("ds_read_b128"):
                    m = re.match(r"ds_read_b128 (v\[\d+:\d+\]), %\[r([ab])(\d)(\d)\] offset:(\d+)", ln)
                    reg, op, ls, kk, off = _regs(m.group(1)), m.group(2), int(m.group(3)), int(m.group(4)), int(m.group(5))
                    st = ls ^ par
                    idx = off // 2048
                    assert not any(o[0] == "load" and o[2] == st for o in vm), \
                        "read of a stage with a load in flight"
                    whos = set(visible[st].values())
                    assert len(visible[st]) == 16 and len(whos) == 1, "read of an incompletely published stage"
                    who = whos.pop()
                    assert who[0] == tile, f"tile {tile} reads tile {who}'s data"
                    reads_since_barrier[st] += 1
                    frag.pop(reg, None)
                    lgkm.append((reg, (who[1], kk, op, idx)))
                elif ln.startswith("v_mfma_f32_16x16x32_f16"):
                    m = re.match(r"v_mfma_f32_16x16x32_f16 (a\[(\d+):\d+\]), (v\[\d+:\d+\]), (v\[\d+:\d+\]), (\S+)$", ln)
                    acc, blk, breg, areg, src_c = m.group(1), int(m.group(2)) // 4, _regs(m.group(3)), _regs(m.group(4)), m.group(5)
                    # each block accumulates k steps in order, sub-step 0 before
                    # sub-step 1 (whatever the order across blocks)
                    step, kk = divmod(per_block.get(blk, 0), 2)
                    per_block[blk] = per_block.get(blk, 0) + 1
                    assert not any(4 * blk + r in acc_read for r in range(4)), "MFMA on an accumulator already written out"
                    if step == kt - 1 and kk == 1:
                        final_at[blk] = pc
                        since_final[blk] = 0
                    for b_ in since_final:
                        since_final[b_] += 4       # an MFMA issue is at least 4 wait states
                    i, j = blk // NB, blk % NB
                    assert frag.get(areg) == (step, kk, "a", i), f"MFMA {mfma}: A operand {frag.get(areg)}"
                    assert frag.get(breg) == (step, kk, "b", j), f"MFMA {mfma}: B operand {frag.get(breg)}"
                    if step == 0 and kk == 0:
                        assert src_c == "0" and blk not in acc_started
                        acc_started.add(blk)
                    else:
                        assert src_c == acc and blk in acc_started
                    mfma += 1
                pc += 1
            assert not lgkm, "LDS operations in flight at the end of the block"
            assert not any(o[0] == "load" and o[1][0] == tile for o in vm), "this tile's loads in flight at its end"
            assert all(n == 2 * kt for n in per_block.values()) and len(per_block) == NB * NB, "MFMAs per block"
            assert acc_read == set(range(4 * NB * NB)), "accumulators not all written out"
            assert sorted(stores) == [(i, q) for i in range(NB) for q in range(4)], "output rows not all stored once"
            # between tiles: the workgroup barrier after the block
            if has_next:
                epoch += 1
                reads_since_barrier = {0: 0, 1: 0}
                for st in (0, 1):
                    for n, who in landed[st].items():
                        visible[st][n] = who
                    landed[st] = {}
                par = par_next
                first = 0 if hasn else 1
        if self.tiles == 1:
            assert not any(o[0] == "load" for o in vm), "loads in flight at the end"
        return {"mfma": mfma, "epoch": epoch, "acc": acc_started, "loaded": loaded_steps}


@pytest.mark.parametrize("kt", [2, 3, 4, 5, 6, 7, 8, 9, 16, 33, 64])
def test_third_form_ring_protocol(kt):
    res = Sim(GEN.generate3(GEN.DEFAULT3), kt).run()
    assert res["mfma"] == 2 * NB * NB * kt
    assert res["epoch"] == 2 * (kt - 1)              # prologue, release and publish per step, none in the last
    assert len(res["acc"]) == NB * NB
    assert sorted(res["loaded"]) == list(range(kt))
    assert all(v == set(range(16)) for v in res["loaded"].values())


@pytest.mark.parametrize("params", [
    {"rel": 20, "load_every": 6, "pub": 80}, {"rel": 30, "load_every": 8, "pub": 84},
    {"rel": 24, "load_every": 4, "pub": 96, "f0_lat": 8}, {"f1_every": 2, "rel": 34, "load_every": 7},
    {"rel": 24, "load_every": 9, "pub": 92, "f0_lat": 6},    # late loads run past the next release
])
def test_third_form_variants_keep_protocol(params):
    p = dict(GEN.DEFAULT3)
    p.update(params)
    for kt in (2, 3, 4, 7):
        Sim(GEN.generate3(p), kt).run()


def test_third_form_one_instruction_per_gap():
    """In the steady-state steps at most one instruction sits between two
    MFMAs, except after the last MFMA of a step (the branches)."""
    lines = GEN.generate3(GEN.DEFAULT3).split("\n")
    body = lines[lines.index("1:") + 1: lines.index("5:")]
    runs, n = [], 0
    for ln in body:
        if ln.startswith("v_mfma"):
            runs.append(n)
            n = 0
        elif not ln.endswith(":"):
            n += 1
    assert runs[0] == 0 and len(runs) == 2 * 2 * NB * NB
    inner = [r for k, r in enumerate(runs) if k % (2 * NB * NB) != 0]   # gap 127 of a step precedes MFMA 0
    assert max(inner) <= 1


@pytest.mark.parametrize("kt", [2, 3, 4, 5, 6, 7, 8, 9, 16, 33, 64])
def test_fourth_form_ring_protocol(kt):
    res = Sim(GEN.generate4(GEN.DEFAULT4), kt).run()
    assert res["mfma"] == 2 * NB * NB * kt
    assert res["epoch"] == 2 * (kt - 1)              # prologue, release and publish per step, none in the last
    assert len(res["acc"]) == NB * NB
    assert sorted(res["loaded"]) == list(range(kt))
    assert all(v == set(range(16)) for v in res["loaded"].values())


@pytest.mark.parametrize("params", [
    {"rel": 16, "pub": 72}, {"rel": 10, "load_every": 7, "pub": 56}, {"read_limit": 100, "a_delay": 2},
    {"rel": 12, "load_every": 9, "pub": 64, "f0_lat": 6},   # late loads run past the next release
])
def test_fourth_form_variants_keep_protocol(params):
    p = dict(GEN.DEFAULT4)
    p.update(params)
    for kt in (2, 3, 4, 7):
        Sim(GEN.generate4(p), kt).run()


def test_fourth_form_pairs_sub_steps():
    """Each block's sub-step-1 MFMA follows its sub-step-0 MFMA directly."""
    lines = [ln for ln in GEN.generate4(GEN.DEFAULT4).split("\n") if ln.startswith("v_mfma")]
    accs = [ln.split()[1].rstrip(",") for ln in lines]
    assert all(accs[2 * k] == accs[2 * k + 1] for k in range(len(accs) // 2))


def test_simulator_catches_epilogue_temporaries_in_live_fragments(monkeypatch):
    """The last step's epilogue temporaries in the B set its MFMAs still
    read must be caught."""
    monkeypatch.setattr(GEN, "epi_set4", lambda par: 128 + 64 * par)
    with pytest.raises(AssertionError):
        Sim(GEN.generate4(GEN.DEFAULT4), 3).run()


def test_simulator_catches_an_uncompensated_offset():
    """An instruction offset on lane offsets that were not reduced by it
    reads the wrong k step."""
    text = GEN.generate3(GEN.DEFAULT3).replace("%[ax1]", "%[ao1]", 1)
    with pytest.raises(AssertionError):
        Sim(text, 4).run()


def test_simulator_catches_a_head_mask_of_the_wrong_parity():
    """Row group 1 with the even groups' head mask zeroes the wrong chunks
    when K is not a multiple of 64."""
    text = GEN.generate4(GEN.DEFAULT4).replace("%[ax1], %[hm1]", "%[ax1], %[hm0]", 1)
    with pytest.raises(AssertionError):
        Sim(text, 3).run()


def test_simulator_catches_a_swapped_head_offset():
    """Step 0's load of row group 0 from row group 1's head offset lands
    the wrong rows."""
    text = GEN.generate4(GEN.DEFAULT4).replace("buffer_load_dwordx4 v64,", "buffer_load_dwordx4 v65,", 1)
    with pytest.raises(AssertionError):
        Sim(text, 3).run()


def test_head_step_loads_are_step_zeros_only():
    """The fourth form reads every step-0 row group through a masked
    offset: its own prologue's (first tile) into v64..v79, and the next
    tile's from the last step (both copies) through %[ht]; no later step
    does."""
    lines = GEN.generate4(GEN.DEFAULT4).split("\n")
    own = [ln for ln in lines if re.match(r"v_or_b32 v\d+,", ln)]
    nxt = [ln for ln in lines if ln.startswith("v_or_b32 %[ht]")]
    assert len(own) == GEN.NLOAD and len(nxt) == 2 * GEN.NLOAD
    head_loads = [n for n, ln in enumerate(lines) if re.match(r"buffer_load_dwordx4 v\d+,", ln)]
    next_loads = [n for n, ln in enumerate(lines) if ln.startswith("buffer_load_dwordx4 %[ht]")]
    assert len(head_loads) == GEN.NLOAD and len(next_loads) == 2 * GEN.NLOAD
    first_other = next(n for n, ln in enumerate(lines) if ln.startswith("buffer_load_dwordx4 %["))
    assert max(head_loads) < first_other < min(next_loads)
    last_steps = [lines.index("2:"), lines.index("3:")]
    assert all(n > min(last_steps) for n in next_loads)


@pytest.mark.parametrize("kt", [2, 3, 4, 5, 8, 9])
@pytest.mark.parametrize("tiles", [2, 3, 4])
def test_fourth_form_carries_the_ring_across_tiles(kt, tiles):
    """Consecutive tiles of a workgroup: each later tile's step 0 is loaded
    during the last step of the tile before, into the stage that step does
    not read (the logical stages swap when KT is odd), and waited for with
    that tile's late stores still in flight; every tile reads only its own
    data."""
    for carry in (True, False):
        res = Sim(GEN.generate4(GEN.DEFAULT4), kt, tiles, carry).run()
        assert res["mfma"] == 2 * NB * NB * kt * tiles
        assert sorted(res["loaded"]) == list(range(kt))


def test_simulator_catches_a_short_next_tile_wait():
    """Waiting for fewer operations than were issued after the next tile's
    step-0 loads reads a stage before those loads have landed."""
    text = GEN.generate4(GEN.DEFAULT4)
    m = re.search(r"12:\ns_waitcnt vmcnt\((\d+)\)", text)
    planted = text.replace(m.group(0), f"12:\ns_waitcnt vmcnt({int(m.group(1)) + 1})", 1)
    with pytest.raises(AssertionError):
        Sim(planted, 3, 2).run()


def test_simulator_catches_next_tile_loads_into_the_busy_stage():
    """The next tile's step 0 into the stage the last step still reads."""
    text = GEN.generate4(GEN.DEFAULT4)
    last = text.index("\n2:\n")
    body = text[last:].replace("s_add_u32 m0, %[lb0], 0\n", "s_add_u32 m0, %[lb1], 0\n", 1)
    with pytest.raises(AssertionError):
        Sim(text[:last] + body, 4, 2).run()


def _chunk(w: int, lane: int, q: int) -> int:
    """16-byte chunk of load q of wave w's lane: 8 rows of 8 chunks per
    load, row r's chunks XOR-swizzled with (r / 2) mod 8."""
    r = (w * 8 + q) * 8 + lane // 8
    return (lane % 8) ^ ((r // 2) % 8)


def test_head_mask_depends_on_row_group_parity_only():
    """A lane's chunk in load q depends on q only through its parity, so
    two head masks serve all 8 row groups; for every partial-step length
    the masked chunks are exactly those before the row's first element."""
    for w in range(4):
        for lane in range(64):
            for q in range(8):
                assert _chunk(w, lane, q) == _chunk(0, lane, q % 2)
    for hk in range(0, 64, 8):
        for lane in range(64):
            for q in range(2):
                c = _chunk(0, lane, q)
                masked = 8 * c < hk
                assert masked == all(8 * c + e < hk for e in range(8))
        # every row of a load has hk / 8 masked chunks
        for q in range(2):
            for row in range(8):
                assert sum(8 * _chunk(0, 8 * row + cl, q) < hk for cl in range(8)) == hk // 8


def test_simulator_catches_a_planted_race():
    """Moving one look-ahead load ahead of the release barrier that frees
    its stage must be caught (the third form)."""
    text = GEN.generate3(GEN.DEFAULT3).split("\n")
    loop = text.index("1:")
    bar = text.index("s_barrier", loop)                          # a release barrier
    ld = next(i for i in range(bar, len(text)) if "%[kh] offen" in text[i])
    planted = text[:bar - 2] + [text[ld]] + text[bar - 2: ld] + text[ld + 1:]
    with pytest.raises(AssertionError):
        Sim("\n".join(planted), 5).run()


def test_simulator_catches_an_immediate_offset():
    """A direct-to-LDS load with an instruction offset that its lane offset
    does not compensate lands off its row group in LDS (the offset applies
    to both addresses)."""
    text = GEN.generate3(GEN.DEFAULT3).replace("%[kh] offen lds", "%[kh] offen offset:128 lds", 1)
    with pytest.raises(AssertionError):
        Sim(text, 4).run()


def test_simulator_catches_an_early_epilogue():
    """Queuing each row group as soon as its MFMAs are issued (no delay)
    reads accumulators before the MFMA latency has passed."""
    p = dict(GEN.DEFAULT3)
    p["epi_delay"] = -1
    with pytest.raises(AssertionError):
        Sim(GEN.generate3(p), 3).run()


def test_simulator_catches_a_short_wait():
    """Weakening a fragment wait of the third form so that the reads an MFMA
    needs may still be in flight must be caught."""
    text = GEN.generate3(GEN.DEFAULT3).split("\n")
    loop = text.index("1:")
    k = next(i for i in range(loop, len(text)) if text[i] == "s_waitcnt lgkmcnt(0)"
             and "s_barrier" not in text[i + 1: i + 3])
    text[k] = "s_waitcnt lgkmcnt(15)"
    with pytest.raises(AssertionError):
        Sim("\n".join(text), 4).run()


def test_committed_include_matches_generator():
    with open(os.path.join(CSRC, "ring4_sched.inc")) as f:
        inc = f.read()
    assert GEN.as_macro("G16_RING4_KLOOP3", GEN.generate3(GEN.DEFAULT3)) in inc
    assert GEN.as_macro("G16_RING4_KLOOP4", GEN.generate4(GEN.DEFAULT4)) in inc


# ----------------------------------------------- random schedule parameters

from hypothesis import HealthCheck, assume, given, settings, strategies as st


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(rel=st.integers(8, 20), pub=st.integers(48, 80), load_every=st.integers(5, 9), a_delay=st.integers(0, 3),
       epi_slot=st.integers(4, 8), kt=st.sampled_from([2, 3, 5]), tiles=st.sampled_from([1, 2]))
def test_fourth_form_random_parameters_keep_protocol(rel, pub, load_every, a_delay, epi_slot, kt, tiles):
    """Any schedule the generator accepts (it refuses parameters that do not
    fit a step) keeps the ring protocol, across consecutive tiles too."""
    p = dict(GEN.DEFAULT4)
    p.update(rel=rel, pub=pub, load_every=load_every, a_delay=a_delay, epi_slot=epi_slot)
    try:
        text = GEN.generate4(p)
    except AssertionError:
        assume(False)
    Sim(text, kt, tiles, tiles > 1).run()
