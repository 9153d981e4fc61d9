"""Host checks of the generated k loop of the 384 x 256 ring (rung 11).

The schedule (dense_fp16_gemm_nt_amd/csrc/wide_sched.inc) is straight-line
assembly produced by gen_wide_sched.py.  These tests execute its control
flow on the CPU for a range of k-step counts and check the ring protocol
("TIRx GEMM detailed technical notes", V5 "Software Pipeline with
Double-Buffered SMEM"; V9 for the tile shape):

  * the loop ends, after exactly KT steps, for every KT;
  * every k step is loaded exactly once, into stage step % 2, at the LDS
    row group its lane offsets name, and no load reaches beyond K; a load
    into a stage is issued only after the barrier that follows the last read
    of the stage's previous contents;
  * a fragment read sees a stage whose loads were waited for (vmcnt) and
    published by a barrier, with no load into it in flight, and it never
    overwrites a register an MFMA read less than one MFMA earlier;
  * every MFMA consumes the fragments of its own k step, sub-step, block row
    and block column, after an lgkmcnt wait that covers their reads (LDS
    reads complete in issue order), and accumulates into its block's
    registers (AGPRs for rows 0-7, VGPRs for rows 8-11), from 0 in the first
    step;
  * the epilogue converts each accumulator once, after the MFMA that
    finished it and the result latency, stages each row in its buffer,
    reads it back only after its writes completed, stores every row once at
    its own row offset, and never writes a register a store in flight may
    still read;
  * the committed include is what the generator writes.

All four waves run the same instruction stream (wave 0 stands for them);
every barrier is where all waves' earlier waited-for loads become visible.
"""
from __future__ import annotations

import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_fp16_gemm_nt_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_wide_sched", os.path.join(CSRC, "gen_wide_sched.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GEN = _gen()
NBM, NBN = GEN.NBM, GEN.NBN
STAGE, B_OFF = GEN.STAGE, GEN.B_OFF


def _vr(spec: str) -> int:
    return int(re.match(r"v\[(\d+):\d+\]", spec).group(1))


def _block_of_acc(spec: str):
    """(row, column) of the block whose accumulator is `spec`."""
    m = re.match(r"([av])\[(\d+):(\d+)\]$", spec)
    kind, b = m.group(1), int(m.group(2))
    if kind == "a":
        return divmod(b // 4, NBN)
    assert 128 <= b < 256 and b % 4 == 0, spec
    i, j = divmod((b - 128) // 4, NBN)
    return i + 8, j


class Sim:
    def __init__(self, text: str, kt: int):
        self.lines = text.split("\n")
        self.kt = kt
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
        rem, ko, kh, m0, scc, sdo = kt, 0, None, None, 0, None
        vm: list[tuple] = []                       # in issue order: ("load", stage, key, step) | ("store", regs)
        landed = {0: {}, 1: {}}                    # stage -> {(op, q): step} waited for
        visible = {0: {}, 1: {}}                   # stage -> {(op, q): step} published
        reads_since_barrier = {0: 0, 1: 0}
        loaded: dict[int, set] = {}
        lgkm: list[tuple] = []                     # (dest reg or None, content)
        frag: dict[int, tuple] = {}                # vgpr base -> content once the read completed
        last_mfma_read: dict[int, int] = {}        # vgpr base -> index of the last MFMA reading it
        per_block: dict[tuple, int] = {}
        final_ws: dict[tuple, int] = {}            # block -> wait states since its last MFMA
        acc_done: set = set()
        vreg: dict[int, tuple] = {}                # epilogue contents of VGPRs
        staged: dict[int, tuple] = {}              # buffer -> (row, set of j) completed
        stores: list = []
        mfma = 0
        pc = 0
        budget = 10 * (len(self.lines) + 200 * kt)

        def vgprs_of(spec: str) -> range:
            m = re.match(r"v\[(\d+):(\d+)\]$", spec)
            if m:
                return range(int(m.group(1)), int(m.group(2)) + 1)
            return range(int(spec[1:]), int(spec[1:]) + 1)

        def write_vgpr(v: int, what: str) -> None:
            # a write must not clobber data a store in flight still reads
            for op_ in vm:
                if op_[0] == "store":
                    assert v not in op_[1], f"{what} writes v{v}, which a store in flight reads"
            for base in [b for b in frag if b <= v < b + 4]:
                del frag[base]

        def tick(n: int = 1) -> None:
            for b in final_ws:
                final_ws[b] += n

        while pc < len(self.lines):
            budget -= 1
            assert budget > 0, "the loop does not end"
            ln = self.lines[pc]
            if not ln.startswith("v_mfma"):
                nop = re.match(r"s_nop (\d+)$", ln)
                tick(int(nop.group(1)) + 1 if nop else 1)
            if ln.startswith("s_cmp_eq_u32 %[rem], "):
                scc = int(rem == int(ln.split(",")[1]))
            elif ln.startswith("s_cbranch_scc1 "):
                if scc:
                    pc = self.target(ln.split()[1], pc)
                    continue
            elif ln.startswith("s_branch "):
                pc = self.target(ln.split()[1], pc)
                continue
            elif ln.startswith("s_sub_u32 %[rem]"):
                rem -= 1
                scc = None                                   # SCC is the borrow now
            elif ln == "s_add_u32 %[ko], %[ko], 128":
                ko += 128
                scc = None
            elif ln == "s_add_u32 %[kh], %[ko], 128":
                kh = ko + 128
                scc = None
            elif ln == "s_add_u32 %[kh], %[kh], 128":
                kh += 128
                scc = None
            elif ln.startswith("s_add_u32 m0, %[lb"):
                m = re.match(r"s_add_u32 m0, %\[lb([ab])\], (\d+)$", ln)
                m0 = (m.group(1), int(m.group(2)))
                scc = None
            elif ln.startswith("s_mul_i32 %[sdo], %[gstr], "):
                sdo = int(ln.split(",")[2])
            elif ln.startswith("buffer_load_dwordx4"):
                m = re.match(r"buffer_load_dwordx4 %\[([ab])x(\d+)\], %\[rs([ab])\], %\[(k[oh])\] offen"
                             r"( offset:(\d+))? lds$", ln)
                assert m, ln
                op, q, rop, koff, imm = m.group(1), int(m.group(2)), m.group(3), m.group(4), int(m.group(6) or 0)
                assert op == rop and m0 is not None and m0[0] == op, "operand, buffer and LDS base disagree"
                assert imm == 1024 * (q % 4), "the instruction offset is not the one the lane offset leaves out"
                step = (ko if koff == "ko" else kh) // 128
                assert 0 <= step < kt, f"load of step {step} beyond K (KT={kt})"
                dst = m0[1] + imm
                st, off = divmod(dst, STAGE)
                assert st in (0, 1) and off % 1024 == 0
                assert off // 1024 == q, f"{op} load {q} lands at row group {off // 1024}"
                assert st == step % 2, f"step {step} loaded into stage {st}"
                assert reads_since_barrier[st] == 0, "load into a stage read since the last barrier"
                vm.append(("load", st, (op, q), step))
                loaded.setdefault(step, set()).add((op, q))
            elif ln.startswith("s_waitcnt"):
                m = re.search(r"vmcnt\((\d+)\)", ln)
                if m:
                    keep = int(m.group(1))
                    done, vm = (vm[: len(vm) - keep], vm[len(vm) - keep:]) if keep else (vm, [])
                    for op_ in done:
                        if op_[0] == "load":
                            landed[op_[1]][op_[2]] = op_[3]
                m = re.search(r"lgkmcnt\((\d+)\)", ln)
                if m:
                    keep = int(m.group(1))
                    done, lgkm = (lgkm[: len(lgkm) - keep], lgkm[len(lgkm) - keep:]) if keep else (lgkm, [])
                    for reg, content in done:
                        if content[0] == "epi_w":
                            buf, row, j = content[1:]
                            cur = staged.get(buf)
                            if cur is None or cur[0] != row:
                                cur = (row, set())
                            cur[1].add(j)
                            staged[buf] = cur
                        elif content[0] == "epi_r":
                            vreg[reg] = content[1:]
                        else:
                            frag[reg] = content
            elif ln == "s_barrier":
                assert not lgkm, "barrier with LDS reads in flight"
                reads_since_barrier = {0: 0, 1: 0}
                for st in (0, 1):
                    visible[st].update(landed[st])
                    landed[st] = {}
            elif ln.startswith("ds_read_b128") and "%[er" in ln:
                m = re.match(r"ds_read_b128 (v\[\d+:\d+\]), %\[er(\d)\] offset:(\d+)$", ln)
                reg, q, buf = _vr(m.group(1)), int(m.group(2)), int(m.group(3)) // 4096
                for v in range(reg, reg + 4):
                    write_vgpr(v, "a read-back")
                row, js = staged.get(buf, (None, set()))
                assert js == set(range(NBN)), f"read-back of buffer {buf} before all its writes completed"
                lgkm.append((reg, ("epi_r", row, q)))
            elif ln.startswith("ds_read_b128"):
                m = re.match(r"ds_read_b128 (v\[\d+:\d+\]), %\[r([ab])(\d)(\d)\] offset:(\d+)$", ln)
                reg, op, st, h, off = _vr(m.group(1)), m.group(2), int(m.group(3)), int(m.group(4)), int(m.group(5))
                idx = off // 2048
                assert mfma - last_mfma_read.get(reg, -10) >= 1 and last_mfma_read.get(reg, -10) < mfma, \
                    "fragment read over a register the last MFMA still reads"
                assert not any(o[0] == "load" and o[1] == st for o in vm), "read of a stage with a load in flight"
                whos = set(visible[st].values())
                assert len(visible[st]) == GEN.NLOAD and len(whos) == 1, "read of an incompletely published stage"
                for v in range(reg, reg + 4):
                    write_vgpr(v, "a fragment read")
                reads_since_barrier[st] += 1
                lgkm.append((reg, (whos.pop(), h, op, idx)))
            elif ln.startswith("v_mfma_f32_16x16x32_f16"):
                m = re.match(r"v_mfma_f32_16x16x32_f16 ([av]\[\d+:\d+\]), (v\[\d+:\d+\]), (v\[\d+:\d+\]), (\S+)$", ln)
                c, breg, areg, src_c = m.group(1), _vr(m.group(2)), _vr(m.group(3)), m.group(4)
                i, j = _block_of_acc(c)
                step, h = divmod(per_block.get((i, j), 0), 2)
                per_block[(i, j)] = per_block.get((i, j), 0) + 1
                assert (i, j) not in acc_done, "MFMA on an accumulator already written out"
                assert frag.get(areg) == (step, h, "a", i), f"MFMA {mfma} block {(i, j)}: A operand {frag.get(areg)}"
                assert frag.get(breg) == (step, h, "b", j), f"MFMA {mfma} block {(i, j)}: B operand {frag.get(breg)}"
                assert src_c == ("0" if step == 0 and h == 0 else c), "accumulator chain"
                if c.startswith("v"):
                    for v in vgprs_of(c):
                        for op_ in vm:
                            assert op_[0] != "store" or v not in op_[1], "MFMA writes a register a store reads"
                last_mfma_read[areg] = mfma
                last_mfma_read[breg] = mfma
                tick(4)
                if step == kt - 1 and h == 1:
                    final_ws[(i, j)] = 0
                mfma += 1
            elif ln.startswith("v_accvgpr_read_b32"):
                m = re.match(r"v_accvgpr_read_b32 v(\d+), a(\d+)$", ln)
                v, a = int(m.group(1)), int(m.group(2))
                blk = divmod(a // 4, NBN)
                assert blk in final_ws and final_ws[blk] >= 11, f"a{a} read too early"
                write_vgpr(v, "an accumulator read")
                vreg[v] = ("acc", blk, a % 4)
            elif ln.startswith("v_cvt_pk_f16_f32"):
                m = re.match(r"v_cvt_pk_f16_f32 v(\d+), v(\d+), v(\d+)$", ln)
                d, x, y = int(m.group(1)), int(m.group(2)), int(m.group(3))
                cx, cy = vreg.get(x), vreg.get(y)
                if cx is None and 128 <= x < 256:
                    # rows 8-11 convert their VGPR accumulators in place
                    blk = (8 + (x - 128) // 4 // NBN, (x - 128) // 4 % NBN)
                    assert blk in final_ws and final_ws[blk] >= 19, f"v{x} converted too early"
                    cx, cy = ("acc", blk, (x - 128) % 4), ("acc", blk, (y - 128) % 4)
                assert cx and cy and cx[0] == "acc" and cy[0] == "acc" and cx[1] == cy[1] and cy[2] == cx[2] + 1, \
                    "conversion pair"
                write_vgpr(d, "a conversion")
                vreg[d] = ("pk", cx[1], cx[2])
                acc_done.add(cx[1])
            elif ln.startswith("ds_write_b64"):
                m = re.match(r"ds_write_b64 %\[ew(\d)\], v\[(\d+):(\d+)\] offset:(\d+)$", ln)
                j, r0, buf = int(m.group(1)), int(m.group(2)), int(m.group(4)) // 4096
                lo, hi = vreg.get(r0), vreg.get(r0 + 1)
                assert lo and hi and lo[0] == "pk" and hi[0] == "pk" and lo[1] == hi[1], "staging unconverted data"
                assert lo[2] == 0 and hi[2] == 2 and lo[1][1] == j, f"block {lo[1]} staged as column {j}"
                row = lo[1][0]
                cur = staged.get(buf)
                if cur is not None and cur[0] != row:
                    del staged[buf]
                lgkm.append((None, ("epi_w", buf, row, j)))
            elif ln.startswith("buffer_store_dwordx4"):
                m = re.match(r"buffer_store_dwordx4 (v\[\d+:\d+\]), %\[so(\d)\], %\[rsd\], %\[sdo\] offen nt$", ln)
                reg, q = _vr(m.group(1)), int(m.group(2))
                assert vreg.get(reg) == (sdo, q), f"store of {vreg.get(reg)} at row {sdo}, quarter {q}"
                stores.append((sdo, q))
                vm.append(("store", set(range(reg, reg + 4))))
            pc += 1
        assert not lgkm, "LDS operations in flight at the end of the block"
        assert not any(o[0] == "load" for o in vm), "loads in flight at the end"
        assert all(n == 2 * kt for n in per_block.values()) and len(per_block) == NBM * NBN, "MFMAs per block"
        assert acc_done == set(per_block), "accumulators not all written out"
        assert sorted(stores) == [(i, q) for i in range(NBM) for q in range(4)], "rows not all stored once"
        return {"mfma": mfma, "loaded": loaded}


@pytest.mark.parametrize("kt", [2, 3, 4, 5, 6, 7, 8, 9, 16, 33, 64, 128])
def test_wide_ring_protocol(kt):
    res = Sim(GEN.generate(GEN.DEFAULT), kt).run()
    assert res["mfma"] == NBM * NBN * 2 * kt
    assert sorted(res["loaded"]) == list(range(kt))
    assert all(v == set(GEN.LOADS) for v in res["loaded"].values())


@pytest.mark.parametrize("params", [{"load_every": 3}, {"load_every": 4}, {"load_every": 8}, {"epi_slot": 4}])
def test_wide_variants_keep_protocol(params):
    p = dict(GEN.DEFAULT)
    p.update(params)
    for kt in (2, 3, 4, 7):
        Sim(GEN.generate(p), kt).run()


def test_wide_catches_an_early_load():
    """A look-ahead load moved ahead of the barrier that frees its stage."""
    text = GEN.generate(GEN.DEFAULT).split("\n")
    loop = text.index("1:")
    bar = text.index("s_barrier", loop)
    ld = next(i for i in range(bar, len(text)) if "%[kh] offen" in text[i])
    planted = text[:bar - 2] + [text[ld]] + text[bar - 2: ld] + text[ld + 1:]
    with pytest.raises(AssertionError):
        Sim("\n".join(planted), 5).run()


def test_wide_catches_a_short_publish_wait():
    """Publishing the next step before this wave's loads of it landed."""
    text = GEN.generate(GEN.DEFAULT).replace("s_waitcnt vmcnt(0) lgkmcnt(0)", "s_waitcnt vmcnt(4) lgkmcnt(0)")
    with pytest.raises(AssertionError):
        Sim(text, 4).run()


def test_wide_catches_an_early_epilogue():
    p = dict(GEN.DEFAULT)
    p["epi_delay"] = 0
    with pytest.raises(AssertionError):
        Sim(GEN.generate(p), 3).run()


def test_wide_catches_a_wrong_stage_base():
    """A B fragment read from the stage the step does not hold."""
    text = GEN.generate(GEN.DEFAULT)
    k = text.index("%[rb1")
    with pytest.raises(AssertionError):
        Sim(text[:k] + "%[rb0" + text[k + 5:], 3).run()


def test_committed_wide_include_matches_generator():
    with open(os.path.join(CSRC, "wide_sched.inc")) as f:
        inc = f.read()
    assert GEN.as_macro("G16_WIDE_KLOOP", GEN.generate(GEN.DEFAULT)) in inc


from hypothesis import HealthCheck, assume, given, settings, strategies as st


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(load_every=st.integers(2, 8), a_delay=st.integers(0, 2), epi_slot=st.integers(2, 10),
       epi_delay=st.integers(5, 9), kt=st.sampled_from([2, 3, 4, 7]))
def test_wide_random_parameters_keep_protocol(load_every, a_delay, epi_slot, epi_delay, kt):
    """Any schedule the generator accepts (it refuses parameters that do not
    fit a step) keeps the ring protocol and the epilogue's hazards."""
    p = dict(GEN.DEFAULT)
    p.update(load_every=load_every, a_delay=a_delay, epi_slot=epi_slot, epi_delay=epi_delay)
    try:
        text = GEN.generate(p)
    except AssertionError:
        assume(False)
    res = Sim(text, kt).run()
    assert res["mfma"] == NBM * NBN * 2 * kt
