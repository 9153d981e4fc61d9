"""Host model of rung 5's producer/consumer handoff ("GEMM III", Step 7
"Four barriers = two producer-consumer rings" and "The subtlest bug:
opposite initial phases"; "TIRx GEMM detailed technical notes", V7).

Rung 5 (csrc/persistent_ws.hpp) joins its 4 producer waves and 8 consumer
waves through two counters per ring stage in LDS, never reset: a producer
adds 1 to ready[s] once its own loads of the step in stage s have landed (a
vmcnt wait that leaves the loads of its later steps in flight), a consumer
adds 1 to free[s] once it has read the step.  The counts each side waits
for come from the library itself (gemm_f16_nt_handoff_plan, evaluating the
same functions the kernel calls).

The model runs each wave's loop as the kernel writes it -- producer
iteration g publishes step g - (depth - 1), then refills step g; consumer
iteration g reads step g -- under many random interleavings, with every
load landing at a random later time (in issue order per wave, as vmcnt
counts them).  It checks:

  * safety: a consumer reads a stage only when every producer's loads of
    that step have landed there, and a producer refills a stage only when
    every consumer has read the step it held;
  * liveness: no interleaving deadlocks (some wave can always move, or a
    load is still to land);

and that planted mistakes in the counts or in the publish wait are caught.
"""
import random

import pytest

import dense_fp16_gemm_nt_amd as g

P, C = 4, 8   # producer and consumer waves of rung 5


class Ring:
    def __init__(self, depth, steps, ready_t, free_t, vm_slack=0):
        self.depth, self.steps = depth, steps
        self.ready_t, self.free_t = ready_t, free_t
        self.vm_slack = vm_slack           # a planted mistake: publish with this many more steps in flight
        self.ready = [0] * depth
        self.free = [0] * depth
        self.holds = [dict() for _ in range(depth)]        # stage -> {producer: step landed}
        self.inflight = [[] for _ in range(P)]             # producer -> [(step, stage)] in issue order
        self.readers = {}                                  # step -> consumers that read it

    # ---- one producer iteration at a time, as the kernel's loop:
    # publish step it - (depth - 1), then refill step it
    def producer(self, p):
        D, S = self.depth, self.steps
        for it in range(S + D - 1):
            j = it - (D - 1)
            if j >= 0:
                younger = min(it - 1, S - 1) - j + self.vm_slack
                while len(self.inflight[p]) > younger:
                    yield "vmwait"
                self.ready[j % D] += 1
                yield "arrive"
            if it < S:
                s = it % D
                while self.free[s] < self.free_t[it]:
                    yield "wait"
                if it >= D:
                    assert self.readers.get(it - D) == set(range(C)), \
                        f"producer {p} refills stage {s} with step {it} before every consumer read step {it - D}"
                self.holds[s].pop(p, None)
                self.inflight[p].append((it, s))
                yield "issue"

    def consumer(self, c):
        D, S = self.depth, self.steps
        for it in range(S):
            s = it % D
            while self.ready[s] < self.ready_t[it]:
                yield "wait"
            for p in range(P):
                assert self.holds[s].get(p) == it, \
                    f"consumer {c} reads step {it} from stage {s} before producer {p}'s loads of it landed"
            self.readers.setdefault(it, set()).add(c)
            yield "read"
            self.free[s] += 1
            yield "arrive"

    def land(self, p):
        step, s = self.inflight[p].pop(0)
        self.holds[s][p] = step


def run(depth, steps, seed, ready_t=None, free_t=None, vm_slack=0):
    rt, ft = g.handoff_plan(depth, P, C, steps)
    ring = Ring(depth, steps, ready_t if ready_t is not None else [int(x) for x in rt],
                free_t if free_t is not None else [int(x) for x in ft], vm_slack)
    rng = random.Random(seed)
    # how eagerly loads land, per interleaving: slow landings let waves run
    # ahead of their loads, fast ones let consumers catch up at once
    land_p = (0.02, 0.2, 0.6)[seed % 3]
    waves = {("p", p): ring.producer(p) for p in range(P)}
    waves.update({("c", c): ring.consumer(c) for c in range(C)})
    last = {w: None for w in waves}
    stalled_rounds = 0
    while waves:
        # a random wave moves, or a random producer's oldest load lands
        landing = [("land", p) for p in range(P) if ring.inflight[p]]
        w = rng.choice(landing) if landing and rng.random() < land_p else rng.choice(list(waves))
        if w[0] == "land":
            ring.land(w[1])
            stalled_rounds = 0
            continue
        try:
            last[w] = next(waves[w])
        except StopIteration:
            del waves[w]
            stalled_rounds = 0
            continue
        if last[w] in ("wait", "vmwait"):
            stalled_rounds += 1
            # every remaining wave waiting and no load left to land: deadlock
            if stalled_rounds > 2000 * (len(waves) + P) and not any(ring.inflight):
                raise AssertionError("deadlock")
        else:
            stalled_rounds = 0
    assert all(not q for q in ring.inflight), "loads in flight at the end"
    assert ring.ready == [P * len(range(s, steps, depth)) for s in range(depth)]
    assert ring.free == [C * len(range(s, steps, depth)) for s in range(depth)]


def test_handoff_targets_match_the_pages_phases():
    """Step k is the (k // depth)-th use of its stage: consumers wait for
    every producer's arrival of that use, producers for every consumer's
    release of the use before (none for the first lap: the producers start
    with all stages free, the consumers blocked)."""
    rt, ft = g.handoff_plan(4, P, C, 12)
    assert list(rt) == [P * (k // 4 + 1) for k in range(12)]
    assert list(ft) == [C * (k // 4) for k in range(12)]
    assert g.lib().gemm_f16_nt_handoff_plan(0, P, C, 4, None, None) == g.INVALID_ARG


@pytest.mark.parametrize("depth,steps", [(4, 1), (4, 3), (4, 4), (4, 9), (4, 37), (2, 11), (3, 10)])
@pytest.mark.parametrize("seed", range(12))
def test_handoff_is_safe_and_live(depth, steps, seed):
    run(depth, steps, seed)


def _caught(depth, steps, seeds, **kw):
    for seed in seeds:
        try:
            run(depth, steps, seed, **kw)
        except AssertionError:
            return True
    return False


def test_planted_short_ready_count_is_caught():
    rt, ft = g.handoff_plan(4, P, C, 16)
    bad = [int(x) - 1 for x in rt]          # one producer arrival short
    assert _caught(4, 16, range(40), ready_t=bad)


def test_planted_short_free_count_is_caught():
    rt, ft = g.handoff_plan(4, P, C, 16)
    bad = [max(0, int(x) - 1) for x in ft]  # one consumer release short
    assert _caught(4, 16, range(40), free_t=bad)


def test_planted_early_publish_is_caught():
    # publishing a step while one more of its loads may still be in flight
    assert _caught(4, 16, range(40), vm_slack=1)


def test_planted_same_phase_start_deadlocks():
    # the pages' "subtlest bug": producers that also start blocked (waiting
    # for a release of the first lap, which never comes) deadlock
    rt, ft = g.handoff_plan(4, P, C, 8)
    bad = [int(x) + C for x in ft]
    with pytest.raises(AssertionError, match="deadlock"):
        run(4, 8, 0, free_t=bad)
