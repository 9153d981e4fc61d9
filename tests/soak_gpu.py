"""Random soak of every entry point on the GPU (test infrastructure, run by
hand: ``python -m tests.soak_gpu --seconds 240 --seed 1``; pytest does not
collect it).

Each case draws a kind (the library's choice, one rung, split-K with a
workspace or with the library's scratch array, operands at element offsets,
padded strided batches), a shape (M, N up to 2600; K below 200, a multiple
of 8 or 64, or anything up to 5000) and seeded uniform[-1, 1] operands made
on the host.  D starts as NaN and must be written everywhere (row padding of
a strided D must stay NaN), and 302 sampled outputs per product, the
corners among them, must meet the oracle's tolerance.  The first failure
stops the run with the case printed; every case is printed before it runs.
"""
import argparse
import sys
import time

import numpy as np
import torch

import dense_fp16_gemm_nt_amd as g
import oracle
from tests.parity import compare

DEV = "cuda:0"


def operand(rng, rows, cols):
    return (rng.random((rows, cols)) * 2 - 1).astype(np.float16)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def check(rng, D, Ah, Bh, K, what):
    M, N = D.shape
    if torch.isnan(D).any().item():
        raise AssertionError(f"output elements left unwritten: {what}")
    rows = np.concatenate([[0, M - 1], rng.integers(0, M, 300)])
    cols = np.concatenate([[N - 1, 0], rng.integers(0, N, 300)])
    want, _ = oracle.gemm_nt_sampled(Ah, Bh, rows, cols)
    got = bits(D[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)])
    ok, worst, nbad, first = compare(got, want, K)
    if not ok:
        raise AssertionError(f"parity: {what}: {nbad} outside the tolerance, first at sample {first}")
    return worst


def pick_k(rng):
    form = rng.integers(0, 4)
    if form == 0:
        return int(rng.integers(1, 200))
    if form == 1:
        return 8 * int(rng.integers(1, 600))
    if form == 2:
        return 64 * int(rng.integers(1, 80))
    return int(rng.integers(1, 5000))


def one_case(rng, n):
    kind = str(rng.choice(["lib", "lib", "rung", "strided", "splitk", "noalloc", "offset"]))
    hi = 300 if rng.random() < 0.3 else 2600
    M, N = (int(x) for x in rng.integers(1, hi, 2))
    K = pick_k(rng)
    what = f"#{n} {kind} M={M} N={N} K={K}"
    Ah, Bh = operand(rng, M, K), operand(rng, N, K)
    if kind == "strided":
        batch = int(rng.integers(1, 4))
        pa, pb, pd = (int(x) for x in rng.integers(0, 20, 3))
        what += f" batch={batch} pads={pa},{pb},{pd}"
        print(what, flush=True)
        A3 = [Ah] + [operand(rng, M, K) for _ in range(batch - 1)]
        B3 = [Bh] + [operand(rng, N, K) for _ in range(batch - 1)]
        Af = torch.zeros((batch, M, K + pa), dtype=torch.float16, device=DEV)
        Bf = torch.zeros((batch, N, K + pb), dtype=torch.float16, device=DEV)
        for b in range(batch):
            Af[b, :, :K] = dev(A3[b])
            Bf[b, :, :K] = dev(B3[b])
        Df = torch.full((batch, M, N + pd), float("nan"), dtype=torch.float16, device=DEV)
        g.gemm_f16_nt_strided_batched(Af[:, :, :K], Bf[:, :, :K], Df[:, :, :N])
        torch.cuda.synchronize()
        if not torch.isnan(Df[:, :, N:]).all().item():
            raise AssertionError(f"row padding of D written: {what}")
        return max(check(rng, Df[b, :, :N], A3[b], B3[b], K, f"{what} entry {b}") for b in range(batch))
    A, B = dev(Ah), dev(Bh)
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    if kind == "rung":
        rung = int(rng.choice([3, 4, 5, 8, 9, 10, 11, 12, 13]))
        what += f" rung={rung}"
        if g.check(rung, M, N, K, A.data_ptr(), B.data_ptr(), D.data_ptr()) != g.OK:
            print(what + " (shape not taken)", flush=True)
            return 0.0
        print(what, flush=True)
        g.gemm_f16_nt_rung(rung, A, B, D)
    elif kind in ("splitk", "noalloc"):
        splits = int(rng.choice([0, int(rng.integers(2, 65 if kind == "splitk" else 17))]))
        what += f" splits={splits}"
        print(what, flush=True)
        if kind == "splitk":
            g.gemm_f16_nt_splitk(A, B, D, splits=splits)
        else:
            try:
                g.gemm_f16_nt_splitk_noalloc(A, B, D, splits=splits)
            except g.GemmError as e:
                if e.status != g.SCRATCH:
                    raise
                return 0.0
    elif kind == "offset":
        oa, ob, od = (int(x) for x in rng.integers(0, 9, 3))
        what += f" offsets={oa},{ob},{od}"
        print(what, flush=True)
        Af = torch.zeros(M * K + oa, dtype=torch.float16, device=DEV)
        Bf = torch.zeros(N * K + ob, dtype=torch.float16, device=DEV)
        Af[oa:] = A.reshape(-1)
        Bf[ob:] = B.reshape(-1)
        Df = torch.full((M * N + od,), float("nan"), dtype=torch.float16, device=DEV)
        D = Df[od:].view(M, N)
        g.gemm_f16_nt(Af[oa:].view(M, K), Bf[ob:].view(N, K), D)
    else:
        print(what, flush=True)
        g.gemm_f16_nt(A, B, D)
    torch.cuda.synchronize()
    return check(rng, D, Ah, Bh, K, what)


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--seconds", type=float, default=240.0)
    p.add_argument("--seed", type=int, default=1)
    a = p.parse_args(argv)
    rng = np.random.default_rng(a.seed)
    t0 = time.time()
    n, worst = 0, 0.0
    while time.time() - t0 < a.seconds:
        worst = max(worst, one_case(rng, n))
        n += 1
    print(f"[soak] seed {a.seed}: {n} cases in {time.time() - t0:.0f} s, all written and within the "
          f"tolerance (worst err/tol {worst:.3f})", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
