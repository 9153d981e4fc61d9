"""The five fixed workloads of the fp16 NT GEMM (shapes, seeds, operand
distributions).  B is always stored N x K row-major; every product
accumulates in fp32 and is rounded to fp16 once.

Seeds are 1..5 in this order.  ``sigma`` of the normal workload is read as
the standard deviation (numpy ``scale`` / torch ``std`` convention); the
clip at +-4 is then 16 sigma and never binds in practice.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    dist: dict = field(hash=False, compare=False)

    @property
    def flop(self) -> int:
        return 2 * self.M * self.N * self.K

    def describe(self) -> str:
        d = self.dist
        if d["kind"] == "uniform":
            ds = f"uniform[{d['lo']},{d['hi']}]"
        else:
            ds = f"normal(0,sigma={d['sigma']}) clip +-{d['clip']}"
        return f"{self.name}: M={self.M} N={self.N} K={self.K} {ds} seed={self.seed}"


U11 = {"kind": "uniform", "lo": -1.0, "hi": 1.0}
U05 = {"kind": "uniform", "lo": -0.5, "hi": 0.5}
N025 = {"kind": "normal", "sigma": 0.25, "clip": 4.0}

WORKLOADS = [
    Workload("single_tile_128x128x64", 128, 128, 64, 1, U11),
    Workload("kloop_grid_256x256x512", 256, 256, 512, 2, U11),
    Workload("square_4096", 4096, 4096, 4096, 3, U11),
    Workload("square_8192", 8192, 8192, 8192, 4, N025),
    Workload("tall_32768x1024x8192", 32768, 1024, 8192, 5, U05),
]
BY_NAME = {w.name: w for w in WORKLOADS}
HEADLINE = BY_NAME["square_4096"]
