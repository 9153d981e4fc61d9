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


@dataclass(frozen=True)
class ExtraWorkload:
    """A product beyond the five fixed workloads, for the general-shape and
    attention-score entry points: `batch` independent products D[b] =
    A[b] @ B[b]^T of M x N x K.

    kind  "gemm"       one contiguous product through gemm_f16_nt
          "splitk"     one contiguous product through gemm_f16_nt_splitk with
                       the library's choice of split (and its workspace)
          "strided"    contiguous batch entries through the strided-batched
                       entry point
          "heads_rows" attention scores with the heads interleaved in the
                       rows of Q and K ((S, H, d) storage read as H products
                       of S x S x d: leading dimension H*d, batch stride d)
    Operands are drawn as one (batch*M) x K and one (batch*N) x K matrix
    from the input generator and split into batch entries in order."""
    name: str
    kind: str
    batch: int
    M: int
    N: int
    K: int
    seed: int
    dist: dict = field(hash=False, compare=False)

    @property
    def flop(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        """Compulsory HBM bytes: every operand element read once and every
        output element written once, 2 bytes each."""
        return 2 * self.batch * (self.M * self.K + self.N * self.K + self.M * self.N)

    def describe(self) -> str:
        d = self.dist
        ds = f"uniform[{d['lo']},{d['hi']}]" if d["kind"] == "uniform" else f"normal(0,{d['sigma']})"
        return f"{self.name}: {self.kind} batch={self.batch} M={self.M} N={self.N} K={self.K} {ds} seed={self.seed}"


EXTRA_WORKLOADS = [
    # ragged M, N and K (K % 64 != 0): the four-wave ring, partial first k step
    ExtraWorkload("ragged_4000", "gemm", 1, 4000, 4000, 4000, 11, U11),
    # ragged M and N, whole 64-wide k steps: the four-wave ring with clamped edge tiles
    ExtraWorkload("ragged_mn_4000x4000x4096", "gemm", 1, 4000, 4000, 4096, 12, U11),
    # K % 8 != 0: operand rows are not 16-byte aligned, so the 8-wave ring
    # stages its loads through registers
    ExtraWorkload("unaligned_k_4096x4096x4095", "gemm", 1, 4096, 4096, 4095, 13, U11),
    # N % 8 != 0: rows of D are not 16-byte aligned, so the four-wave ring
    # stores its 16-byte chunks of D unaligned
    ExtraWorkload("ragged_n_4096x4092x4096", "gemm", 1, 4096, 4092, 4096, 20, U11),
    # M = 128: 256 x 256 tiles would be half padding and fill half the device,
    # so the library takes 128 x 128 tiles
    ExtraWorkload("thin_m_128x32768x4096", "gemm", 1, 128, 32768, 4096, 21, U11),
    # one side of 16 rows (a small batch against a large weight): rung 12
    # splits K among each workgroup's waves
    ExtraWorkload("skinny_16x4096x14336", "gemm", 1, 16, 4096, 14336, 24, U11),
    # few output tiles and a long K (128- and 256-row tiles would keep a
    # sixteenth of the compute units busy): rung 13 splits K among the waves
    # of many small tiles
    ExtraWorkload("few_tiles_256x1024x8192", "gemm", 1, 256, 1024, 8192, 25, U11),
    ExtraWorkload("few_tiles_128x4096x14336", "gemm", 1, 128, 4096, 14336, 26, U11),
    # a small last round of tiles (2.25 rounds on 256 compute units, and a
    # ragged M): whole rounds unsplit, the remaining rows split K
    ExtraWorkload("splitk_rounds_6144x6144x6144", "splitk", 1, 6144, 6144, 6144, 18, U11),
    ExtraWorkload("splitk_rounds_6280x5888x4096", "splitk", 1, 6280, 5888, 4096, 19, U11),
    # 384 x 256 tiles (each staged B band feeds two waves of 192 A rows):
    # one round of them against 1.5 rounds of 256 x 256 tiles, and a shape
    # both tile sizes fill in whole rounds
    ExtraWorkload("wide_6144x4096x4096", "gemm", 1, 6144, 4096, 4096, 22, U11),
    ExtraWorkload("wide_12288x4096x4096", "gemm", 1, 12288, 4096, 4096, 23, U11),
    # a batch of mid-size products, one launch
    ExtraWorkload("batched_16x1024x1024x4096", "strided", 16, 1024, 1024, 4096, 14, U11),
    # attention scores S = Q K^T, 32 heads of 4096 x 4096, head dimension 128 and 64
    ExtraWorkload("attn_scores_h32_s4096_d128", "strided", 32, 4096, 4096, 128, 15, U11),
    ExtraWorkload("attn_scores_h32_s4096_d64", "strided", 32, 4096, 4096, 64, 16, U11),
    # the same with the heads interleaved in the rows of Q and K
    ExtraWorkload("attn_scores_rows_h32_s4096_d128", "heads_rows", 32, 4096, 4096, 128, 17, U11),
]
EXTRA_BY_NAME = {w.name: w for w in EXTRA_WORKLOADS}
