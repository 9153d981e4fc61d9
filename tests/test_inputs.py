"""The seeded operand generator: SplitMix64 against its published first
output, independence of chunking, determinism, and the moments of each
workload's distribution."""
import numpy as np
import pytest

from dense_fp16_gemm_nt_amd import inputs, workloads


def _splitmix64_scalar(state: int) -> int:
    # the published algorithm with Python integers (mod 2^64)
    mask = (1 << 64) - 1
    z = (state + 0x9E3779B97F4A7C15) & mask
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
    return z ^ (z >> 31)


def test_splitmix64_known_answer():
    # first output of SplitMix64 started from state 0
    assert int(inputs.splitmix64(np.array([0], dtype=np.uint64))[0]) == 0xE220A8397B1DCDAF
    xs = np.array([1, 2, 0xFFFFFFFFFFFFFFFF, 0x123456789ABCDEF0], dtype=np.uint64)
    got = inputs.splitmix64(xs)
    assert [int(v) for v in got] == [_splitmix64_scalar(int(x)) for x in xs]


def test_counter_layout():
    seed, stream, idx = 3, 1, 12345
    x = (seed * 0x9E3779B97F4A7C15 + stream * 0xD1B54A32D192ED03 + idx) & ((1 << 64) - 1)
    u = (_splitmix64_scalar(x) >> 11) * 2.0 ** -53
    assert inputs.uniform01(seed, stream, idx, 1)[0] == u


@pytest.mark.parametrize("dist", [workloads.U11, workloads.N025])
def test_chunking_does_not_change_values(dist, monkeypatch):
    a = inputs.generate(64, 1000, 7, 0, dist)
    monkeypatch.setattr(inputs, "_CHUNK", 4096)
    b = inputs.generate(64, 1000, 7, 0, dist)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_deterministic_and_streams_differ():
    a1, b1 = inputs.operands(64, 48, 128, 5, workloads.U05)
    a2, b2 = inputs.operands(64, 48, 128, 5, workloads.U05)
    assert np.array_equal(a1.view(np.uint16), a2.view(np.uint16))
    assert np.array_equal(b1.view(np.uint16), b2.view(np.uint16))
    assert a1.shape == (64, 128) and b1.shape == (48, 128)
    assert not np.array_equal(a1[:48].view(np.uint16), b1.view(np.uint16))
    a3, _ = inputs.operands(64, 48, 128, 6, workloads.U05)
    assert not np.array_equal(a1.view(np.uint16), a3.view(np.uint16))


@pytest.mark.parametrize("dist,mean,var,bound", [
    (workloads.U11, 0.0, 1.0 / 3.0, 1.0),
    (workloads.U05, 0.0, 1.0 / 12.0, 0.5),
    (workloads.N025, 0.0, 0.0625, 4.0),
])
def test_moments(dist, mean, var, bound):
    x = inputs.generate(512, 1024, 11, 0, dist).astype(np.float64)
    n = x.size
    assert abs(x.mean() - mean) < 5 * np.sqrt(var / n)
    assert abs(x.var() / var - 1.0) < 0.01
    assert np.abs(x).max() <= bound
    assert np.isfinite(x).all()


def test_batched_operands_split_one_draw_in_order():
    A3, B3 = inputs.batched_operands(3, 4, 5, 16, 9, workloads.U11)
    A, B = inputs.operands(12, 15, 16, 9, workloads.U11)
    assert A3.shape == (3, 4, 16) and B3.shape == (3, 5, 16)
    assert np.array_equal(A3.reshape(12, 16), A) and np.array_equal(B3.reshape(15, 16), B)


def test_extra_workloads_are_well_formed():
    names = [w.name for w in workloads.EXTRA_WORKLOADS]
    assert len(set(names)) == len(names)
    for w in workloads.EXTRA_WORKLOADS:
        assert w.kind in ("gemm", "splitk", "strided", "heads_rows")
        assert w.batch >= 1 and min(w.M, w.N, w.K) >= 1
        assert w.kind not in ("gemm", "splitk") or w.batch == 1
        assert w.flop == 2 * w.batch * w.M * w.N * w.K


def test_periodic_index():
    assert inputs.periodic_index(7, 3, 1).tolist() == [1, 2, 0, 1, 2, 0, 1]
    idx = inputs.periodic_index(10 ** 6 + 3, 997, 13)
    assert idx.dtype == np.int64 and idx.min() == 0 and idx.max() == 996
    assert idx[986895] == (986895 + 13) % 997
