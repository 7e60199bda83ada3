"""Seeded random problems through the C ABI against the fp64 oracle.

Each of 40 small problems draws its own shard count (1 to 12), rank, shard rows (multiples
of 8), N and K (multiples of 8, including values below one tile), type, staging layout,
bias, direct-local reading, tile size, k-group size, fetcher count and algorithm. The
planner and the kernel families then meet combinations that the hand-picked cases do not
list. Every output must lie within the oracle's tolerance, and the fused output must be
bit-identical to the baseline's (same GEMM code, same K order) when no tile is split. 30
larger problems (up to 8192 rows, N up to 4096, K up to 8192, 16 shards, 128 fetchers)
follow the same recipe with wider ranges.
"""
import numpy as np
import pytest

from agmm_testlib import assert_close, oracle_full, out_bits, run_gpu
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _problems(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.integers(1, 13))
        Ms = 8 * int(rng.integers(1, 1 + (1536 // 8) // D + 1))
        N = 8 * int(rng.integers(1, 129))
        K = 8 * int(rng.integers(1, 257))
        dt = str(rng.choice(["f16", "bf16"]))
        layout = str(rng.choice(["k_contiguous", "m_contiguous"]))
        bias = bool(rng.integers(0, 2))
        direct = bool(rng.integers(0, 4) > 0)
        dist = str(rng.choice(["normal_sqrtk", "uniform_sqrtk"]))
        tun = {}
        bm = int(rng.choice([0, 0, 64, 128, 256]))
        if bm:
            tun["block_m"] = bm
        if rng.integers(0, 2):
            tun["k_per_flag"] = int(rng.choice([1, 2, 4, 8, 16]))
        if rng.integers(0, 3) == 0:
            tun["num_fetch_wgs"] = int(rng.integers(1, 65))
        if rng.integers(0, 4) == 0:
            tun["tail_split"] = 1
        w = Workload(f"rnd{i:02d}_{D}x{Ms}_{N}_{K}_{dt}_{layout[0]}", D, D * Ms, N, K, dt, dist,
                     bias, layout, direct, 5000 + i, rank=int(rng.integers(0, D)))
        out.append((w, tun))
    return out


def _large_problems(n=30, seed=5, max_macs=2e10):
    """Larger draws: 1 to 16 shards of up to 8192 rows in all, N up to 4096, K up to 8192,
    k-groups up to 32 K-tiles and up to 128 fetchers; problems over max_macs are redrawn, so
    the oracle stays within a second per problem."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        D = int(rng.integers(1, 17))
        Ms = 8 * int(rng.integers(1, 1 + 8192 // 8 // D))
        N = 8 * int(rng.integers(1, 513))
        K = 8 * int(rng.integers(1, 1025))
        if D * Ms * N * K > max_macs:
            continue
        dt = str(rng.choice(["f16", "bf16"]))
        layout = str(rng.choice(["k_contiguous", "m_contiguous"]))
        bias = bool(rng.integers(0, 2))
        direct = bool(rng.integers(0, 4) > 0)
        tun = {}
        bm = int(rng.choice([0, 0, 64, 128, 256]))
        if bm:
            tun["block_m"] = bm
        if rng.integers(0, 2):
            tun["k_per_flag"] = int(rng.choice([1, 2, 4, 8, 16, 32]))
        if rng.integers(0, 3) == 0:
            tun["num_fetch_wgs"] = int(rng.integers(1, 129))
        if rng.integers(0, 4) == 0:
            tun["tail_split"] = 1
        i = len(out)
        w = Workload(f"big{i:02d}_{D}x{Ms}_{N}_{K}_{dt}_{layout[0]}", D, D * Ms, N, K, dt,
                     "normal_sqrtk", bias, layout, direct, 9000 + i, rank=int(rng.integers(0, D)))
        out.append((w, tun))
    return out


PROBLEMS = _problems() + _large_problems()


@pytest.mark.parametrize("w,tun", PROBLEMS, ids=[p[0].name for p in PROBLEMS])
def test_random_problem(w, tun):
    print(f"case {w.name} {tun}", flush=True)
    inp = make_inputs(w)
    dev = inp.to("cuda")
    C, _ = oracle_full(w, inp)
    f = run_gpu(w, inp, "fused", dev_inp=dev, **tun)
    fo = out_bits(f.out)
    assert_close(w, fo, C, f"fused {tun}")
    b = run_gpu(w, inp, "baseline", dev_inp=dev, **tun)
    bo = out_bits(b.out)
    assert_close(w, bo, C, f"baseline {tun}")
    if f.config["split_tiles"] == 0 and b.config["split_tiles"] == 0:
        assert np.array_equal(fo, bo), w.name
