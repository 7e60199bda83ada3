"""Stress of the fused kernel's flag protocol on the GPU (the fetch perturbed through its debug
knobs, results unchanged). Fetchers sleep a hash-seeded number of back-off steps before each
unit, and/or claim the units in reverse fetch order, so units complete far out of the order
the tiles need them; every wait must still see the data it acquired. The output must stay
bit-identical to the barrier baseline's (same GEMM kernel and K order), with no timeout
recorded and every staged unit's flag at the run's epoch, over runs that alternate between
two input sets on one handle (a wait that let a tile read stale staging would show the other
set's data).
"""
import numpy as np
import pytest

from agmm_testlib import out_bits, run_gpu
from oracle import schedule_model as sm
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (D, M_s, N, K, dtype, layout, block_m, k_per_flag, fetchers): per-k-group waits in the
    # K loop (fetchers < units) and whole-row waits (one fetcher per unit)
    (4, 256, 512, 1024, "f16", "m_contiguous", 128, 4, 5),
    (8, 128, 392, 776, "bf16", "k_contiguous", 64, 2, 7),
    (3, 512, 1032, 2056, "f16", "k_contiguous", 256, 8, 4),
    (2, 256, 264, 1032, "bf16", "m_contiguous", 128, 8, 0),
]
KNOBS = [
    dict(debug_fetch_reverse=1),
    dict(debug_fetch_delay=64, debug_fetch_seed=1),
    dict(debug_fetch_delay=200, debug_fetch_seed=7, debug_fetch_reverse=1),
]


@pytest.mark.parametrize("knobs", KNOBS, ids=["reverse", "delay", "reverse_delay"])
@pytest.mark.parametrize("D,Ms,N,K,dt,layout,bm,kpf,nf", CASES)
def test_perturbed_fetch_bit_identical(D, Ms, N, K, dt, layout, bm, kpf, nf, knobs):
    import torch
    import all_gather_gemm_amd as A
    w = Workload(f"stress_{D}x{Ms}_{N}_{K}_{dt}_{layout}", D, D * Ms, N, K, dt, "normal_sqrtk",
                 True, layout, True, 500 + D + K, rank=D // 2)
    print(f"case {w.name} {knobs}", flush=True)
    sets = [make_inputs(w, seed=w.seed + i) for i in range(2)]
    devs = [s.to("cuda") for s in sets]
    refs = [out_bits(run_gpu(w, s, "baseline", dev_inp=d, block_m=bm).out)
            for s, d in zip(sets, devs)]
    tun = dict(block_m=bm, k_per_flag=kpf, **knobs)
    if nf:
        tun["num_fetch_wgs"] = nf
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=dt, layout=layout, rank=w.rank, has_bias=True,
                    **tun)
    cfg = op.config.as_dict()
    g = sm.Geometry(w.D, w.M, w.N, w.K, cfg["block_m"], cfg["block_n"], cfg["block_k"],
                    cfg["k_per_flag"], w.rank, True, cfg["num_fetch_wgs"], cfg["num_wgs"],
                    num_cus=cfg["num_cus"])
    outs = [torch.empty((w.M, w.N), dtype=w.torch_dtype(), device="cuda") for _ in range(6)]
    for it in range(6):
        i = it % 2
        op.run(devs[i].shards, devs[i].B, devs[i].bias, out=outs[it])
    assert op.sync_status() == 0
    for it in range(6):
        assert np.array_equal(out_bits(outs[it]), refs[it % 2]), (it, knobs)
    assert np.array_equal(op.flags(), sm.expected_flags(g, 6))
    op.close()
