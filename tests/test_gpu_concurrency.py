"""Handles run concurrently on two streams, through the C ABI.

Each handle owns its workspace (staging, flags, counters, queues), so runs of different
handles on different streams, enqueued so that they can overlap, do not interfere. When the
persistent grids of two handles share the chip, each grid's fetcher workgroups are its
lowest-numbered ones and are dispatched first, so every flag wait of either grid ends. Runs
of each handle alternate between two input sets on its stream, with the other stream's runs
enqueued between them. Every output must match the same handle's eager run on the same
inputs bit for bit, and one of each handle's outputs must be within the oracle's tolerance.
"""
import numpy as np
import pytest

from agmm_testlib import assert_close, oracle_full, out_bits, run_gpu
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

# small grids (tens of workgroups), so both fit on the chip at once
PAIRS = [
    (Workload("conc_a", 4, 4 * 256, 1032, 2056, "bf16", "normal_sqrtk", True, "m_contiguous",
              True, 61, rank=1), dict(block_m=128),
     Workload("conc_b", 3, 3 * 200, 328, 424, "f16", "normal_sqrtk", True, "k_contiguous",
              True, 62, rank=2), dict(block_m=64)),
    (Workload("conc_c", 8, 8 * 256, 768, 1024, "f16", "normal_sqrtk", False, "k_contiguous",
              True, 63, rank=5), dict(),
     Workload("conc_d", 2, 2 * 264, 520, 1032, "bf16", "uniform", True, "m_contiguous",
              True, 64, rank=0), dict(block_m=128, k_per_flag=2)),
]


@pytest.mark.parametrize("algo_b", ["fused", "baseline"])
@pytest.mark.parametrize("wa,ta,wb,tb", PAIRS, ids=[p[0].name + "+" + p[2].name for p in PAIRS])
def test_two_handles_on_two_streams(wa, ta, wb, tb, algo_b):
    import torch
    import all_gather_gemm_amd as A
    print(f"case {wa.name}(fused) + {wb.name}({algo_b})", flush=True)
    jobs = []
    for w, tun, algo in ((wa, ta, "fused"), (wb, tb, algo_b)):
        sets = [make_inputs(w, seed=w.seed + i) for i in range(2)]
        devs = [s.to("cuda") for s in sets]
        refs = [out_bits(run_gpu(w, s, algo, dev_inp=d, **tun).out) for s, d in zip(sets, devs)]
        op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, algo=algo,
                        rank=w.rank, has_bias=w.has_bias, **tun)
        outs = [torch.full((w.M, w.N), float("nan"), dtype=w.torch_dtype(), device="cuda")
                for _ in range(4)]
        jobs.append(dict(w=w, sets=sets, devs=devs, refs=refs, op=op, outs=outs,
                         stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    for it in range(4):
        for j in jobs:
            d = j["devs"][it % 2]
            with torch.cuda.stream(j["stream"]):
                j["op"].run(d.shards, d.B, d.bias, out=j["outs"][it])
    for j in jobs:
        j["stream"].synchronize()
    for j in jobs:
        for it in range(4):
            assert np.array_equal(out_bits(j["outs"][it]), j["refs"][it % 2]), (j["w"].name, it)
        assert j["op"].sync_status() == 0
        C, _ = oracle_full(j["w"], j["sets"][1])
        assert_close(j["w"], out_bits(j["outs"][3]), C, "concurrent")
        j["op"].close()
