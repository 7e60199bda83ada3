"""The entry point that allocates nothing (ag_matmul_run_static), through the C ABI: its
output against the handle path's (ag_matmul_create + ag_matmul_run, the same kernels and K
order: bit for bit) and against the fp64 oracle within the output tolerance, on consecutive
calls whose shapes shrink (the scratch keeps the previous call's contents, so stale tables,
flags or staging would show), for the fused and baseline algorithms and both staging
layouts; a workspace beyond the scratch is refused with TOO_LARGE before anything runs, and
repeated calls change the device's free memory by nothing."""
import numpy as np
import pytest

from agmm_testlib import assert_close, oracle_full, out_bits, run_gpu
from workloads import LARGE_16384, MID_4096, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # the largest workload that fits the scratch, then smaller ones, in this order
    MID_4096,
    Workload("static_mid_m", 4, 4 * 512, 1032, 2056, "bf16", "normal_sqrtk", True,
             "m_contiguous", True, 71, rank=1),
    Workload("static_ragged", 3, 3 * 200, 328, 424, "f16", "normal_sqrtk", True,
             "k_contiguous", True, 72, rank=2),
    Workload("static_tiny", 2, 256, 256, 256, "bf16", "uniform", False, "k_contiguous", True, 73),
]


def _static_run(A, w, dev, algo, out):
    import torch
    desc = A.ag_matmul_desc_init(
        D=w.D, M=w.M, N=w.N, K=w.K, rank=w.rank, dtype={"f16": A.F16, "bf16": A.BF16}[w.dtype],
        layout={"k_contiguous": A.K_CONTIGUOUS, "m_contiguous": A.M_CONTIGUOUS}[w.layout],
        algo={"fused": A.ALGO_FUSED, "baseline": A.ALGO_BASELINE}[algo],
        direct_local=int(w.direct_local), has_bias=int(w.has_bias))
    rc = A.ag_matmul_run_static(desc, [t.data_ptr() for t in dev.shards], dev.B.data_ptr(),
                                dev.bias.data_ptr() if dev.bias is not None else None,
                                out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return rc


def test_no_alloc_entry_point():
    import torch
    import all_gather_gemm_amd as A
    outs = {}
    for algo in ("fused", "baseline"):
        for w in CASES:
            print(f"case {w.name} {algo}", flush=True)
            inp = make_inputs(w)
            dev = inp.to("cuda")
            out = torch.full((w.M, w.N), float("nan"), dtype=w.torch_dtype(), device="cuda")
            assert _static_run(A, w, dev, algo, out) == 0
            torch.cuda.synchronize()
            got = out_bits(out)
            ref = out_bits(run_gpu(w, inp, algo, dev_inp=dev).out)
            assert np.array_equal(got, ref), (w.name, algo)
            if w.name not in outs:
                C, _ = oracle_full(w, inp)
                assert_close(w, got, C, f"static {algo}")
                outs[w.name] = got
            else:
                assert np.array_equal(got, outs[w.name]), (w.name, algo)
    # the same shape twice more: the tables are reused, flags and counters cleared each call,
    # and the device's free memory does not change
    w = CASES[2]
    inp = make_inputs(w)
    dev = inp.to("cuda")
    out = torch.empty((w.M, w.N), dtype=w.torch_dtype(), device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        out.fill_(float("nan"))
        assert _static_run(A, w, dev, "fused", out) == 0
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), outs[w.name])
    assert torch.cuda.mem_get_info()[0] == free0
    # too large for the scratch (a 256 MiB staging buffer): refused, nothing enqueued
    big = LARGE_16384
    desc = A.ag_matmul_desc_init(D=big.D, M=big.M, N=big.N, K=big.K, has_bias=1,
                                 layout=A.M_CONTIGUOUS)
    rc = A.ag_matmul_run_static(desc, [0] * big.D, 0, 0, 0, 0)
    assert rc == -8  # TOO_LARGE
    # refused options
    for kw in (dict(debug=1), dict(gather_a=1), dict(tail_split=1),
               dict(algo=A.ALGO_PIPELINED), dict(fetch_kernel=1)):
        d = A.ag_matmul_desc_init(D=2, M=256, N=256, K=256, **kw)
        assert A.ag_matmul_run_static(d, [0, 0], 0, 0, 0, 0) == -2, kw
