"""ag_matmul_run's argument checks on a live handle, through the C ABI.

Every device pointer must be 16-byte aligned, the output must not overlap an input, a
bias pointer must match has_bias, and every shard pointer must be given. A refused call
returns INVALID_ARG before anything is enqueued: the output keeps the NaN it was filled
with, and the handle runs correctly afterwards (a refusal does not poison it).
"""
import numpy as np
import pytest

from agmm_testlib import out_bits, run_gpu
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

INV = -1


def test_run_refuses_bad_pointers_and_enqueues_nothing():
    import torch
    import all_gather_gemm_amd as A
    w = Workload("refuse_run", 4, 4 * 128, 264, 520, "f16", "normal_sqrtk", True,
                 "m_contiguous", True, 121, rank=2)
    inp = make_inputs(w)
    dev = inp.to("cuda")
    ref = out_bits(run_gpu(w, inp, "fused", dev_inp=dev).out)
    op = A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank,
                    direct_local=w.direct_local, has_bias=True)
    s = torch.cuda.current_stream().cuda_stream
    out = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device="cuda")
    big = torch.empty(w.M * w.N + 64, dtype=torch.float16, device="cuda")
    shards = [t.data_ptr() for t in dev.shards]
    B, bias, o = dev.B.data_ptr(), dev.bias.data_ptr(), out.data_ptr()

    def run(sh=None, b=B, bi=bias, out_ptr=o):
        return A.ag_matmul_run(op.handle, shards if sh is None else sh, b, bi, out_ptr, s)

    bad = {
        "misaligned shard": run(sh=shards[:1] + [shards[1] + 2] + shards[2:]),
        "null shard": run(sh=shards[:3] + [0]),
        "misaligned B": run(b=B + 8),
        "misaligned bias": run(bi=bias + 2),
        "missing bias": run(bi=None),
        "misaligned out": run(out_ptr=o + 4),
        "null out": run(out_ptr=0),
        "out over a shard": run(out_ptr=shards[0]),
        "out over B": run(out_ptr=B),
        "out overlapping the bias": run(out_ptr=bias - 64),
    }
    for what, rc in bad.items():
        assert rc == INV, (what, rc)
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "a refused call wrote the output"
    # a handle without bias refuses a bias pointer
    nb = A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=False)
    assert A.ag_matmul_run(nb.handle, shards, B, bias, o, s) == INV
    nb.close()
    # the handle is not poisoned: a correct call still gives the reference output
    assert run() == 0
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(out), ref)
    assert op.sync_status() == 0
    # the output may sit anywhere outside the inputs, e.g. inside a larger allocation
    o2 = big[16:16 + w.M * w.N].view(w.M, w.N)
    assert run(out_ptr=o2.data_ptr()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(o2), ref)
    op.close()
