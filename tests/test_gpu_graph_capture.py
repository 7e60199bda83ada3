"""HIP graph capture, through the C ABI.

ag_matmul_run_static clears its flags and counters in every call and runs at the first
epoch, so a graph captured from it is valid on every replay: each replay, with the inputs
rewritten in place and another static call (another shape, which overwrites the scratch's
tables and flags) run eagerly before it, gives the handle path's output bit for bit, for the
fused and baseline algorithms and both staging layouts.

The runs whose kernels compare flags or split counters with a handle's run number (a fused
handle, a handle with split tiles, the per-tile flag all-reduce) fix that number when they
are enqueued, so they refuse a capturing stream with UNSUPPORTED and enqueue nothing; the
handle then runs eagerly as before. A debug run, which synchronizes its stream, refuses it
too. A baseline handle without split tiles compares nothing
with a run number and may be captured and replayed.
"""
import ctypes

import numpy as np
import pytest

from agmm_testlib import assert_close, oracle_full, out_bits, run_gpu
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

UNSUPPORTED = -2

STATIC = [
    Workload("graph_ragged", 3, 3 * 200, 328, 424, "f16", "normal_sqrtk", True,
             "k_contiguous", True, 91, rank=2),
    Workload("graph_mid_m", 4, 4 * 512, 1032, 2056, "bf16", "normal_sqrtk", True,
             "m_contiguous", True, 92, rank=1),
]
# run eagerly between replays: another shape, so the scratch's tables and flags change
OTHER = Workload("graph_other", 2, 256, 256, 256, "bf16", "uniform", False, "k_contiguous",
                 True, 93)


def _desc(A, w, algo):
    return A.ag_matmul_desc_init(
        D=w.D, M=w.M, N=w.N, K=w.K, rank=w.rank, dtype={"f16": A.F16, "bf16": A.BF16}[w.dtype],
        layout={"k_contiguous": A.K_CONTIGUOUS, "m_contiguous": A.M_CONTIGUOUS}[w.layout],
        algo={"fused": A.ALGO_FUSED, "baseline": A.ALGO_BASELINE}[algo],
        direct_local=int(w.direct_local), has_bias=int(w.has_bias))


def _static(A, desc, dev, out):
    import torch
    return A.ag_matmul_run_static(desc, [t.data_ptr() for t in dev.shards], dev.B.data_ptr(),
                                  dev.bias.data_ptr() if dev.bias is not None else None,
                                  out.data_ptr(), torch.cuda.current_stream().cuda_stream)


def _copy_into(dst, src):
    for a, b in zip(dst.shards, src.shards):
        a.copy_(b)
    dst.B.copy_(src.B)
    if dst.bias is not None:
        dst.bias.copy_(src.bias)


@pytest.mark.parametrize("algo", ["fused", "baseline"])
@pytest.mark.parametrize("w", STATIC, ids=[w.name for w in STATIC])
def test_static_run_captured_and_replayed(w, algo):
    import torch
    import all_gather_gemm_amd as A
    print(f"case {w.name} {algo}", flush=True)
    sets = [make_inputs(w, seed=w.seed + i) for i in range(2)]
    srcs = [s.to("cuda") for s in sets]
    refs = [out_bits(run_gpu(w, s, algo, dev_inp=d).out) for s, d in zip(sets, srcs)]
    other_inp = make_inputs(OTHER)
    other_dev = other_inp.to("cuda")
    other_ref = out_bits(run_gpu(OTHER, other_inp, "fused", dev_inp=other_dev).out)
    other_desc = _desc(A, OTHER, "fused")
    other_out = torch.empty((OTHER.M, OTHER.N), dtype=OTHER.torch_dtype(), device="cuda")

    dev = sets[0].to("cuda")   # the buffers the graph reads
    out = torch.full((w.M, w.N), float("nan"), dtype=w.torch_dtype(), device="cuda")
    desc = _desc(A, w, algo)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # eager warm-up on a side stream, as before any capture
        assert _static(A, desc, dev, out) == 0
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(out), refs[0])

    g = torch.cuda.CUDAGraph()
    rcs = []
    with torch.cuda.graph(g):
        rcs.append(_static(A, desc, dev, out))
    assert rcs == [0]
    for it in range(5):
        i = it % 2
        _copy_into(dev, srcs[i])
        assert _static(A, other_desc, other_dev, other_out) == 0
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), refs[i]), (w.name, algo, it)
        assert np.array_equal(out_bits(other_out), other_ref), (w.name, algo, it)
    if algo == "fused" and w is STATIC[0]:
        C, _ = oracle_full(w, sets[0])
        _copy_into(dev, srcs[0])
        g.replay()
        torch.cuda.synchronize()
        assert_close(w, out_bits(out), C, "static, replayed")
    # eager calls after the capture still give the same bits (every call now writes its
    # tables, since a replay may have rewritten them)
    _copy_into(dev, srcs[1])
    assert _static(A, desc, dev, out) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(out), refs[1])
    del g


def _raw_run(A, op, dev, out, stream):
    return A.ag_matmul_run(op.handle, [t.data_ptr() for t in dev.shards], dev.B.data_ptr(),
                           dev.bias.data_ptr() if dev.bias is not None else None,
                           out.data_ptr(), stream)


def test_epoch_runs_refuse_capture():
    import torch
    import all_gather_gemm_amd as A
    w = Workload("graph_refuse", 2, 2 * 544, 1024, 2048, "f16", "normal_sqrtk", True,
                 "m_contiguous", True, 94, rank=1)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    dev = inp.to("cuda")
    plain = out_bits(run_gpu(w, inp, "baseline", dev_inp=dev, block_m=64).out)
    handles = {
        "fused": A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=True,
                            block_m=64),
        "split": A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=True,
                            block_m=64, algo="baseline", tail_split=1),
        "fetch_kernel": A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank,
                                   has_bias=True, block_m=64, fetch_kernel=1),
        # a debug run synchronizes its stream
        "debug": A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=True,
                            block_m=64, algo="baseline", debug=True),
    }
    assert handles["split"].config.split_tiles > 0
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    for name, op in handles.items():
        print(f"  handle {name}", flush=True)
        op.run(dev.shards, dev.B, dev.bias, out=out)   # one eager run first
        torch.cuda.synchronize()
        ref = out_bits(out)
        if name != "split":   # split tiles sum their K pieces in another order
            assert np.array_equal(ref, plain), name
        g = torch.cuda.CUDAGraph()
        rcs = []
        with torch.cuda.graph(g):
            rcs.append(_raw_run(A, op, dev, out, torch.cuda.current_stream().cuda_stream))
        assert rcs == [UNSUPPORTED], name
        del g
        # nothing was enqueued and the handle is as it was: the next eager runs are correct
        for _ in range(2):
            out.fill_(float("nan"))
            op.run(dev.shards, dev.B, dev.bias, out=out)
            torch.cuda.synchronize()
            assert np.array_equal(out_bits(out), ref), name
        assert op.sync_status() == 0
        op.close()

    # the per-tile flag all-reduce: refused the same way
    D, M, N, Kl = 2, 128, 256, 192
    gen = torch.Generator().manual_seed(95)
    Ap = [torch.randn(M, Kl, generator=gen).half().cuda() for _ in range(D)]
    Bp = [torch.randn(Kl, N, generator=gen).half().cuda() for _ in range(D)]
    h = A.GemmAllReduceFlags(D, M, N, Kl)
    r0 = out_bits(h.run(Ap, Bp))
    torch.cuda.synchronize()
    o = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ap = (ctypes.c_void_p * D)(*[ctypes.c_void_p(t.data_ptr()) for t in Ap])
    bp = (ctypes.c_void_p * D)(*[ctypes.c_void_p(t.data_ptr()) for t in Bp])
    g = torch.cuda.CUDAGraph()
    rcs = []
    with torch.cuda.graph(g):
        rcs.append(A.lib.ag_gemm_ar_flags_run(
            ctypes.c_void_p(h.handle), ap, bp, None, ctypes.c_void_p(o.data_ptr()),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    assert rcs == [UNSUPPORTED]
    del g
    o2 = h.run(Ap, Bp)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(o2), r0)
    h.close()

    # a baseline handle without split tiles compares nothing with a run number: captured,
    # its replays match the eager run
    op = A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=True,
                    block_m=64, algo="baseline")
    assert op.config.split_tiles == 0
    op.run(dev.shards, dev.B, dev.bias, out=out)
    g = torch.cuda.CUDAGraph()
    rcs = []
    with torch.cuda.graph(g):
        rcs.append(_raw_run(A, op, dev, out, torch.cuda.current_stream().cuda_stream))
    assert rcs == [0]
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), plain)
    del g
    op.close()
