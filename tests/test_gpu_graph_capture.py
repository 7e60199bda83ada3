"""HIP graph capture, through the C ABI.

ag_matmul_run_static clears its flags and counters in every call and runs at the first
epoch, so a graph captured from it is valid on every replay: each replay, with the inputs
rewritten in place and another static call (another shape, which overwrites the scratch's
tables and flags) run eagerly before it, gives the handle path's output bit for bit, for the
fused and baseline algorithms and both staging layouts.

A handle's kernels take a run's epoch from the run counter in its workspace, which the last
workgroup of every run advances, so a captured run of a handle replays correctly too, also
interleaved with eager runs of the same handle on the same stream: fused runs in both
layouts, runs with split tiles (whose piece counters are epoch-valued), the gathered-A run,
the host pipeline (its chunk streams join the capture through its events) and the per-tile
flag all-reduce. Every replay and every eager run must give the eager
output bit for bit, and after all of them every staged unit's flag must equal the number of
runs the device executed. A debug run (it synchronizes its stream) and a fetch-kernel run
(it orders a stream of the handle's with events) refuse a capturing stream with UNSUPPORTED
and enqueue nothing.
"""
import ctypes

import numpy as np
import pytest

from agmm_testlib import assert_close, oracle_full, out_bits, run_gpu
import oracle
from workloads import Workload, bits, make_inputs

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


def _raw_run(A, op, dev, out, stream, a_out=None):
    ptrs = [t.data_ptr() for t in dev.shards]
    bias = dev.bias.data_ptr() if dev.bias is not None else None
    if a_out is not None:
        return A.ag_matmul_run_gather(op.handle, ptrs, dev.B.data_ptr(), bias, out.data_ptr(),
                                      a_out.data_ptr(), stream)
    return A.ag_matmul_run(op.handle, ptrs, dev.B.data_ptr(), bias, out.data_ptr(), stream)


HANDLES = [
    # (name, workload, tunables)
    ("fused_m", Workload("graph_h_m", 2, 2 * 544, 1024, 2048, "f16", "normal_sqrtk", True,
                         "m_contiguous", True, 96, rank=1), dict(block_m=64)),
    ("fused_k", Workload("graph_h_k", 4, 4 * 200, 328, 1032, "bf16", "normal_sqrtk", True,
                         "k_contiguous", True, 97, rank=2), dict(block_m=128, k_per_flag=2)),
    ("fused_split", Workload("graph_h_s", 2, 2 * 544, 1024, 2048, "f16", "normal_sqrtk", True,
                             "m_contiguous", True, 98, rank=1),
     dict(block_m=64, num_fetch_wgs=8, tail_split=1)),
    ("baseline_split", Workload("graph_h_bs", 2, 2 * 544, 1024, 2048, "bf16", "normal_sqrtk",
                                False, "k_contiguous", True, 99, rank=0),
     dict(block_m=64, algo="baseline", tail_split=1)),
    ("gather_a", Workload("graph_h_g", 4, 4 * 200, 328, 1032, "bf16", "normal_sqrtk", True,
                          "k_contiguous", True, 100, rank=3), dict(gather_a=True)),
    # the host stream pipeline: its chunk streams join the capture through its events
    ("pipelined", Workload("graph_h_p", 4, 4 * 256, 392, 520, "f16", "normal_sqrtk", True,
                           "k_contiguous", True, 101, rank=2),
     dict(block_m=64, algo="pipelined", pipeline_chunks=4)),
]


@pytest.mark.parametrize("name,w,tun", HANDLES, ids=[h[0] for h in HANDLES])
def test_handle_run_captured_and_replayed(name, w, tun):
    import torch
    import all_gather_gemm_amd as A
    from oracle import schedule_model as sm
    print(f"case {name} {w.name} {tun}", flush=True)
    tun = dict(tun)
    algo = tun.pop("algo", "fused")
    gather = tun.get("gather_a", False)
    sets = [make_inputs(w, seed=w.seed + i) for i in range(2)]
    srcs = [s.to("cuda") for s in sets]
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, algo=algo, rank=w.rank,
                    has_bias=w.has_bias, **tun)
    cfg = op.config.as_dict()
    if "tail_split" in tun:
        assert cfg["split_tiles"] > 0
    td = w.torch_dtype()
    out = torch.empty((w.M, w.N), dtype=td, device="cuda")
    a_out = torch.empty((w.M, w.K), dtype=td, device="cuda") if gather else None
    stream = lambda: torch.cuda.current_stream().cuda_stream
    # eager references, each set run twice (runs 1 .. 4)
    refs = []
    for i in (0, 1, 0, 1):
        assert _raw_run(A, op, srcs[i], out, stream(), a_out) == 0
        torch.cuda.synchronize()
        b = out_bits(out)
        if len(refs) < 2:
            refs.append(b)
        assert np.array_equal(b, refs[i]), (name, "eager", i)
    runs = 4
    dev = sets[0].to("cuda")   # the buffers the graph reads
    g = torch.cuda.CUDAGraph()
    rcs = []
    with torch.cuda.graph(g):
        rcs.append(_raw_run(A, op, dev, out, stream(), a_out))
    assert rcs == [0]
    # replays, eager runs of the same handle between them
    for it in range(6):
        i = it % 2
        _copy_into(dev, srcs[i])
        out.fill_(float("nan"))
        g.replay()
        runs += 1
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), refs[i]), (name, "replay", it)
        if gather:
            assert np.array_equal(out_bits(a_out).reshape(w.M, w.K),
                                  oracle.all_gather([bits(x) for x in sets[i].shards])), it
        if it % 2 == 1:
            j = 1 - i
            out.fill_(float("nan"))
            assert _raw_run(A, op, srcs[j], out, stream(), a_out) == 0
            runs += 1
            torch.cuda.synchronize()
            assert np.array_equal(out_bits(out), refs[j]), (name, "eager between", it)
    assert op.sync_status() == 0
    if algo == "fused" and cfg["num_units"] > 0:
        geo = sm.Geometry(w.D, w.M, w.N, w.K, cfg["block_m"], cfg["block_n"], cfg["block_k"],
                          cfg["k_per_flag"], w.rank, True, cfg["num_fetch_wgs"],
                          cfg["num_wgs"], num_cus=cfg["num_cus"], gather_a=gather)
        assert np.array_equal(op.flags(), sm.expected_flags(geo, runs)), name
    if name == "fused_m":
        C, _ = oracle_full(w, sets[0])
        _copy_into(dev, srcs[0])
        g.replay()
        torch.cuda.synchronize()
        assert_close(w, out_bits(out), C, "handle, replayed")
    del g
    op.close()


def test_allreduce_flags_captured_and_replayed():
    """The per-tile flag all-reduce captured and replayed between eager runs: bit-identical
    to the eager run every time (its result does not depend on timing)."""
    import torch
    import all_gather_gemm_amd as A
    D, M, N, Kl = 3, 320, 264, 192
    gen = torch.Generator().manual_seed(95)
    Ap = [(torch.randn(M, Kl, generator=gen) / 8).half().cuda() for _ in range(D)]
    Bp = [(torch.randn(Kl, N, generator=gen) / 8).half().cuda() for _ in range(D)]
    bias = torch.randn(N, generator=gen).half().cuda()
    h = A.GemmAllReduceFlags(D, M, N, Kl, block_m=64)
    o = torch.empty((M, N), dtype=torch.float16, device="cuda")
    h.run(Ap, Bp, bias, out=o)
    torch.cuda.synchronize()
    ref = out_bits(o)
    ap = (ctypes.c_void_p * D)(*[ctypes.c_void_p(t.data_ptr()) for t in Ap])
    bp = (ctypes.c_void_p * D)(*[ctypes.c_void_p(t.data_ptr()) for t in Bp])
    g = torch.cuda.CUDAGraph()
    rcs = []
    with torch.cuda.graph(g):
        rcs.append(A.lib.ag_gemm_ar_flags_run(
            ctypes.c_void_p(h.handle), ap, bp, ctypes.c_void_p(bias.data_ptr()),
            ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    assert rcs == [0]
    for it in range(4):
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(o), ref), ("replay", it)
        o.fill_(float("nan"))
        h.run(Ap, Bp, bias, out=o)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(o), ref), ("eager", it)
    del g
    h.close()


def test_debug_and_fetch_kernel_runs_refuse_capture():
    import torch
    import all_gather_gemm_amd as A
    w = Workload("graph_refuse", 2, 2 * 544, 1024, 2048, "f16", "normal_sqrtk", True,
                 "m_contiguous", True, 94, rank=1)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    dev = inp.to("cuda")
    plain = out_bits(run_gpu(w, inp, "baseline", dev_inp=dev, block_m=64).out)
    handles = {
        "fetch_kernel": A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank,
                                   has_bias=True, block_m=64, fetch_kernel=1),
        "debug": A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=True,
                            block_m=64, debug=True),
    }
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    for name, op in handles.items():
        print(f"  handle {name}", flush=True)
        op.run(dev.shards, dev.B, dev.bias, out=out)   # one eager run first
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), plain), name
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
            assert np.array_equal(out_bits(out), plain), name
        assert op.sync_status() == 0
        op.close()
