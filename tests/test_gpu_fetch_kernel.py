"""The fused algorithm with its fetch as a kernel of its own (desc.fetch_kernel = 1): a fetch
kernel on a stream of the handle's, one workgroup per CU beside the persistent GEMM grid,
which then has no fetchers and waits for each staged k-group in its K loop.

Same bar as the in-grid fetchers: the output bit-identical to the barrier baseline's (same
GEMM kernel and K order) and within the oracle's tolerance, every staged unit's flag at the
run's epoch, runs alternating between two input sets on one handle, the fetch perturbed by
the stress knobs, the gathered A bit-exact, the fetch kernel's trace records covering every
unit once, and a never-published unit reported as a timeout with every workgroup of both
kernels exiting.
"""
import numpy as np
import pytest

from agmm_testlib import assert_close, oracle_full, out_bits, run_gpu
from oracle import schedule_model as sm
from workloads import Workload, bits, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (D, M_s, N, K, dtype, layout, block_m (0 = auto), k_per_flag (0 = auto), fetch wgs
    # (0 = auto), rank): ragged tiles and K tails, both layouts and dtypes, every tile family
    (2, 136, 264, 1032, "f16", "k_contiguous", 128, 4, 0, 1),
    (4, 72, 520, 200, "bf16", "m_contiguous", 64, 1, 3, 0),
    (3, 200, 328, 424, "f16", "m_contiguous", 256, 2, 0, 2),
    (8, 128, 1024, 1024, "bf16", "k_contiguous", 0, 0, 0, 3),
    (8, 512, 1024, 2048, "f16", "m_contiguous", 0, 0, 17, 5),
    (2, 520, 520, 1032, "bf16", "k_contiguous", 256, 8, 0, 0),
]
KNOBS = [dict(), dict(debug_fetch_reverse=1), dict(debug_fetch_delay=64, debug_fetch_seed=3)]


@pytest.mark.parametrize("knobs", KNOBS, ids=["plain", "reverse", "delay"])
@pytest.mark.parametrize("D,Ms,N,K,dt,layout,bm,kpf,nf,rank", CASES)
def test_fetch_kernel_bit_identical(D, Ms, N, K, dt, layout, bm, kpf, nf, rank, knobs):
    import torch
    import all_gather_gemm_amd as A
    w = Workload(f"fk_{D}x{Ms}_{N}_{K}_{dt}_{layout}", D, D * Ms, N, K, dt, "normal_sqrtk",
                 True, layout, True, 700 + D + K, rank=rank)
    print(f"case {w.name} {knobs}", flush=True)
    sets = [make_inputs(w, seed=w.seed + i) for i in range(2)]
    devs = [s.to("cuda") for s in sets]
    tun = {k: v for k, v in (("block_m", bm), ("k_per_flag", kpf), ("num_fetch_wgs", nf)) if v}
    refs = [out_bits(run_gpu(w, s, "baseline", dev_inp=d, **tun).out) for s, d in zip(sets, devs)]
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=dt, layout=layout, rank=rank, has_bias=True,
                    fetch_kernel=1, **tun, **knobs)
    cfg = op.config.as_dict()
    assert cfg["fetch_kernel"] == 1 and cfg["row_wait"] == 0
    assert cfg["num_fetch_wgs"] == min(nf or cfg["num_cus"], cfg["num_units"])
    assert cfg["num_wgs"] == min(cfg["num_cus"], cfg["num_items"])
    g = sm.Geometry(w.D, w.M, w.N, w.K, cfg["block_m"], cfg["block_n"], cfg["block_k"],
                    cfg["k_per_flag"], w.rank, True, cfg["num_fetch_wgs"], cfg["num_wgs"],
                    num_cus=cfg["num_cus"])
    outs = [torch.empty((w.M, w.N), dtype=w.torch_dtype(), device="cuda") for _ in range(4)]
    for it in range(4):
        i = it % 2
        op.run(devs[i].shards, devs[i].B, devs[i].bias, out=outs[it])
    assert op.sync_status() == 0
    for it in range(4):
        assert np.array_equal(out_bits(outs[it]), refs[it % 2]), (it, knobs)
    assert np.array_equal(op.flags(), sm.expected_flags(g, 4))
    if not knobs:
        C, _ = oracle_full(w, sets[1])
        assert_close(w, out_bits(outs[3]), C, "fetch_kernel")
    op.close()


def test_fetch_kernel_gather_a():
    """gather_a: the fetch kernel also copies the local shard's units, which no tile waits
    for; the caller's stream still waits for them, so the gathered A is whole when the run's
    stream work ends."""
    import torch
    import all_gather_gemm_amd as A
    import oracle
    w = Workload("fk_gather", 4, 4 * 200, 328, 1032, "bf16", "normal_sqrtk", True,
                 "k_contiguous", True, 777, rank=2)
    inp = make_inputs(w)
    g = inp.to("cuda")
    A_ref = oracle.all_gather([bits(s) for s in inp.shards])
    plain = out_bits(run_gpu(w, inp, "baseline", dev_inp=g).out)
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, rank=w.rank,
                    has_bias=True, gather_a=True, fetch_kernel=1)
    for it in range(2):
        a_out = torch.full((w.M, w.K), float("nan"), dtype=torch.bfloat16, device="cuda")
        a, out = op.run(g.shards, g.B, g.bias, a_out=a_out)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(a).reshape(w.M, w.K), A_ref), it
        assert np.array_equal(out_bits(out), plain), it
    op.close()


def test_fetch_kernel_trace_records_every_unit():
    """debug: the fetch kernel's workgroups write their unit records after the GEMM grid's
    rows of the trace; together they hold each unit of the plan exactly once, and the GEMM
    grid holds every tile exactly once."""
    import torch
    import all_gather_gemm_amd as A
    w = Workload("fk_trace", 4, 4 * 256, 512, 1024, "f16", "normal_sqrtk", False,
                 "m_contiguous", True, 778, rank=1)
    g = make_inputs(w).to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, debug=True, trace_cap=64,
                    fetch_kernel=1, num_fetch_wgs=5, block_m=128, k_per_flag=2)
    op.run(g.shards, g.B, None)
    torch.cuda.synchronize()
    c = op.config
    counts, recs = op.trace()
    assert len(counts) == c.num_wgs + c.num_fetch_wgs
    units = op.units()
    seen_units, seen_tiles = [], []
    for wg in range(len(counts)):
        n = int(counts[wg])
        assert n <= c.trace_cap
        for r in recs[wg, :n]:
            if r["event"] == 1:
                assert wg >= c.num_wgs          # only the fetch kernel fetches
                seen_units.append(int(r["id"]))
                assert (int(r["a"]), int(r["b"])) == tuple(units[int(r["id"])])
            elif r["event"] == 2:
                assert wg < c.num_wgs
                seen_tiles.append(int(r["id"]) & 0xFFFFFF)
    assert sorted(seen_units) == list(range(c.num_units))
    assert sorted(seen_tiles) == list(range(c.num_tiles))
    op.close()


def test_fetch_kernel_timeout_reported():
    """A never-published unit: the GEMM grid's bounded wait gives up, both kernels' workgroups
    exit, sync_status reports TIMEOUT and the handle refuses further runs."""
    import torch
    import all_gather_gemm_amd as A
    w = Workload("fk_skip", 2, 2 * 128, 256, 512, "f16", "uniform", False, "k_contiguous", True,
                 779)
    inp = make_inputs(w).to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, block_m=64, k_per_flag=1, debug_skip_unit=1,
                    spin_limit=2000, fetch_kernel=1)
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    ptrs = [s.data_ptr() for s in inp.shards]
    s = torch.cuda.current_stream().cuda_stream
    assert A.ag_matmul_run(op.handle, ptrs, inp.B.data_ptr(), None, out.data_ptr(), s) == 0
    assert op.sync_status() == -5   # TIMEOUT
    assert A.ag_matmul_run(op.handle, ptrs, inp.B.data_ptr(), None, out.data_ptr(), s) == -7
    torch.cuda.synchronize()
    op.close()


def test_fetch_kernel_on_a_side_stream_and_gather_only():
    """Runs on a caller stream other than the default one: the fetch kernel is ordered after
    the work before each run on that stream and the stream waits for it, so outputs of runs
    alternating two input sets, read after synchronizing that stream alone, match the
    baseline bit for bit. And a gathered-A handle with N = 0 (no output tile: the fetch
    kernel alone writes the gathered A, beside a grid with nothing to compute)."""
    import torch
    import all_gather_gemm_amd as A
    import oracle
    w = Workload("fk_side", 4, 4 * 128, 264, 520, "f16", "normal_sqrtk", True, "m_contiguous",
                 True, 780, rank=3)
    sets = [make_inputs(w, seed=w.seed + i) for i in range(2)]
    devs = [s.to("cuda") for s in sets]
    refs = [out_bits(run_gpu(w, s, "baseline", dev_inp=d, block_m=64).out)
            for s, d in zip(sets, devs)]
    op = A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=True,
                    block_m=64, k_per_flag=2, fetch_kernel=1)
    side = torch.cuda.Stream()
    outs = [torch.empty((w.M, w.N), dtype=torch.float16, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for it in range(4):
            i = it % 2
            op.run(devs[i].shards, devs[i].B, devs[i].bias, out=outs[it])
    side.synchronize()
    for it in range(4):
        assert np.array_equal(out_bits(outs[it]), refs[it % 2]), it
    assert op.sync_status() == 0
    op.close()

    sh = [torch.randn(64, 72, device="cuda").to(torch.bfloat16) for _ in range(2)]
    A_ref = oracle.all_gather([bits(s.cpu()) for s in sh])
    og = A.AgMatmul(2, 128, 0, 72, dtype="bf16", rank=1, gather_a=True, fetch_kernel=1)
    assert og.config.fetch_kernel == 1
    a_out = torch.full((128, 72), float("nan"), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((72, 0), dtype=torch.bfloat16, device="cuda")
    a, _ = og.run(sh, B, None, a_out=a_out)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(a).reshape(128, 72), A_ref)
    og.close()
