"""The device's run count across 2^32, through the C ABI.

A run's epoch is the workspace's run count plus one, kept mod 2^32. Flags grow by one per
run, split counters by the pieces per run, and the per-tile flag variant stores the epoch.
Every comparison with the epoch is an equality, so the counts may wrap: runs whose epochs
pass from 2^32 - 2 through 0 to 3 give the same outputs as the first runs of a fresh handle,
bit for bit, in eager runs and in replays of a captured graph. Afterwards the staged units'
flags are at the wrapped count and the rest stay where they were set.
ag_matmul_debug_set_runs puts a handle's counters where 2^32 - 3 runs would have left them.
"""
import numpy as np
import pytest

from agmm_testlib import out_bits, run_gpu
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

START = (1 << 32) - 3

CASES = [
    # fused, m_contiguous, tail tiles split along K (piece counters), per-k-group waits
    (Workload("wrap_split_m", 2, 2 * 544, 1024, 2048, "f16", "normal_sqrtk", True,
              "m_contiguous", True, 111, rank=1), dict(block_m=64, num_fetch_wgs=8, tail_split=1)),
    # fused, k_contiguous, whole-row waits
    (Workload("wrap_row_k", 8, 8 * 128, 1024, 1024, "bf16", "normal_sqrtk", False,
              "k_contiguous", True, 112, rank=3), dict()),
    # fused with the gathered A (the local shard's units are fetched too)
    (Workload("wrap_gather", 4, 4 * 200, 328, 1032, "bf16", "normal_sqrtk", True,
              "k_contiguous", True, 113, rank=2), dict(gather_a=True, block_m=128)),
    # baseline with split tail tiles
    (Workload("wrap_base", 2, 2 * 544, 1024, 2048, "bf16", "normal_sqrtk", True,
              "k_contiguous", True, 114, rank=0), dict(block_m=64, algo="baseline", tail_split=1)),
]


@pytest.mark.parametrize("w,tun", CASES, ids=[c[0].name for c in CASES])
def test_runs_across_the_wrap(w, tun):
    import torch
    import all_gather_gemm_amd as A
    from oracle import schedule_model as sm
    print(f"case {w.name} {tun}", flush=True)
    tun = dict(tun)
    algo = tun.pop("algo", "fused")
    gather = tun.get("gather_a", False)
    sets = [make_inputs(w, seed=w.seed + i) for i in range(2)]
    devs = [s.to("cuda") for s in sets]
    td = w.torch_dtype()
    a_out = torch.empty((w.M, w.K), dtype=td, device="cuda") if gather else None

    def run(op, d, out):
        if gather:
            op.run(d.shards, d.B, d.bias, out=out, a_out=a_out)
        else:
            op.run(d.shards, d.B, d.bias, out=out)

    # references: the first two runs of a fresh handle
    ref_op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, algo=algo,
                        rank=w.rank, has_bias=w.has_bias, **tun)
    refs = []
    for i in range(2):
        o = torch.empty((w.M, w.N), dtype=td, device="cuda")
        run(ref_op, devs[i], o)
        torch.cuda.synchronize()
        refs.append(out_bits(o))
    ref_op.close()

    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, algo=algo, rank=w.rank,
                    has_bias=w.has_bias, **tun)
    cfg = op.config.as_dict()
    if "tail_split" in tun:
        assert cfg["split_tiles"] > 0
    op.set_runs(START)
    out = torch.empty((w.M, w.N), dtype=td, device="cuda")
    # epochs 2^32 - 2, 2^32 - 1 eagerly; 0 and 1 as replays of a captured run; 2, 3 eagerly
    for it in range(2):
        out.fill_(float("nan"))
        run(op, devs[it % 2], out)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), refs[it % 2]), (w.name, "eager", it)
    dev = sets[0].to("cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(op, dev, out)
    for it in range(2):
        for a, b in zip(dev.shards, devs[it % 2].shards):
            a.copy_(b)
        dev.B.copy_(devs[it % 2].B)
        if dev.bias is not None:
            dev.bias.copy_(devs[it % 2].bias)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), refs[it % 2]), (w.name, "replay", it)
    del g
    for it in range(2):
        out.fill_(float("nan"))
        run(op, devs[it % 2], out)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), refs[it % 2]), (w.name, "eager after", it)
    assert op.sync_status() == 0
    if algo == "fused":
        geo = sm.Geometry(w.D, w.M, w.N, w.K, cfg["block_m"], cfg["block_n"], cfg["block_k"],
                          cfg["k_per_flag"], w.rank, True, cfg["num_fetch_wgs"],
                          cfg["num_wgs"], num_cus=cfg["num_cus"], gather_a=gather)
        prior = np.full(cfg["T_m"] * cfg["G"], START, dtype=np.uint32)
        expect = sm.expected_flags(geo, (START + 6) % (1 << 32), prior)
        assert np.array_equal(op.flags(), expect.astype(np.uint32)), w.name
    op.close()


def test_allreduce_flags_across_the_wrap():
    """The per-tile flag all-reduce stores the epoch in its flags: runs whose epochs pass
    2^32 are bit-identical to a fresh handle's."""
    import torch
    import all_gather_gemm_amd as A
    D, M, N, Kl = 3, 320, 264, 192
    gen = torch.Generator().manual_seed(115)
    Ap = [(torch.randn(M, Kl, generator=gen) / 8).half().cuda() for _ in range(D)]
    Bp = [(torch.randn(Kl, N, generator=gen) / 8).half().cuda() for _ in range(D)]
    h0 = A.GemmAllReduceFlags(D, M, N, Kl, block_m=64)
    ref = out_bits(h0.run(Ap, Bp))
    h0.close()
    h = A.GemmAllReduceFlags(D, M, N, Kl, block_m=64)
    rc = A.ag_matmul_debug_set_runs(h.handle, START, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    for it in range(5):
        o = h.run(Ap, Bp)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(o), ref), it
    h.close()


def test_set_runs_refusals():
    import all_gather_gemm_amd as A
    import torch
    op = A.AgMatmul(2, 256, 256, 256, algo="pipelined")
    assert A.ag_matmul_debug_set_runs(op.handle, 5, 0) == -1
    op.close()
    g = A.GemmAllReduce(2, 0, 128, 128, 128)
    assert A.ag_matmul_debug_set_runs(g.handle, 5, 0) == -1
    g.close()
    assert A.ag_matmul_debug_set_runs(None, 5, 0) == -1
    torch.cuda.synchronize()
