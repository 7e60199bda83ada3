"""GPU bookkeeping, bit for bit against the schedule model (oracle/schedule_model.py):
schedule tables, final flag array, staging contents (staging poisoned with NaN first), the
fetch units (each claimed once, in increasing order per workgroup), every output tile
computed exactly once, every wait seeing the run's epoch. Also: stale-staging races (alternating inputs, poisoned staging), and the
bounded flag wait (a unit whose flag the host never lets the fetcher publish)."""
import itertools

import numpy as np
import pytest

from agmm_testlib import NAN16, oracle_full, out_bits, run_gpu
from oracle import schedule_model as sm
from workloads import Workload, bits, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    Workload("bk_k", 4, 4 * 256, 512, 2048, "f16", "normal_sqrtk", True, "k_contiguous", True, 31,
             rank=2),
    Workload("bk_m", 3, 3 * 200, 264, 1096, "bf16", "normal_sqrtk", False, "m_contiguous", True,
             32, rank=0),
    Workload("bk_off", 2, 2 * 128, 384, 640, "f16", "uniform", False, "k_contiguous", False, 33,
             rank=1),
    # 17 x 16 tiles of 64 with bm=64 (272 > 256 workgroups): the last 16 tiles split along K
    Workload("bk_split", 2, 2 * 544, 1024, 2048, "f16", "normal_sqrtk", True, "m_contiguous",
             True, 34, rank=1),
]


def geometry(w, cfg):
    return sm.Geometry(w.D, w.M, w.N, w.K, cfg["block_m"], cfg["block_n"], cfg["block_k"],
                       cfg["k_per_flag"], w.rank, w.direct_local, cfg["num_fetch_wgs"],
                       cfg["num_wgs"], num_cus=cfg["num_cus"], tail_split=1)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("bm", [64, 128])
@pytest.mark.parametrize("kpf,nf", [(2, 5), (32, 64)], ids=["kloop_waits", "row_waits"])
def test_bookkeeping_matches_model(w, bm, kpf, nf):
    """(2, 5): fetchers take many units each and the K loop waits per k-group; (32, 64): every
    unit has a fetcher of its own and tiles wait for their whole row at their start."""
    import torch
    import all_gather_gemm_amd as A
    print(f"case {w.name} bm={bm} kpf={kpf} fetchers={nf}", flush=True)
    inp = make_inputs(w)
    g_in = inp.to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, rank=w.rank,
                    direct_local=w.direct_local, has_bias=w.has_bias, debug=True, block_m=bm,
                    k_per_flag=kpf, num_fetch_wgs=nf, trace_cap=4096, tail_split=1)
    cfg = op.config.as_dict()
    g = geometry(w, cfg)
    n_units = len(sm.fetch_units(g))
    assert cfg["row_wait"] == int(n_units > 0 and cfg["num_fetch_wgs"] >= n_units)
    if kpf == 32 and n_units:
        assert cfg["row_wait"] == 1
    # tables
    assert [tuple(u) for u in op.units()] == sm.fetch_units(g)
    assert op.queues() == sm.tile_queues(g)
    assert (cfg["split_tiles"], cfg["split_pieces"]) == sm.split_plan(g)[:2]
    if w.name == "bk_split" and bm == 64 and cfg["num_cus"] == 256:
        assert cfg["split_tiles"] == 16
    mt = op.mtiles()
    assert [int(x & 0x7FFFFFFF) for x in mt] == sm.mtile_order(g)
    assert [bool(x >> 31) for x in mt] == [sm.is_direct(g, t) for t in sm.mtile_order(g)]
    C, _ = oracle_full(w, inp)
    A_bits = np.concatenate([bits(s) for s in inp.shards])
    prior = np.zeros(g.T_m * g.G, dtype=np.uint32)
    for epoch in (1, 2, 3):
        op.fill_staging(NAN16[w.dtype])
        out = op.run(g_in.shards, g_in.B, g_in.bias)
        torch.cuda.synchronize()
        import oracle
        r = oracle.check(w.dtype, out_bits(out), C)
        assert r["bad"] == 0, r
        flags = op.flags()
        exp = sm.expected_flags(g, epoch, prior)
        assert np.array_equal(flags, exp)
        prior = flags.copy()
        if cfg["staging_elems"]:
            st = op.staging()
            assert np.array_equal(st, sm.expected_staging(g, A_bits, w.layout, NAN16[w.dtype]))
        counts, recs = op.trace()
        assert (counts <= cfg["trace_cap"]).all()
        fetched = {wg: [] for wg in range(cfg["num_wgs"])}
        units = sm.fetch_units(g)
        tiles = []
        for wg in range(cfg["num_wgs"]):
            for rec in recs[wg, :counts[wg]]:
                if rec["event"] == A.EV_FETCH:
                    u = int(rec["id"])
                    fetched[wg].append(u)
                    assert wg < g.F, "only fetcher workgroups fetch"
                    assert (int(rec["a"]), int(rec["b"])) == units[u]
                elif rec["event"] == A.EV_GEMM:
                    tiles.append(int(rec["id"]))
                    tile = int(rec["id"]) & sm.TILE_MASK
                    assert (int(rec["a"]), int(rec["b"])) == sm.gemm_tiles(g)[tile]
                elif rec["event"] == A.EV_GEMM_WAIT:
                    assert int(rec["a"]) == epoch
                    t_m, kg = divmod(int(rec["id"]), g.G)
                    assert not sm.is_direct(g, t_m)
                else:
                    raise AssertionError(rec)
            # a workgroup takes tiles from each queue in that queue's order
            mine = [int(r["id"]) for r in recs[wg, :counts[wg]] if r["event"] == A.EV_GEMM]
            for qlist in sm.tile_queues(g):
                posn = {t: i for i, t in enumerate(qlist)}
                seq = [posn[t] for t in mine if t in posn]
                assert seq == sorted(seq)
        # every unit fetched exactly once; a workgroup's claims ascend (one counter)
        assert sorted(itertools.chain(*fetched.values())) == list(range(len(units)))
        assert all(v == sorted(v) for v in fetched.values())
        # every queue entry (tile, or piece of a split tile) computed exactly once
        assert sorted(tiles) == sorted(itertools.chain(*sm.tile_queues(g)))
        assert np.array_equal(op.status(), np.zeros(4, dtype=np.uint32))
    op.close()


@pytest.mark.parametrize("algo,layout", [("fused", "m_contiguous"), ("fused", "k_contiguous"),
                                         ("baseline", "k_contiguous")])
def test_debug_run_poisons_staging(algo, layout):
    """A debug run fills the staging buffer with the type's quiet NaN before its kernels
    run: after a run that follows an explicit fill with 1.0, every staging element the run
    does not write holds the NaN, and the staged ones hold A, as the model has them."""
    import torch
    import all_gather_gemm_amd as A
    w = Workload(f"poison_{algo}_{layout}", 4, 4 * 256, 512, 1024, "bf16", "normal_sqrtk",
                 True, layout, True, 36, rank=1)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    g_in = inp.to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=layout, algo=algo, rank=w.rank,
                    has_bias=True, debug=True, block_m=128)
    cfg = op.config.as_dict()
    op.fill_staging(0x3F80)  # bf16 1.0
    out = op.run(g_in.shards, g_in.B, g_in.bias)
    torch.cuda.synchronize()
    C, _ = oracle_full(w, inp)
    import oracle
    assert oracle.check(w.dtype, out_bits(out), C)["bad"] == 0
    st = op.staging()
    A_bits = np.concatenate([bits(s) for s in inp.shards])
    if algo == "fused":
        g = geometry(w, cfg)
        exp = sm.expected_staging(g, A_bits, layout, NAN16[w.dtype])
    else:  # the baseline stages every non-local row, [M][K]
        exp = np.full((w.M, w.K), NAN16[w.dtype], dtype=np.uint16)
        for d in range(w.D):
            if d != w.rank:
                exp[d * w.M_s:(d + 1) * w.M_s] = A_bits.reshape(w.M, w.K)[d * w.M_s:(d + 1) * w.M_s]
        exp = exp.reshape(-1)
    assert np.array_equal(st, exp)
    assert (st == NAN16[w.dtype]).any()   # the local rows are never written
    assert not (st == 0x3F80).any()
    op.close()


def test_alternating_inputs_and_poisoned_staging():
    """Two input sets alternate while staging is re-poisoned each run: a read of stale or
    unwritten staging would show up as a mismatch against the baseline output."""
    import torch
    w = Workload("alt", 8, 8 * 128, 768, 1536, "f16", "normal_sqrtk", True, "m_contiguous", True,
                 41, rank=3)
    sets = [make_inputs(w, seed=s) for s in (41, 42)]
    dev = [s.to("cuda") for s in sets]
    refs = [out_bits(run_gpu(w, s, "baseline", dev_inp=d, block_m=128).out)
            for s, d in zip(sets, dev)]
    assert not np.array_equal(refs[0], refs[1])
    import all_gather_gemm_amd as A
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, rank=w.rank,
                    has_bias=True, block_m=128, k_per_flag=1)
    for it in range(12):
        i = it % 2
        if it % 3 == 0:
            op.fill_staging(NAN16[w.dtype])
        out = op.run(dev[i].shards, dev[i].B, dev[i].bias)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), refs[i]), it
    op.close()


def test_flag_wait_is_bounded():
    """A unit whose flag is never published (set from the host): the waiting workgroup gives
    up after its spin limit, the run reports a timeout, every workgroup exits, and the
    handle refuses further runs."""
    import torch
    import all_gather_gemm_amd as A
    w = Workload("skip", 2, 2 * 128, 256, 512, "f16", "uniform", False, "k_contiguous", True, 51)
    inp = make_inputs(w).to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, debug=True, block_m=64, k_per_flag=1,
                    debug_skip_unit=1, spin_limit=2000)
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    rc = A.ag_matmul_run(op.handle, [s.data_ptr() for s in inp.shards], inp.B.data_ptr(), None,
                         out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == -5  # TIMEOUT
    st = op.status()
    assert st[0] == 1
    u = op.units()[1]
    assert st[2] == u[0] * op.config.G + u[1]      # the flag of the skipped unit
    assert st[3] != 1                               # the run's epoch was 1
    rc2 = A.ag_matmul_run(op.handle, [s.data_ptr() for s in inp.shards], inp.B.data_ptr(), None,
                          out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc2 == -7  # POISONED
    torch.cuda.synchronize()
    op.close()


def test_flag_wait_timeout_reported_without_debug():
    """The same never-published unit with debug off: run() returns at once (AGMM_OK, nothing
    synchronized), the kernel's bounded wait gives up and every workgroup exits; the launch's
    last workgroup copies the status to the handle's host word, so ag_matmul_sync_status
    (or, without it, the next run) reports TIMEOUT and later calls POISONED. A handle
    without the skipped unit reports nothing."""
    import torch
    import all_gather_gemm_amd as A
    w = Workload("skip_nodebug", 2, 2 * 128, 256, 512, "f16", "uniform", False, "k_contiguous",
                 True, 52)
    inp = make_inputs(w).to("cuda")
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    ptrs = [t.data_ptr() for t in inp.shards]

    def run(op):
        return A.ag_matmul_run(op.handle, ptrs, inp.B.data_ptr(), None, out.data_ptr(), s)

    kw = dict(block_m=64, k_per_flag=1, spin_limit=2000)
    for algo in ("fused",):
        op = A.AgMatmul(w.D, w.M, w.N, w.K, algo=algo, debug_skip_unit=1, **kw)
        assert run(op) == 0
        assert op.sync_status() == -5          # TIMEOUT
        st = op.status()
        assert st[0] == 1
        u = op.units()[1]
        assert st[2] == u[0] * op.config.G + u[1]
        assert run(op) == -7                   # POISONED
        assert op.sync_status() == -7
        op.close()
        # no sync call: the next run finds the host word set
        op = A.AgMatmul(w.D, w.M, w.N, w.K, algo=algo, debug_skip_unit=1, **kw)
        assert run(op) == 0
        torch.cuda.synchronize()
        assert run(op) == -5
        assert run(op) == -7
        op.close()
    good = A.AgMatmul(w.D, w.M, w.N, w.K, **kw)
    for _ in range(3):
        assert run(good) == 0
    assert good.sync_status() == 0
    good.close()


def test_caller_workspace():
    """A handle created on caller-owned device memory (ag_matmul_workspace_bytes of it)
    computes the same output, bit for bit, as one whose workspace the library allocates; a
    misaligned or too small workspace is refused."""
    import torch
    import all_gather_gemm_amd as A
    w = Workload("ws", 4, 4 * 192, 520, 776, "f16", "normal_sqrtk", True, "m_contiguous", True,
                 53, rank=2)
    inp = make_inputs(w).to("cuda")
    ref = A.AgMatmul(w.D, w.M, w.N, w.K, layout=w.layout, rank=w.rank, has_bias=True)
    want = out_bits(ref.run(inp.shards, inp.B, inp.bias))
    ref.close()
    desc = A.ag_matmul_desc_init(D=w.D, M=w.M, N=w.N, K=w.K, rank=w.rank, has_bias=1,
                                 layout=A.M_CONTIGUOUS)
    nbytes = A.ag_matmul_workspace_bytes(desc)
    assert nbytes > 0
    ws = torch.empty(nbytes + 512, dtype=torch.uint8, device="cuda")
    base = (ws.data_ptr() + 255) // 256 * 256
    for bad_ptr, bad_n in ((base + 16, nbytes), (base, nbytes - 256)):
        with pytest.raises(A.AgmmError) as e:
            A.ag_matmul_create(desc, bad_ptr, bad_n)
        assert e.value.code == -1
    h = A.ag_matmul_create(desc, base, nbytes)
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    for _ in range(2):
        out.fill_(float("nan"))
        rc = A.ag_matmul_run(h, [t.data_ptr() for t in inp.shards], inp.B.data_ptr(),
                             inp.bias.data_ptr(), out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), want)
    A.ag_matmul_destroy(h)


@pytest.mark.parametrize("w", CASES[:3], ids=lambda w: w.name)
@pytest.mark.parametrize("kpf,nf", [(2, 5), (32, 64)], ids=["kloop_waits", "row_waits"])
def test_gather_a_bookkeeping(w, kpf, nf):
    """The op that also returns the gathered A: the caller's [M, K] buffer (poisoned with NaN
    before each run) is the staging buffer; the fetch also copies the local shard's m-tiles,
    after every staged one. Unit table, flags and trace against the model; the gathered A
    bit for bit against the oracle's all_gather."""
    import torch
    import all_gather_gemm_amd as A
    import oracle
    if w.layout != "k_contiguous":
        w = w.with_(layout="k_contiguous")
    print(f"case gather {w.name} kpf={kpf} fetchers={nf}", flush=True)
    inp = make_inputs(w)
    g_in = inp.to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, rank=w.rank,
                    direct_local=w.direct_local, has_bias=w.has_bias, debug=True, block_m=64,
                    k_per_flag=kpf, num_fetch_wgs=nf, trace_cap=4096, gather_a=True)
    cfg = op.config.as_dict()
    assert cfg["staging_elems"] == 0
    g = sm.Geometry(w.D, w.M, w.N, w.K, cfg["block_m"], cfg["block_n"], cfg["block_k"],
                    cfg["k_per_flag"], w.rank, w.direct_local, cfg["num_fetch_wgs"],
                    cfg["num_wgs"], num_cus=cfg["num_cus"], gather_a=True)
    units = sm.fetch_units(g)
    assert [tuple(u) for u in op.units()] == units
    assert sorted(set(t for t, _ in units)) == list(range(g.T_m))   # every m-tile fetched
    A_ref = oracle.all_gather([bits(s) for s in inp.shards])
    C, _ = oracle_full(w, inp)
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    a_out = torch.empty((w.M, w.K), dtype=tdt, device="cuda")
    prior = np.zeros(g.T_m * g.G, dtype=np.uint32)
    for epoch in (1, 2):
        a_out.view(torch.int16).fill_(int(np.array(NAN16[w.dtype], np.uint16).view(np.int16)))
        a, out = op.run(g_in.shards, g_in.B, g_in.bias, a_out=a_out)
        torch.cuda.synchronize()
        assert a.data_ptr() == a_out.data_ptr()
        assert np.array_equal(out_bits(a).reshape(w.M, w.K), A_ref)
        r = oracle.check(w.dtype, out_bits(out), C)
        assert r["bad"] == 0, r
        flags = op.flags()
        assert np.array_equal(flags, sm.expected_flags(g, epoch, prior))
        prior = flags.copy()
        counts, recs = op.trace()
        fetched = []
        for wg in range(cfg["num_wgs"]):
            for rec in recs[wg, :counts[wg]]:
                if rec["event"] == A.EV_FETCH:
                    assert wg < g.F
                    fetched.append(int(rec["id"]))
                    assert (int(rec["a"]), int(rec["b"])) == units[int(rec["id"])]
                elif rec["event"] == A.EV_GEMM_WAIT:
                    assert not sm.is_direct(g, int(rec["id"]) // g.G)   # nobody waits on own tiles
        assert sorted(fetched) == list(range(len(units)))
        assert np.array_equal(op.status(), np.zeros(4, dtype=np.uint32))
    op.close()
