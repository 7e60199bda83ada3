"""The host planner (through the host-only ag_matmul_plan_query, no device) against the
bookkeeping model, over random shapes and options: fetch units and their order, GEMM order of
the m-tiles and which are read in place, the tile queues (split pieces included), the split
plan, the pipelined chunk tables, and the fused wait mode. The GPU bookkeeping tests check
that the kernels follow these tables; this checks the tables themselves on many more
shapes than a GPU run can afford."""
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import all_gather_gemm_amd as A
from oracle import schedule_model as sm


@st.composite
def problems(draw):
    D = draw(st.sampled_from([1, 2, 3, 4, 5, 8, 8, 17, 64]))
    Ms = draw(st.integers(0, 700 if D <= 8 else 40))
    M = D * Ms
    N = 8 * draw(st.integers(0, 300))
    K = 8 * draw(st.integers(0, 1200))
    algo = draw(st.sampled_from([A.ALGO_FUSED, A.ALGO_BASELINE, A.ALGO_PIPELINED]))
    gather = draw(st.booleans())
    layout = A.K_CONTIGUOUS if (gather or M % 8) else draw(st.sampled_from([A.K_CONTIGUOUS,
                                                                             A.M_CONTIGUOUS]))
    kw = dict(D=D, M=M, N=N, K=K, rank=draw(st.integers(0, D - 1)),
              direct_local=int(draw(st.booleans())), algo=algo, layout=layout,
              block_m=draw(st.sampled_from([0, 0, 64, 128, 256])),
              k_per_flag=draw(st.sampled_from([0, 0, 1, 3, 8, 16, 40])),
              num_fetch_wgs=draw(st.sampled_from([0, 0, 1, 5, 32, 300])),
              num_wgs=draw(st.sampled_from([0, 0, 7, 100, 300])),
              tail_split=int(draw(st.booleans())), gather_a=int(gather),
              pipeline_chunks=draw(st.sampled_from([0, 1, 2, 3, 4, 8])),
              fetch_kernel=draw(st.sampled_from([0, 0, -1, 1])))
    return kw, draw(st.sampled_from([256, 80, 304]))


@settings(max_examples=250, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(problems())
def test_planner_matches_model(prob):
    kw, cus = prob
    desc = A.ag_matmul_desc_init(**kw)
    r = A.ag_matmul_plan_query(desc, cus)
    c = r["config"]
    g = sm.Geometry(kw["D"], kw["M"], kw["N"], kw["K"], c.block_m, c.block_n, c.block_k,
                    c.k_per_flag, kw["rank"], bool(kw["direct_local"]), c.num_fetch_wgs,
                    c.num_wgs, num_cus=cus, num_wgs_req=kw["num_wgs"],
                    tail_split=kw["tail_split"], gather_a=bool(kw["gather_a"]))
    assert (c.T_m, c.T_n, c.G) == (g.T_m, g.T_n, g.G)
    units = sm.fetch_units(g)
    assert [tuple(map(int, u)) for u in r["units"]] == units
    assert c.num_units == len(units)
    assert [int(x) & 0x7FFFFFFF for x in r["mtiles"]] == sm.mtile_order(g)
    assert [bool(int(x) >> 31) for x in r["mtiles"]] == [sm.is_direct(g, t) for t in sm.mtile_order(g)]
    assert r["queues"] == sm.tile_queues(g)
    assert (c.split_tiles, c.split_pieces) == sm.split_plan(g)[:2]
    # every unit once; every output tile once (whole, or all of its pieces)
    assert len(set(units)) == len(units)
    tiles = {}
    for q in r["queues"]:
        for e in q:
            tiles.setdefault(e & sm.TILE_MASK, []).append((e >> 24) & 15)
    assert sorted(tiles) == list(range(g.T_m * g.T_n))
    for pieces in tiles.values():
        assert sorted(pieces) == list(range(len(pieces)))
    fk = kw["algo"] == A.ALGO_FUSED and c.num_units > 0 and kw["fetch_kernel"] == 1
    assert c.fetch_kernel == int(fk)
    if fk:
        # the fetch kernel's workgroups beside a grid of GEMM workgroups only
        w_base = min(kw["num_wgs"] or cus, cus)
        assert c.num_fetch_wgs == min(kw["num_fetch_wgs"] or cus, c.num_units)
        assert c.num_wgs == max(1, min(w_base, c.num_items))
        assert c.row_wait == 0
    elif kw["algo"] == A.ALGO_FUSED and c.num_units:
        assert c.row_wait == int(c.num_fetch_wgs >= c.num_units)
        assert 1 <= c.num_fetch_wgs <= c.num_wgs
    if kw["algo"] == A.ALGO_PIPELINED:
        S, chunks = sm.pipeline_plan(g, kw["pipeline_chunks"])
        assert c.pipeline_chunks == S and c.pipeline_streams == min(S, 4)
        assert [ch[0] for ch in r["chunks"]] == [ch[0] for ch in chunks]
        assert [[x & 0x7FFFFFFF for x in ch[1]] for ch in r["chunks"]] == [ch[1] for ch in chunks]
    else:
        assert c.pipeline_chunks == 0


def test_plan_query_rejects_bad_requests():
    d = A.ag_matmul_desc_init(D=2, M=256, N=256, K=256)
    buf = (A.ctypes.c_uint8 * 8)()
    assert A.lib.ag_matmul_plan_query(A.ctypes.byref(d), 0, 0, buf, 8) == -1          # no CUs
    assert A.lib.ag_matmul_plan_query(A.ctypes.byref(d), 256, 99, buf, 8) == -1        # what
    assert A.lib.ag_matmul_plan_query(A.ctypes.byref(d), 256, 0, buf, 8) == -1         # size
    bad = A.ag_matmul_desc_init(D=3, M=256, N=256, K=256)                              # M % D
    assert A.lib.ag_matmul_plan_query(A.ctypes.byref(bad), 256, 0, buf, 8) == -1
