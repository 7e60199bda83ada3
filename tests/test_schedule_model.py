"""Pins of the bookkeeping model (oracle/schedule_model.py) on small hand-checked cases
and on invariants that any correct schedule must satisfy: every staged unit fetched
exactly once, every output tile computed exactly once, local-shard m-tiles never staged,
the local shard's m-tiles first in GEMM order, shards visited in rank-rotated order."""
import itertools

import dataclasses

import numpy as np
import pytest

from oracle import schedule_model as sm


def geo(**kw):
    base = dict(D=2, M=4, N=4, K=4, BM=2, BN=2, BK=1, k_per_flag=2, rank=0, direct_local=True,
                F=2, W=4)
    base.update(kw)
    return sm.Geometry(**base)


def test_hand_example_two_shards():
    g = geo()
    assert (g.T_m, g.T_n, g.G) == (2, 2, 2)
    assert [sm.is_direct(g, t) for t in range(2)] == [True, False]
    assert sm.gemm_tiles(g) == [(0, 0), (0, 1), (1, 0), (1, 1)]
    assert sm.fetch_units(g) == [(1, 0), (1, 1)]
    assert list(sm.expected_flags(g, 7)) == [0, 0, 7, 7]


def test_hand_example_gather_a():
    # the op also returns the gathered A: after the staged unit(s), the direct m-tiles'
    # units, k-group by k-group in GEMM order; every m-tile's flags then hold the epoch
    g = geo(gather_a=True)
    assert sm.fetch_units(g) == [(1, 0), (1, 1), (0, 0), (0, 1)]
    assert list(sm.expected_flags(g, 5)) == [5, 5, 5, 5]
    # rank 2 of 4, M_s = 2, BM = 2: own m-tile 2 last
    g2 = geo(D=4, M=8, BM=2, rank=2, N=2, BN=2, W=2, F=1, K=2, k_per_flag=2, gather_a=True)
    assert sm.fetch_units(g2) == [(3, 0), (0, 0), (1, 0), (2, 0)]
    # nothing read in place: gather_a adds no unit
    g3 = geo(direct_local=False)
    assert sm.fetch_units(g3) == sm.fetch_units(dataclasses.replace(g3, gather_a=True))


def test_hand_example_pipeline_chunks():
    # D=2, M_s=8, BM=2, rank 0 in place: 4 chunks of 2 local rows, so chunk i holds m-tile i
    # of shard 0 (in place) and m-tile 4+i of shard 1 (staged, all its k-groups)
    g = geo(M=16, K=4, k_per_flag=2)
    S, ch = sm.pipeline_plan(g, 4)
    assert S == 4
    assert [c[1] for c in ch] == [[0, 4], [1, 5], [2, 6], [3, 7]]
    assert [c[0] for c in ch] == [[(4 + i, 0), (4 + i, 1)] for i in range(4)]
    # 2 chunks: local rows 0..3 and 4..7
    S2, ch2 = sm.pipeline_plan(g, 2)
    assert S2 == 2 and [c[1] for c in ch2] == [[0, 1, 4, 5], [2, 3, 6, 7]]
    # lowered: M_s = 6 is not a multiple of 4 * 2, but of 3 * 2; M_s = 5: one chunk
    assert sm.pipeline_plan(geo(M=12), 4)[0] == 3
    assert sm.pipeline_plan(geo(M=10), 4)[0] == 1
    # every unit and m-tile in exactly one chunk
    for g2 in (g, geo(M=12, rank=1), geo(M=24, D=4, rank=2, direct_local=False)):
        S3, c3 = sm.pipeline_plan(g2, 0)
        assert sorted(u for c in c3 for u in c[0]) == sorted(sm.fetch_units(g2))
        assert sorted(t for c in c3 for t in c[1]) == list(range(g2.T_m))


def test_hand_example_256_row_tile_flags():
    # D=2, M=512, BM=256: m-tile 0 is read in place, m-tile 1 is one unit; after run 3 its
    # flag holds 3 and a prior value elsewhere is kept
    g = sm.Geometry(2, 512, 64, 64, 256, 64, 32, 2, 0, True, 1, 4)
    assert sm.fetch_units(g) == [(1, 0)]
    assert list(sm.expected_flags(g, 3)) == [0, 3]
    assert list(sm.expected_flags(g, 4, np.array([9, 3]))) == [9, 4]


def test_hand_example_rank_rotation_and_straddle():
    # D=2, M_s=3, BM=2: m-tile 1 (rows 2,3) straddles shards 0 and 1
    g = geo(M=6, rank=1, N=2, BN=2)
    assert [sm.owner(g, t) for t in range(3)] == [0, 0, 1]
    assert [sm.is_direct(g, t) for t in range(3)] == [False, False, True]
    # own (direct) m-tile 2 first, then shard rank+1 = 0: m-tiles 0 and 1
    assert sm.mtile_order(g) == [2, 0, 1]
    # W=4, T_n=1 -> window of 4 m-tiles; k-groups outer inside the window
    assert sm.fetch_units(g) == [(0, 0), (1, 0), (0, 1), (1, 1)]


def test_hand_example_four_shards_rank2():
    g = geo(D=4, M=8, BM=2, rank=2, N=2, BN=2, W=2, F=1, K=2, k_per_flag=2)
    # shards: 0 -> t0, 1 -> t1, 2 -> t2 (own), 3 -> t3
    assert sm.mtile_order(g) == [2, 3, 0, 1]
    assert sm.fetch_units(g) == [(3, 0), (0, 0), (1, 0)]   # window of 2: [3, 0], then [1]


def test_hand_example_fetch_windows_follow_the_queues():
    # 12 m-tiles, one column, all staged: super-rows of 4 go to queues 0, 1, 2. With W = 4
    # workgroups draining the queues evenly, the entries in (i, x) order are m-tiles
    # 0, 4, 8, 1 | 5, 9, 2, 6 | 10, 3, 7, 11, four per round. An m-tile's window is its round;
    # inside a window the order is GEMM order (here the m-tile index).
    g = sm.Geometry(D=2, M=24, N=1, K=2, BM=2, BN=1, BK=1, k_per_flag=2, rank=0,
                    direct_local=False, F=2, W=4)
    assert sm.mtile_order(g) == list(range(12))
    assert sm.tile_queues(g)[:3] == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]]
    assert sm.fetch_units(g) == [(t, 0) for t in (0, 1, 4, 8, 2, 5, 6, 9, 3, 7, 10, 11)]
    # two k-groups: a window is fetched k-group by k-group
    g2 = sm.Geometry(D=2, M=24, N=1, K=4, BM=2, BN=1, BK=1, k_per_flag=2, rank=0,
                     direct_local=False, F=2, W=4)
    assert sm.fetch_units(g2)[:8] == [(0, 0), (1, 0), (4, 0), (8, 0), (0, 1), (1, 1), (4, 1), (8, 1)]


def test_direct_local_off_stages_everything():
    g = geo(direct_local=False)
    assert sorted(sm.fetch_units(g)) == [(0, 0), (0, 1), (1, 0), (1, 1)]
    assert sm.staged_rows(g).all()


@pytest.mark.parametrize("D,M,N,K,BM,BN,BK,kpf,rank,dl,F,W", [
    (8, 1024, 1024, 1024, 128, 128, 64, 4, 0, True, 8, 64),
    (4, 4096, 3584, 8192, 256, 256, 64, 16, 3, True, 32, 256),
    (8, 16384, 3584, 8192, 256, 256, 64, 16, 5, True, 32, 256),
    (3, 300, 200, 130, 64, 64, 64, 1, 1, True, 3, 10),        # ragged everything
    (5, 35, 17, 9, 16, 16, 8, 2, 4, False, 2, 3),
    (1, 64, 64, 64, 32, 32, 32, 1, 0, True, 0, 4),             # D=1: nothing staged
])
def test_invariants(D, M, N, K, BM, BN, BK, kpf, rank, dl, F, W):
    g = sm.Geometry(D, M, N, K, BM, BN, BK, kpf, rank, dl, F, W, num_wgs_req=W)
    tiles = sm.gemm_tiles(g)
    assert sorted(tiles) == sorted(itertools.product(range(g.T_m), range(g.T_n)))
    units = sm.fetch_units(g)
    assert len(set(units)) == len(units)
    staged = {t for t in range(g.T_m) if not sm.is_direct(g, t)}
    assert set(units) == set(itertools.product(sorted(staged), range(g.G)))
    # local-shard m-tiles come first in GEMM order
    order = sm.mtile_order(g)
    nd = sum(sm.is_direct(g, t) for t in range(g.T_m))
    assert all(sm.is_direct(g, t) for t in order[:nd])
    # rank-rotated shard order among the rest
    keys = [(sm.owner(g, t) - rank) % D for t in order[nd:]]
    assert keys == sorted(keys)
    # queues partition the tiles; a split tile appears as its pieces, in the tail queue
    check_queues_partition(g)
    # flags: exactly the staged units carry the epoch
    f = sm.expected_flags(g, 5)
    assert int((f == 5).sum()) == len(units) and int((f == 0).sum()) == f.size - len(units)
    # a k-group is fetched no later than the next k-group of the same m-tile
    pos = {u: i for i, u in enumerate(units)}
    for (t, kg), i in pos.items():
        if kg + 1 < g.G:
            assert pos[(t, kg + 1)] > i


def check_queues_partition(g):
    qs = sm.tile_queues(g)
    tail, S, base = sm.split_plan(g)
    T = g.T_m * g.T_n
    order = sm.mtile_order(g)
    split_q = {sm.mtile_order(g).index(c // g.T_n) * g.T_n + c % g.T_n for c in range(base, T)} \
        if S else set()
    regular = list(itertools.chain(*qs[:8]))
    assert all(e >> 24 == 0 for e in regular)
    assert sorted(regular + sorted(split_q)) == list(range(T))
    assert sorted(qs[8]) == sorted(sm.entry(q, i, S) for q in split_q for i in range(S))
    assert len(split_q) == tail
    for q in split_q:  # split tiles are the last ones in t_m * T_n + t_n order
        assert order[q // g.T_n] * g.T_n + q % g.T_n >= T - tail


@pytest.mark.parametrize("T_m, T_n, K, cus, req, ts, exp", [
    (64, 14, 8192, 256, 0, 1, (128, 2, 768)),    # 16384x3584 at 256x256 tiles: 3.5 rounds
    (16, 18, 2048, 256, 0, 1, (32, 4, 256)),     # 288 tiles: 32 left over, 4 pieces of 16 K-tiles
    (16, 18, 1024, 256, 0, 1, (32, 2, 256)),     # only 32 K-tiles: 2 pieces
    (16, 18, 992, 256, 0, 1, (0, 0, 288)),       # 31 K-tiles: pieces would be under 16
    (16, 16, 8192, 256, 0, 1, (0, 0, 256)),      # exactly one round
    (16, 14, 8192, 256, 0, 1, (0, 0, 224)),      # fewer tiles than workgroups
    (24, 16, 8192, 256, 0, 1, (128, 2, 256)),    # last round exactly half full: split in 2
    (35, 11, 8192, 256, 0, 1, (0, 0, 385)),      # 129 left over: more than half, not split
    (24, 15, 8192, 256, 0, 1, (104, 2, 256)),    # 360 tiles: 104 left over
    (16, 18, 2048, 256, 70, 1, (8, 4, 280)),     # 70 workgroups requested: 288 % 70 = 8
    (64, 14, 8192, 256, 0, 0, (0, 0, 896)),      # splitting not asked for (the default)
])
def test_split_plan_hand_examples(T_m, T_n, K, cus, req, ts, exp):
    g = sm.Geometry(1, T_m * 32, T_n * 32, K, 32, 32, 32, 1, 0, True, 0, cus, num_cus=cus,
                    num_wgs_req=req, tail_split=ts)
    assert sm.split_plan(g) == exp
    check_queues_partition(g)


def test_expected_staging_layouts():
    g = geo(D=2, M=4, K=3, BM=2)
    A = np.arange(12, dtype=np.uint16).reshape(4, 3) + 100
    k = sm.expected_staging(g, A, "k_contiguous", 0xFFFF).reshape(4, 3)
    assert (k[:2] == 0xFFFF).all() and (k[2:] == A[2:]).all()
    m = sm.expected_staging(g, A, "m_contiguous", 0xFFFF).reshape(3, 4)
    assert (m[:, :2] == 0xFFFF).all() and (m[:, 2:] == A[2:].T).all()


def test_queue_hand_example():
    # T_m = 6 m-tiles (GEMM positions 0..5), T_n = 10: super-rows {0..3} -> queue 0,
    # {4, 5} -> queue 1; column blocks of 8 then 2 n-tiles
    g = geo(D=1, M=12, N=20, BM=2, BN=2)
    assert (g.T_m, g.T_n) == (6, 10)
    q = sm.tile_queues(g)
    exp0 = [p * 10 + n for p in range(4) for n in range(8)] + \
           [p * 10 + n for p in range(4) for n in range(8, 10)]
    exp1 = [p * 10 + n for p in (4, 5) for n in range(8)] + [p * 10 + n for p in (4, 5) for n in (8, 9)]
    assert q[0] == exp0 and q[1] == exp1 and all(not x for x in q[2:])
    assert len(q) == 9  # eight XCD queues and the (empty) tail queue
