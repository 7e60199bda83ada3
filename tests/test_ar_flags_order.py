"""The claim order of the per-tile flag GEMM + all-reduce (ROCm/iris PR "Let's make Iris'
All-reduce the best!", the one-shot variant with a ready flag per tile), read through the
host-only ag_gemm_ar_flags_plan: every rank's partial tile is computed once, every tile is
reduced once, and each reduction comes after its tile's producers in the order, which is
what guarantees that a workgroup waiting on flags only waits for work already claimed by
workgroups that never wait. A small simulation of a grid claiming the items in order
checks that every run ends, whatever the grid size."""
import heapq

import numpy as np
import pytest

import all_gather_gemm_amd as AG

REDUCE = 1 << 30


def _decode(items):
    red = (items & REDUCE) != 0
    tile = items & 0xFFFFFF
    rank = (items >> 24) & 63
    return red, tile, rank


@pytest.mark.parametrize("D,M,N,K,bm,cus", [
    (1, 256, 256, 64, 0, 256), (2, 2048, 2048, 256, 128, 256), (8, 16384, 3584, 1024, 0, 256),
    (3, 200, 136, 72, 64, 80), (64, 512, 512, 8, 64, 304), (8, 1024, 1024, 128, 0, 256),
    (5, 4096, 1024, 64, 0, 1),
])
def test_order_covers_everything_once_and_reduces_after_producers(D, M, N, K, bm, cus):
    cfg, items = AG.ag_gemm_ar_flags_plan(D, M, N, K, "f16", bm, cus)
    T = cfg["T_m"] * cfg["T_n"]
    assert T == -(-M // cfg["block_m"]) * -(-N // cfg["block_m"])
    assert items.size == T * (D + 1)
    red, tile, rank = _decode(items.astype(np.int64))
    assert (tile < T).all()
    prod_pos = {}
    for i in np.nonzero(~red)[0]:
        key = (int(tile[i]), int(rank[i]))
        assert key not in prod_pos
        prod_pos[key] = int(i)
    assert len(prod_pos) == T * D and (rank[~red] < D).all()
    red_tiles = tile[red]
    assert sorted(red_tiles.tolist()) == list(range(T))
    for i in np.nonzero(red)[0]:
        t = int(tile[i])
        assert all(prod_pos[(t, r)] < i for r in range(D))


def _simulate(items, D, W):
    """W workgroups claim items in order; a producer takes 1 time unit, a reducer waits for
    its tile's D producers to finish and then takes 1. Returns the end time (never None:
    a stuck wait would raise)."""
    red, tile, rank = _decode(items.astype(np.int64))
    done_at = {}            # (tile, rank) -> finish time
    free = [(0.0, w) for w in range(W)]
    heapq.heapify(free)
    end = 0.0
    for i in range(items.size):
        t0, w = heapq.heappop(free)
        if red[i]:
            deps = [done_at.get((int(tile[i]), r)) for r in range(D)]
            assert all(d is not None for d in deps), "a reducer waits on an unclaimed producer"
            t0 = max([t0] + deps)
        else:
            done_at[(int(tile[i]), int(rank[i]))] = t0 + 1
        heapq.heappush(free, (t0 + 1, w))
        end = max(end, t0 + 1)
    return end


@pytest.mark.parametrize("W", [1, 2, 7, 256])
def test_every_grid_size_drains(W):
    D = 4
    cfg, items = AG.ag_gemm_ar_flags_plan(D, 2048, 1024, 64, "bf16", 128, 256)
    end = _simulate(items, D, W)
    T = cfg["T_m"] * cfg["T_n"]
    assert end >= -(-T * (D + 1) // W)   # at least the items per workgroup


def test_plan_refuses_bad_arguments():
    with pytest.raises(AG.AgmmError):
        AG.ag_gemm_ar_flags_plan(0, 256, 256, 64)
    with pytest.raises(AG.AgmmError):
        AG.ag_gemm_ar_flags_plan(65, 256, 256, 64)
    with pytest.raises(AG.AgmmError):
        AG.ag_gemm_ar_flags_plan(2, 256, 260, 64)      # N not a multiple of 8
