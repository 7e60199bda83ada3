"""Bookkeeping model of the fused all-gather + GEMM (TEST INFRASTRUCTURE ONLY).

The method (ROCm/iris issue "Fused all-gather+GEMM HBM-buffer kernel for iris.ops",
opening summary): workgroups split into fetchers and GEMM workers; fetchers copy A tiles
into a local staging buffer and set one ready flag per tile; GEMM workers wait on those
flags and compute as tiles arrive. Tiles of the local shard are read in place and never
staged (pytorch/helion PR "[Benchmark] Add all gather matmul benchmark", the Kraken
optimization comment). Flag granularity is one flag per (m-tile, group of k_per_flag
K-tiles), after the k_per_flag tunable in the iris issue's defaults table.

This module restates, independently of the GPU library, the static schedule that the GPU
library documents, so that its debug logs, flag array and staging buffer can be checked
bit for bit:

  T_m = ceil(M/BM), T_n = ceil(N/BN), KG = k_per_flag*BK, G = ceil(K/KG)
  owner(t)   = (t*BM) // M_s                         shard of the m-tile's first row
  direct(t)  = direct_local and the whole m-tile lies inside shard `rank`
  S          = direct m-tiles ascending, then the others by ((owner - rank) mod D, t)
  tile q     = (S[q // T_n], q % T_n)                GEMM order, n fastest
  staged S'  = [t in S if not direct(t)]
  units      = staged m-tiles grouped by the round in which the queues first reach them
               (entries in (i, x) order, the k-th in round k // W); window by window, GEMM
               order inside a window: for g in 0..G-1: for t in window: (t, g); with
               gather_a (the op also returns a = all_gather(a_shared), Kraken comment), then
               the direct m-tiles: for g in 0..G-1: for t in direct, GEMM order: (t, g)
  claims     = fetchers take units in increasing u from one counter (so the units of one
               workgroup ascend); every unit is claimed exactly once
  queues     = GEMM-order m-tiles in super-rows of 4; a super-row's tiles listed in column
               blocks of 8 n-tiles (m-tile, then n, inside a block); super-row j appended
               to queue j mod 8 (one queue per XCD); every tile in exactly one queue
  flags[t*G + g] == epoch after a run (each run adds 1), for every staged unit; direct
               units untouched
  staging, k_contiguous:  S[m*K + k] = A[m][k];  m_contiguous: S[k*M + m] = A[m][k]
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Geometry:
    D: int
    M: int
    N: int
    K: int
    BM: int
    BN: int
    BK: int
    k_per_flag: int
    rank: int
    direct_local: bool
    F: int          # fetcher workgroups (may be 0 when nothing is staged)
    W: int          # workgroups in the grid (fetchers included)
    num_cus: int = 256      # compute units of the device
    num_wgs_req: int = 0    # requested grid size (0 = one workgroup per compute unit)
    tail_split: int = 0     # 1 = split the tail tiles along K (0: never)
    gather_a: bool = False  # the run also returns the gathered A: direct m-tiles fetched too

    @property
    def M_s(self) -> int:
        return self.M // self.D

    @property
    def T_m(self) -> int:
        return -(-self.M // self.BM)

    @property
    def T_n(self) -> int:
        return -(-self.N // self.BN)

    @property
    def KG(self) -> int:
        return self.k_per_flag * self.BK

    @property
    def G(self) -> int:
        return -(-self.K // self.KG) if self.K > 0 else 0


def owner(g: Geometry, t: int) -> int:
    return (t * g.BM) // g.M_s


def is_direct(g: Geometry, t: int) -> bool:
    if not g.direct_local:
        return False
    lo = t * g.BM
    hi = min(g.M, (t + 1) * g.BM)
    return g.rank * g.M_s <= lo and hi <= (g.rank + 1) * g.M_s


def mtile_order(g: Geometry) -> List[int]:
    direct = [t for t in range(g.T_m) if is_direct(g, t)]
    other = [t for t in range(g.T_m) if not is_direct(g, t)]
    other.sort(key=lambda t: ((owner(g, t) - g.rank) % g.D, t))
    return direct + other


def gemm_tiles(g: Geometry) -> List[Tuple[int, int]]:
    """Tile q -> (t_m, t_n) in GEMM order."""
    return [(t, n) for t in mtile_order(g) for n in range(g.T_n)]


N_QUEUES, SUPER_ROWS, COL_BLOCK = 8, 4, 8
MAX_SPLIT = 4
TILE_MASK = 0xFFFFFF


def split_plan(g: Geometry) -> Tuple[int, int, int]:
    """(split tiles, pieces per split tile, first split tile t_m * T_n + t_n).

    Only when splitting is asked for (tail_split = 1). With Wg GEMM workgroups a last round holds num_tiles % Wg tiles; when that is at most
    half of Wg (and there is at least one full round), those tiles -- the last ones in
    t_m * T_n + t_n order -- are cut along K into S = min(4, Wg // tail, K-tiles // 16)
    pieces, S >= 2; otherwise nothing is split."""
    T = g.T_m * g.T_n
    w_base = min(g.num_wgs_req or g.num_cus, g.num_cus)
    wg = min(w_base, T)
    kt = -(-g.K // g.BK)
    if not g.tail_split or wg <= 0 or T <= wg or T > TILE_MASK:
        return 0, 0, T
    tail = T % wg
    if tail == 0:
        return 0, 0, T
    S = min(MAX_SPLIT, wg // tail, kt // 16)
    if S < 2:
        return 0, 0, T
    return tail, S, T - tail


def entry(tile: int, piece: int = 0, pieces: int = 1) -> int:
    return tile | (piece << 24) | ((pieces - 1) << 28)


def tile_queues(g: Geometry) -> List[List[int]]:
    """The 8 per-XCD queues and the tail queue, as lists of entries (tile id q = GEMM
    position * T_n + n, plus piece and piece count for split tiles)."""
    tail, S, base = split_plan(g)
    order = mtile_order(g)
    pos_of = {t: i for i, t in enumerate(order)}
    queues = [[] for _ in range(N_QUEUES + 1)]
    for j, s0 in enumerate(range(0, g.T_m, SUPER_ROWS)):
        rows = range(s0, min(g.T_m, s0 + SUPER_ROWS))
        for nb in range(0, g.T_n, COL_BLOCK):
            for pos in rows:
                for n in range(nb, min(g.T_n, nb + COL_BLOCK)):
                    if S and order[pos] * g.T_n + n >= base:
                        continue
                    queues[j % N_QUEUES].append(pos * g.T_n + n)
    for c in range(base, g.T_m * g.T_n if S else base):
        q = pos_of[c // g.T_n] * g.T_n + c % g.T_n
        for piece in range(S):
            queues[N_QUEUES].append(entry(q, piece, S))
    return queues


def fetch_units(g: Geometry) -> List[Tuple[int, int]]:
    """Unit u -> (t_m, k-group) in fetch order.

    The W workgroups are taken to drain the 8 per-XCD queues evenly: list the entries in the
    order (i, x) (entry i of queue x, only those that exist); the k-th is reached in round
    k // W. An m-tile's window is the earliest round over its entries (an m-tile whose tiles
    are all split pieces comes after every round). Staged m-tiles go window by window, in
    GEMM order inside a window, and a window is fetched k-group by k-group."""
    order = mtile_order(g)
    queues = tile_queues(g)[:N_QUEUES]
    first = [float("inf")] * g.T_m
    interleaved = sorted((i, x) for x in range(N_QUEUES) for i in range(len(queues[x])))
    for k, (i, x) in enumerate(interleaved):
        pos = (queues[x][i] & TILE_MASK) // g.T_n
        first[pos] = min(first[pos], k // max(1, g.W))
    staged = sorted((first[pos], pos) for pos in range(g.T_m) if not is_direct(g, order[pos]))
    units = []
    i = 0
    while i < len(staged):
        j = i
        while j < len(staged) and staged[j][0] == staged[i][0]:
            j += 1
        for kg in range(g.G):
            for _, pos in staged[i:j]:
                units.append((order[pos], kg))
        i = j
    if g.gather_a:
        direct = [t for t in order if is_direct(g, t)]
        for kg in range(g.G):
            for t in direct:
                units.append((t, kg))
    return units


def pipeline_plan(g: Geometry, chunks_requested: int = 0):
    """The host stream pipeline (NVIDIA/Fuser PR #3695's AG+GEMM host program): A's rows cut
    into S chunks along each shard, chunk i = local rows [i*M_s/S, (i+1)*M_s/S) of every
    shard. S is the request (default 4) lowered until M_s is a multiple of S*BM, so that
    every m-tile lies in one chunk (1 when M_s is not a multiple of BM). Returns (S,
    [(units of chunk i in fetch order, m-tiles of chunk i in GEMM order)])."""
    S = chunks_requested or 4
    if g.M_s == 0 or g.M_s % g.BM:
        S = 1
    while S > 1 and g.M_s % (S * g.BM):
        S -= 1
    rows = g.M_s // S if S > 1 else 1

    def chunk(t):
        return 0 if S == 1 else ((t * g.BM) % g.M_s) // rows
    units, order = fetch_units(g), mtile_order(g)
    return S, [([u for u in units if chunk(u[0]) == i], [t for t in order if chunk(t) == i])
               for i in range(S)]


def expected_flags(g: Geometry, epoch: int, prior: np.ndarray = None) -> np.ndarray:
    """Flag array [T_m * G] after a run with the given epoch."""
    size = g.T_m * g.G
    flags = np.zeros(size, dtype=np.uint32) if prior is None else prior.astype(np.uint32).copy()
    for (t, kg) in fetch_units(g):
        flags[t * g.G + kg] = epoch
    return flags


def staged_rows(g: Geometry) -> np.ndarray:
    """Boolean mask over the M rows of A: True where the row is staged."""
    mask = np.zeros(g.M, dtype=bool)
    for t in range(g.T_m):
        if not is_direct(g, t):
            mask[t * g.BM:min(g.M, (t + 1) * g.BM)] = True
    return mask


def expected_staging(g: Geometry, A_bits: np.ndarray, layout: str, poison: int) -> np.ndarray:
    """Staging buffer contents (uint16) after a run that started from `poison` everywhere."""
    assert A_bits.shape == (g.M, g.K)
    mask = staged_rows(g)
    if layout == "k_contiguous":
        st = np.full((g.M, g.K), poison, dtype=np.uint16)
        st[mask, :] = A_bits[mask, :]
        return st.reshape(-1)
    if layout == "m_contiguous":
        st = np.full((g.K, g.M), poison, dtype=np.uint16)
        st[:, mask] = A_bits[mask, :].T
        return st.reshape(-1)
    raise ValueError(layout)
