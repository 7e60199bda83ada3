"""Shared helpers for the tests: run the HIP path on seeded inputs and compare with the oracle.

The HIP path is reached only through the C ABI (all_gather_gemm_amd, a ctypes binding of
libagmm.so); the expected values come only from the oracle package.
"""
from __future__ import annotations

import dataclasses
import os
import sys
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import Inputs, Workload, bits, make_inputs  # noqa: E402

NAN16 = {"f16": 0x7E00, "bf16": 0x7FC0}


def agmm():
    """The binding, imported on use so that CPU-only collection never needs the library."""
    import all_gather_gemm_amd
    return all_gather_gemm_amd


@dataclasses.dataclass
class GpuRun:
    out: "object"            # torch tensor on the GPU
    config: dict
    op: "object"             # AgMatmul (closed unless keep=True)


def run_gpu(w: Workload, inp: Inputs, algo: str = "fused", keep: bool = False, dev_inp=None,
            **tunables) -> GpuRun:
    import torch
    A = agmm()
    g = dev_inp if dev_inp is not None else inp.to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, algo=algo, rank=w.rank,
                    direct_local=w.direct_local, has_bias=w.has_bias, **tunables)
    out = op.run(g.shards, g.B, g.bias)
    torch.cuda.synchronize()
    cfg = op.config.as_dict()
    if not keep:
        op.close()
    return GpuRun(out, cfg, op)


def out_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def oracle_full(w: Workload, inp: Inputs):
    sh = [bits(s) for s in inp.shards]
    bias = bits(inp.bias) if inp.bias is not None else None
    C, out16, _ = oracle.agmm(w.dtype, sh, bits(inp.B), bias)
    return C, out16


def sample_points(w: Workload, n: int, seed: int, tile: int = 256):
    """Random (row, col) samples plus every corner of every tile edge that the shape has:
    first/last rows and columns, tile boundaries, shard boundaries."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, w.M, n))
    cols = list(rng.integers(0, w.N, n))
    special_r = {0, w.M - 1}
    for b in range(0, w.M, tile):
        special_r.update({b, min(w.M - 1, b + tile - 1)})
    for d in range(w.D):
        special_r.update({d * w.M_s, min(w.M - 1, (d + 1) * w.M_s - 1)})
    special_c = {0, w.N - 1}
    for b in range(0, w.N, tile):
        special_c.update({b, min(w.N - 1, b + tile - 1)})
    sr = sorted(r for r in special_r if 0 <= r < w.M)
    sc = sorted(c for c in special_c if 0 <= c < w.N)
    for r in sr:
        for c in rng.choice(sc, size=min(len(sc), 8), replace=False):
            rows.append(r)
            cols.append(int(c))
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def oracle_sampled(w: Workload, inp: Inputs, rows, cols) -> np.ndarray:
    sh = [bits(s) for s in inp.shards]
    bias = bits(inp.bias) if inp.bias is not None else None
    return oracle.agmm_at(w.dtype, sh, bits(inp.B), bias, rows, cols)


def assert_close(w: Workload, got_bits: np.ndarray, C: np.ndarray, what: str = ""):
    r = oracle.check(w.dtype, got_bits, C)
    assert r["bad"] == 0, f"{w.name} {what}: {r}"
    return r
