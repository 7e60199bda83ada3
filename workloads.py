"""Seeded synthetic workloads for the fused all-gather + GEMM.

This module is shared by the GPU path's tests/bench and by the oracle's tests. It holds
only workload definitions and random-number generation: no part of the contraction, the
gather or any rounding beyond the one cast of freshly drawn fp32 values to the 16-bit
storage type.

Shapes follow the pages' workloads: the iris fused all-gather+GEMM results (ROCm/iris
issue "Fused all-gather+GEMM HBM-buffer kernel for iris.ops", "Results" tables:
fp16, N=3584, K=8192, M in {1024, 4096, 16384}, 2/4/8 ranks) and the bf16 cube sweep
of the Helion all-gather matmul benchmark (pytorch/helion PR "[Benchmark] Add all gather
matmul benchmark", shape table, cubes 256..4096).

Recipe (fixed order, CPU ``torch.Generator`` seeded with the workload's seed):
  1. the full gathered A [M, K] drawn in fp32, then cast to the storage type (RNE);
  2. B [K, N] drawn the same way;
  3. bias [N] (only when the workload has one), uniform[-1, 1] in fp32, cast.
A is then cut into D equal row blocks; block d holds global rows [d*M/D, (d+1)*M/D)
(the row order that the Helion thread's local-tile index formula implies). Each block
is a separate tensor, and on the GPU a separate allocation.

Distributions:
  "normal_sqrtk":  randn / sqrt(K)
  "uniform":       rand * 2 - 1
  "uniform_sqrtk": (rand * 2 - 1) / sqrt(K)
  "int":           integers drawn uniformly from {-2, ..., 2} (exact-integer variant)
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

F16 = "f16"
BF16 = "bf16"
K_CONTIGUOUS = "k_contiguous"
M_CONTIGUOUS = "m_contiguous"

_TORCH_DTYPE = {F16: torch.float16, BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    D: int
    M: int
    N: int
    K: int
    dtype: str            # "f16" | "bf16": inputs, bias and output share it
    dist: str             # see module docstring
    has_bias: bool
    layout: str           # staging layout
    direct_local: bool    # own-shard tiles read in place
    seed: int
    rank: int = 0

    @property
    def M_s(self) -> int:
        return self.M // self.D

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, smallest first. The large one (16384x3584x8192 fp16, D=8,
# m_contiguous staging, fp16 bias) is the headline throughput case.
TINY = Workload("tiny_256_d2_bf16", 2, 256, 256, 256, BF16, "uniform", False, K_CONTIGUOUS, True, 1)
SQUARE_1024 = Workload("square_1024_d8_bf16", 8, 1024, 1024, 1024, BF16, "normal_sqrtk", False,
                       K_CONTIGUOUS, True, 2)
MID_4096 = Workload("ag_4096x3584x8192_d4_f16", 4, 4096, 3584, 8192, F16, "normal_sqrtk", False,
                    K_CONTIGUOUS, True, 3)
LARGE_16384 = Workload("ag_16384x3584x8192_d8_f16_bias", 8, 16384, 3584, 8192, F16, "normal_sqrtk",
                       True, M_CONTIGUOUS, True, 4)
SQUARE_4096 = Workload("square_4096_d8_bf16", 8, 4096, 4096, 4096, BF16, "uniform_sqrtk", False,
                       K_CONTIGUOUS, True, 5)

WORKLOADS: List[Workload] = [TINY, SQUARE_1024, MID_4096, LARGE_16384, SQUARE_4096]
BY_NAME = {w.name: w for w in WORKLOADS}


def _draw(gen: torch.Generator, shape, dist: str, K: int) -> torch.Tensor:
    if dist == "normal_sqrtk":
        return torch.randn(shape, generator=gen, dtype=torch.float32) / math.sqrt(K)
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2 - 1
    if dist == "uniform_sqrtk":
        return (torch.rand(shape, generator=gen, dtype=torch.float32) * 2 - 1) / math.sqrt(K)
    if dist == "int":
        return torch.randint(-2, 3, shape, generator=gen).to(torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


@dataclasses.dataclass
class Inputs:
    shards: List[torch.Tensor]     # D tensors [M_s, K], CPU, storage dtype
    B: torch.Tensor                # [K, N]
    bias: Optional[torch.Tensor]   # [N] or None

    def to(self, device) -> "Inputs":
        # one separate allocation per shard
        return Inputs([s.to(device).contiguous().clone() for s in self.shards],
                      self.B.to(device).contiguous(),
                      None if self.bias is None else self.bias.to(device).contiguous())


def make_inputs(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw the workload's tensors on the CPU, in the recipe's fixed order."""
    if w.M % w.D != 0:
        raise ValueError("M must be a multiple of D")
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    td = w.torch_dtype()
    A = _draw(gen, (w.M, w.K), w.dist, w.K).to(td)
    B = _draw(gen, (w.K, w.N), w.dist, w.K).to(td)
    bias = None
    if w.has_bias:
        bdist = "int" if w.dist == "int" else "uniform"
        bias = _draw(gen, (w.N,), bdist, w.K).to(td)
    ms = w.M // w.D
    shards = [A[d * ms:(d + 1) * ms].clone().contiguous() for d in range(w.D)]
    return Inputs(shards, B.contiguous(), bias)


def bits(t: torch.Tensor):
    """Raw 16-bit patterns of a CPU tensor as a numpy uint16 array (a view, no conversion)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")
