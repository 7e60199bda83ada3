"""The largest shapes the library accepts, through the C ABI.

create takes M < 2^23 and N, K < 2^22. The kernels address a tile through 32-bit buffer
offsets from a per-tile base:
- a K-major operand or output tile spans 256 rows of a K- or N-element stride, just under
  2^31 bytes at the maximum;
- the m_contiguous staging spans 32 rows of an M-element stride per K-tile.

Each case sits at one of these limits, with shards whose rows do not fill whole tiles, so
fetch units cross shard boundaries and take the copy's per-row path. The inputs are small
integers, so every partial sum is exact in fp32, and the outputs of both algorithms must
equal the fp64 oracle's RNE-rounded ones bit for bit. A dropped or repeated K block, a wrong
row or a wrapped offset would change them.
"""
import numpy as np
import pytest

from agmm_testlib import oracle_full, out_bits, run_gpu
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

K_MAX = (1 << 22) - 8
N_MAX = (1 << 22) - 8
M_MAX = (1 << 23) - 64   # a multiple of 8 shards of 8-row multiples

CASES = [
    # K at its limit with 256-row tiles: a K-major tile spans 2^31 - 4096 bytes
    (Workload("max_k", 2, 256, 64, K_MAX, "f16", "int", True, "k_contiguous", True, 91, rank=1),
     dict(block_m=256)),
    (Workload("max_k_m", 2, 256, 64, K_MAX, "bf16", "int", False, "m_contiguous", True, 92,
              rank=0), dict(block_m=256)),
    # N at its limit: B and output rows of 8 MiB, an output tile spans 2^31 - 4096 bytes
    (Workload("max_n", 2, 256, N_MAX, 64, "bf16", "int", True, "m_contiguous", True, 93, rank=1),
     dict(block_m=256)),
    # M at its limit: m_contiguous staging rows of 16 MiB, shards of 1048568 rows
    (Workload("max_m", 8, M_MAX, 64, 32, "f16", "int", True, "m_contiguous", True, 94, rank=3),
     dict()),
    (Workload("max_m_k", 8, M_MAX, 16, 64, "bf16", "int", False, "k_contiguous", True, 95,
              rank=6), dict(block_m=256)),
]


@pytest.mark.parametrize("w,tun", CASES, ids=[c[0].name for c in CASES])
def test_max_size_bit_exact(w, tun):
    print(f"case {w.name} M={w.M} N={w.N} K={w.K} {tun}", flush=True)
    inp = make_inputs(w)
    dev = inp.to("cuda")
    _, out16 = oracle_full(w, inp)
    for algo in ("fused", "baseline"):
        r = run_gpu(w, inp, algo, dev_inp=dev, **tun)
        got = out_bits(r.out).reshape(w.M, w.N)
        bad = int((got != out16.reshape(w.M, w.N)).sum())
        assert bad == 0, (w.name, algo, bad, r.config)
        print(f"  {algo}: bit-exact, {r.config['num_tiles']} tiles, block_m "
              f"{r.config['block_m']}", flush=True)
