"""GPU parity of the GEMM + all-reduce share (atomics), through the C ABI.

Every rank's share runs on this GPU, one after another on one stream (and, in one test, on
two streams at once), adding into the D fp32 result buffers. Reference: the oracle's fp64
sum over ranks. Bound (the pages give none; from the arithmetic): the products of 16-bit
values are exact in fp32, a rank's K_local-term fp32 sum errs by at most K_local u S and the
D additions by at most D u S, with u = 2^-24 and S = |A| @ |B| (computed by the oracle from
the absolute values), so |C_gpu - C| <= (K_local + D + 2) u S. The finalized 16-bit output
is held to the op's usual tolerance. Ranks run in order add to every buffer in the same
order, so the D buffers agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from agmm_testlib import out_bits

pytestmark = pytest.mark.gpu

CASES = [
    # (D, M, N, K_local, dtype, block_m)
    (1, 256, 256, 256, "f16", 0),
    (2, 520, 264, 1032, "bf16", 128),
    (4, 384, 392, 200, "f16", 64),
    (8, 1024, 1024, 128, "bf16", 0),
    (3, 200, 136, 72, "f16", 256),
    (2, 130, 72, 0, "bf16", 0),      # K_local = 0: the result is zero (+ bias)
]


def _parts(D, M, N, Kl, dt, seed):
    g = torch.Generator().manual_seed(seed)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    K = max(D * Kl, 1)
    A = [(torch.randn(M, Kl, generator=g) / K ** 0.5).to(tdt) for _ in range(D)]
    B = [(torch.randn(Kl, N, generator=g) / K ** 0.5).to(tdt) for _ in range(D)]
    bias = torch.rand(N, generator=g).mul(2).sub(1).to(tdt)
    return A, B, bias


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _reference(D, dt, A, B):
    C, _, _ = oracle.gemm_allreduce(dt, [_bits(a) for a in A], [_bits(b) for b in B])
    S, _, _ = oracle.gemm_allreduce(dt, [_bits(a) & 0x7FFF for a in A], [_bits(b) & 0x7FFF for b in B])
    return C, S


@pytest.mark.parametrize("D,M,N,Kl,dt,bm", CASES)
def test_allreduce_shares_match_oracle(D, M, N, Kl, dt, bm):
    import all_gather_gemm_amd as AG
    print(f"case ar D={D} {M}x{N}x{Kl} {dt} bm={bm}", flush=True)
    A, B, bias = _parts(D, M, N, Kl, dt, 500 + D)
    Ad, Bd = [a.cuda() for a in A], [b.cuda() for b in B]
    C = [torch.zeros((M, N), dtype=torch.float32, device="cuda") for _ in range(D)]
    hs = [AG.GemmAllReduce(D, r, M, N, Kl, dt, bm) for r in range(D)]
    for r in range(D):
        hs[r].run(Ad[r], Bd[r], C)
    torch.cuda.synchronize()
    Cref, S = _reference(D, dt, A, B)
    bound = (Kl + D + 2) * 2.0 ** -24 * S
    got = [c.cpu().numpy().astype(np.float64) for c in C]
    for r in range(D):
        err = np.abs(got[r] - Cref)
        assert (err <= bound).all(), (r, float((err - bound).max()))
        assert np.array_equal(got[r], got[0])
    out = hs[0].finalize(C[0], bias.cuda())
    torch.cuda.synchronize()
    bdec = oracle.decode(dt, _bits(bias))
    r = oracle.check(dt, out_bits(out), Cref + bdec[None, :])
    assert r["bad"] == 0, r
    for h in hs:
        h.close()


def test_allreduce_concurrent_shares():
    """Two ranks' shares on two streams at once: the atomic additions interleave, the result
    stays within the bound (the two buffers may differ in their last bits)."""
    import all_gather_gemm_amd as AG
    D, M, N, Kl, dt = 2, 512, 384, 512, "f16"
    A, B, _ = _parts(D, M, N, Kl, dt, 77)
    Ad, Bd = [a.cuda() for a in A], [b.cuda() for b in B]
    C = [torch.zeros((M, N), dtype=torch.float32, device="cuda") for _ in range(D)]
    hs = [AG.GemmAllReduce(D, r, M, N, Kl, dt) for r in range(D)]
    streams = [torch.cuda.Stream() for _ in range(D)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for r in range(D):
        hs[r].run(Ad[r], Bd[r], C, stream=streams[r])
    torch.cuda.synchronize()
    Cref, S = _reference(D, dt, A, B)
    bound = (Kl + D + 2) * 2.0 ** -24 * S
    for c in C:
        assert (np.abs(c.cpu().numpy().astype(np.float64) - Cref) <= bound).all()
    for h in hs:
        h.close()


def test_allreduce_empty_output():
    """M = 0: nothing to add and nothing to round; both calls succeed and launch nothing."""
    import all_gather_gemm_amd as AG
    g = AG.GemmAllReduce(2, 1, 0, 64, 64)
    A = torch.zeros((1, 64), dtype=torch.float16, device="cuda")
    C = [torch.zeros((1, 64), dtype=torch.float32, device="cuda") for _ in range(2)]
    assert g.run(A, A, C) == 0
    out = torch.full((1, 64), 7.0, dtype=torch.float16, device="cuda")
    assert g.finalize(C[0], None, out=out) is out
    torch.cuda.synchronize()
    assert (out == 7.0).all()
    g.close()


def test_allreduce_refusals():
    import all_gather_gemm_amd as AG
    lib, vp = AG.lib, AG.ctypes.c_void_p
    h = vp()
    assert lib.ag_gemm_ar_create(0, 0, 64, 64, 64, 0, 0, AG.ctypes.byref(h)) == -1     # D
    assert lib.ag_gemm_ar_create(2, 2, 64, 64, 64, 0, 0, AG.ctypes.byref(h)) == -1     # rank
    g = AG.GemmAllReduce(2, 0, 64, 64, 64)
    A = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    C = [torch.zeros((64, 64), dtype=torch.float32, device="cuda") for _ in range(2)]
    s = torch.cuda.current_stream().cuda_stream
    arr = (vp * 2)(vp(C[0].data_ptr()), vp(C[0].data_ptr()))                          # aliasing
    assert lib.ag_gemm_ar_run(vp(g.handle), vp(A.data_ptr()), vp(A.data_ptr()), arr, vp(s)) == -1
    assert AG.ag_matmul_run(g.handle, [A.data_ptr()], A.data_ptr(), None, C[0].data_ptr(), s) == -1
    plain = AG.AgMatmul(1, 64, 64, 64)
    ok = (vp * 2)(vp(C[0].data_ptr()), vp(C[1].data_ptr()))
    assert lib.ag_gemm_ar_run(vp(plain.handle), vp(A.data_ptr()), vp(A.data_ptr()), ok, vp(s)) == -1
    torch.cuda.synchronize()
    g.close()
    plain.close()


FLAG_CASES = CASES + [(2, 2048, 2048, 256, "f16", 128)]   # more tiles than the reducer lag


@pytest.mark.parametrize("D,M,N,Kl,dt,bm", FLAG_CASES)
def test_allreduce_flags_matches_oracle_and_atomics(D, M, N, Kl, dt, bm):
    """The per-tile flag variant (every rank's share in one launch): within the 16-bit
    tolerance of the oracle, the same bits on a second run, and bit-identical to the atomics
    variant's shares run in rank order and finalized (both add the same fp32 partial tiles
    in rank order, then the bias, then round once)."""
    import all_gather_gemm_amd as AG
    print(f"case ar-flags D={D} {M}x{N}x{Kl} {dt} bm={bm}", flush=True)
    A, B, bias = _parts(D, M, N, Kl, dt, 900 + D)
    Ad, Bd, bd = [a.cuda() for a in A], [b.cuda() for b in B], bias.cuda()
    h = AG.GemmAllReduceFlags(D, M, N, Kl, dt, bm)
    out = h.run(Ad, Bd, bd)
    out2 = h.run(Ad, Bd, bd)
    C = [torch.zeros((M, N), dtype=torch.float32, device="cuda") for _ in range(D)]
    hs = [AG.GemmAllReduce(D, r, M, N, Kl, dt, bm) for r in range(D)]
    for r in range(D):
        hs[r].run(Ad[r], Bd[r], C)
    fin = hs[0].finalize(C[(1) % D], bd)   # rank 0 adds into rank 1's buffer first; all equal
    torch.cuda.synchronize()
    Cref, _ = _reference(D, dt, A, B)
    bdec = oracle.decode(dt, _bits(bias))
    res = oracle.check(dt, out_bits(out), Cref + bdec[None, :])
    assert res["bad"] == 0, res
    assert np.array_equal(out_bits(out), out_bits(out2))
    assert np.array_equal(out_bits(out), out_bits(fin))
    for x in hs + [h]:
        x.close()


def test_allreduce_flags_refusals():
    import all_gather_gemm_amd as AG
    lib, vp = AG.lib, AG.ctypes.c_void_p
    h = vp()
    assert lib.ag_gemm_ar_flags_create(0, 64, 64, 64, 0, 0, AG.ctypes.byref(h)) == -1
    g = AG.GemmAllReduceFlags(2, 64, 64, 64)
    A = [torch.zeros((64, 64), dtype=torch.float16, device="cuda") for _ in range(2)]
    s = torch.cuda.current_stream().cuda_stream
    ap = (vp * 2)(*[vp(a.data_ptr()) for a in A])
    assert lib.ag_gemm_ar_flags_run(vp(g.handle), ap, ap, None, vp(A[1].data_ptr()), vp(s)) == -1  # out = an input
    C = [torch.zeros((64, 64), dtype=torch.float32, device="cuda") for _ in range(2)]
    cp = (vp * 2)(*[vp(c.data_ptr()) for c in C])
    assert lib.ag_gemm_ar_run(vp(g.handle), vp(A[0].data_ptr()), vp(A[0].data_ptr()), cp, vp(s)) == -1
    assert lib.ag_gemm_ar_finalize(vp(g.handle), vp(C[0].data_ptr()), None, vp(A[0].data_ptr()), vp(s)) == -1
    assert AG.ag_matmul_run(g.handle, [A[0].data_ptr()], A[0].data_ptr(), None, A[1].data_ptr(), s) == -1
    plain = AG.GemmAllReduce(2, 0, 64, 64, 64)
    out = torch.empty((64, 64), dtype=torch.float16, device="cuda")
    assert lib.ag_gemm_ar_flags_run(vp(plain.handle), ap, ap, None, vp(out.data_ptr()), vp(s)) == -1
    torch.cuda.synchronize()
    g.close()
    plain.close()
