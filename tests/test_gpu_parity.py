"""GPU parity: the HIP path (through the C ABI) against the oracle.

Tolerance (unrounded fp64 reference C): |out - C| <= 2^-7 |C| + 1e-2 for bf16 output and
2^-10 |C| + 1e-3 for fp16 output. Exact-integer inputs make every fp32 partial sum exact,
so there the GPU must equal the oracle's rounded result bit for bit. Variants that only
change where A is read from (fused vs baseline, staging layout, local shard in place or
staged, shard count D, rank) share one K order on the GPU and must agree bit for bit.
"""
import numpy as np
import pytest

from agmm_testlib import NAN16, assert_close, oracle_full, out_bits, run_gpu
from workloads import (LARGE_16384, MID_4096, SQUARE_1024, SQUARE_4096, TINY, Workload,
                       make_inputs)

pytestmark = pytest.mark.gpu


def _both(w, inp, **kw):
    f = run_gpu(w, inp, "fused", **kw)
    b = run_gpu(w, inp, "baseline", **kw)
    return out_bits(f.out), out_bits(b.out), f.config


@pytest.mark.parametrize("w", [TINY, SQUARE_1024], ids=lambda w: w.name)
def test_small_workloads_full_oracle(w):
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    C, _ = oracle_full(w, inp)
    fo, bo, cfg = _both(w, inp)
    assert_close(w, fo, C, "fused")
    assert_close(w, bo, C, "baseline")
    assert np.array_equal(fo, bo)


RAGGED = [
    # (D, M_s, N, K, dtype, layout, bias, block_m)
    (3, 200, 328, 424, "f16", "k_contiguous", True, 64),
    (3, 200, 328, 424, "bf16", "m_contiguous", False, 64),
    (2, 136, 264, 1032, "f16", "m_contiguous", True, 128),
    (4, 72, 520, 200, "bf16", "k_contiguous", True, 128),
    (2, 264, 392, 1096, "f16", "k_contiguous", False, 256),
    (5, 104, 264, 136, "f16", "m_contiguous", True, 256),
    (1, 296, 136, 72, "bf16", "k_contiguous", True, 256),
]


@pytest.mark.parametrize("D,Ms,N,K,dt,layout,bias,bm", RAGGED)
def test_ragged_shapes_full_oracle(D, Ms, N, K, dt, layout, bias, bm):
    w = Workload(f"ragged_{D}x{Ms}_{N}_{K}_{dt}_{layout}_{bm}", D, D * Ms, N, K, dt,
                 "normal_sqrtk", bias, layout, True, 100 + D + K, rank=D - 1)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    C, _ = oracle_full(w, inp)
    fo, bo, cfg = _both(w, inp, block_m=bm, k_per_flag=1, num_fetch_wgs=3)
    assert cfg["block_m"] == bm
    assert_close(w, fo, C, "fused")
    assert_close(w, bo, C, "baseline")
    assert np.array_equal(fo, bo)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["k_contiguous", "m_contiguous"])
@pytest.mark.parametrize("bm", [64, 128, 256])
def test_exact_integer_bit_exact(dt, layout, bm):
    w = Workload(f"int_{dt}_{layout}_{bm}", 4, 4 * 192, 520, 776, dt, "int", True, layout, True,
                 7, rank=1)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    _, out16 = oracle_full(w, inp)
    fo, bo, _ = _both(w, inp, block_m=bm)
    assert np.array_equal(fo, out16)
    assert np.array_equal(bo, out16)


def test_k_zero_gives_bias_or_zero():
    import torch
    for bias in (False, True):
        w = Workload(f"k0_{bias}", 2, 64, 72, 0, "f16", "uniform", bias, "k_contiguous", True, 3)
        inp = make_inputs(w)
        C, out16 = oracle_full(w, inp)
        fo, bo, _ = _both(w, inp)
        assert np.array_equal(fo, out16) and np.array_equal(bo, out16)


def test_empty_m_or_n_is_a_noop():
    import torch
    import all_gather_gemm_amd as A
    for (M, N) in ((0, 64), (64, 0)):
        op = A.AgMatmul(2, M, N, 64)
        sh = [torch.zeros((M // 2, 64), dtype=torch.float16, device="cuda") for _ in range(2)]
        B = torch.zeros((64, N), dtype=torch.float16, device="cuda")
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        op.run(sh, B, out=out)
        torch.cuda.synchronize()
        op.close()


def test_invariances_bit_exact():
    """Same A cut into D = 1, 2, 4, 8 shards, every rank, both layouts, local shard in place
    or staged, fused or baseline: one output, bit for bit (one tile configuration)."""
    base = Workload("inv", 1, 1024, 512, 1536, "bf16", "normal_sqrtk", True, "k_contiguous",
                    True, 9)
    inp1 = make_inputs(base)
    A_full = inp1.shards[0]
    ref = None
    for D in (1, 2, 4, 8):
        ms = base.M // D
        for rank in sorted({0, D - 1, D // 2}):
            for layout in ("k_contiguous", "m_contiguous"):
                for dl in (True, False):
                    w = base.with_(D=D, rank=rank, layout=layout, direct_local=dl)
                    inp = type(inp1)([A_full[d * ms:(d + 1) * ms].clone() for d in range(D)],
                                     inp1.B, inp1.bias)
                    for algo in ("fused", "baseline"):
                        o = out_bits(run_gpu(w, inp, algo, block_m=128).out)
                        if ref is None:
                            ref = o
                            C, _ = oracle_full(base, inp1)
                            assert_close(base, ref, C)
                        assert np.array_equal(o, ref), (D, rank, layout, dl, algo)


@pytest.mark.parametrize("w", [MID_4096, LARGE_16384, SQUARE_4096], ids=lambda w: w.name)
def test_full_size_full_oracle(w):
    """The full-size workloads in the launch configuration the bench times (auto tile config):
    every output element against the fp64 oracle, and fused == baseline bit for bit."""
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    dev = inp.to("cuda")
    f = run_gpu(w, inp, "fused", dev_inp=dev)
    b = run_gpu(w, inp, "baseline", dev_inp=dev)
    fo = out_bits(f.out)
    assert np.array_equal(fo, out_bits(b.out))
    del f, b
    C, _ = oracle_full(w, inp)
    r = assert_close(w, fo, C, "fused")
    print(f"  {w.name}: {r['count']} outputs, max |err| {r['max_abs_err']:.3g}, "
          f"max err/tol {r['max_ratio']:.3g}", flush=True)


@pytest.mark.parametrize("w", [MID_4096, LARGE_16384, SQUARE_4096], ids=lambda w: w.name)
def test_full_size_exact_integer(w):
    """Full-size shapes with exact-integer inputs (every fp32 partial sum exact): the whole
    output bit-exact against the oracle's single rounding, fused and baseline. A dropped or
    repeated k-tile anywhere changes some output by an integer and fails here, whatever the
    tolerance."""
    wi = w.with_(dist="int", name=w.name + "_int")
    print(f"case {wi.name}", flush=True)
    inp = make_inputs(wi)
    dev = inp.to("cuda")
    fo = out_bits(run_gpu(wi, inp, "fused", dev_inp=dev).out)
    bo = out_bits(run_gpu(wi, inp, "baseline", dev_inp=dev).out)
    _, out16 = oracle_full(wi, inp)
    assert np.array_equal(fo, out16)
    assert np.array_equal(bo, out16)


def _selection_B(K, cols, dtype):
    """B [K, len(cols)] with a single 1 in each column j, at row cols[j]: A @ B = A[:, cols]."""
    import torch
    B = torch.zeros((K, len(cols)), dtype=dtype)
    B[torch.as_tensor(cols), torch.arange(len(cols))] = 1
    return B


@pytest.mark.parametrize("layout", ["k_contiguous", "m_contiguous"])
@pytest.mark.parametrize("kind", ["identity", "permutation"])
def test_selection_B_bit_exact_mid_shape(kind, layout):
    """Identity B (N = K) and a column-selecting permutation B at the 4096x3584x8192 fp16
    shape (4 shards): every output equals the selected element of A exactly (one nonzero
    product per sum), so any wrong row, column, shard or k index of the GEMM shows.
    Compared by value (a -0 input may come out as +0)."""
    import torch
    import oracle
    from workloads import Inputs, bits
    base = make_inputs(MID_4096)
    K = MID_4096.K
    A_bits = np.concatenate([bits(s) for s in base.shards])
    if kind == "identity":
        cols = np.arange(K)
    else:
        cols = np.random.default_rng(33).permutation(K)[:MID_4096.N]
    w = MID_4096.with_(N=len(cols), layout=layout, name=f"mid_{kind}_{layout}")
    print(f"case {w.name}", flush=True)
    inp = Inputs(base.shards, _selection_B(K, cols, torch.float16), None)
    dev = inp.to("cuda")
    want = oracle.decode(w.dtype, A_bits[:, cols])
    for algo in ("fused", "baseline"):
        got = oracle.decode(w.dtype, out_bits(run_gpu(w, inp, algo, dev_inp=dev).out))
        assert np.array_equal(got, want), algo


def test_identity_B_bit_exact_bf16_cube():
    """Identity B at the 4096^3 bf16 shape with 8 shards: out == A exactly."""
    import torch
    import oracle
    from workloads import Inputs, bits
    base = make_inputs(SQUARE_4096)
    K = SQUARE_4096.K
    inp = Inputs(base.shards, _selection_B(K, np.arange(K), torch.bfloat16), None)
    A_bits = np.concatenate([bits(s) for s in base.shards])
    want = oracle.decode("bf16", A_bits)
    dev = inp.to("cuda")
    for algo in ("fused", "baseline"):
        got = oracle.decode("bf16", out_bits(run_gpu(SQUARE_4096, inp, algo, dev_inp=dev).out))
        assert np.array_equal(got, want), algo


SPLIT = [
    # (D, M_s, N, K, dtype, layout, bias, num_wgs): 17 x 16 tiles of 64, so with 256 (or 128)
    # workgroups 16 tiles are left for a last round and split along K
    (2, 544, 1024, 2048, "f16", "m_contiguous", True, 0),      # 4 pieces of 16 K-tiles
    (2, 544, 1024, 2048, "bf16", "k_contiguous", False, 128),  # 4 pieces
    (4, 272, 1024, 1024, "f16", "k_contiguous", True, 0),      # 2 pieces
]


@pytest.mark.parametrize("D,Ms,N,K,dt,layout,bias,nw", SPLIT)
def test_tail_split_full_oracle(D, Ms, N, K, dt, layout, bias, nw):
    """Tiles of the last round cut along K: every piece's partial sums go to the workspace
    and the piece that completes the tile adds them in piece order. Output against the
    oracle, fused == baseline bit for bit, identical over repeated runs (the per-tile piece
    counters are epoch-valued), the same shape without splitting within tolerance, and
    exact-integer inputs bit-exact."""
    from oracle import schedule_model as sm
    w = Workload(f"split_{D}x{Ms}_{N}_{K}_{dt}_{layout}_{nw}", D, D * Ms, N, K, dt,
                 "normal_sqrtk", bias, layout, True, 200 + K + nw, rank=D - 1)
    print(f"case {w.name}", flush=True)
    kw = dict(block_m=64, num_fetch_wgs=8, tail_split=1)
    if nw:
        kw["num_wgs"] = nw
    inp = make_inputs(w)
    dev = inp.to("cuda")
    C, _ = oracle_full(w, inp)
    f = run_gpu(w, inp, "fused", keep=True, dev_inp=dev, **kw)
    cfg = f.config
    g = sm.Geometry(w.D, w.M, w.N, w.K, 64, 64, cfg["block_k"], cfg["k_per_flag"], w.rank, True,
                    cfg["num_fetch_wgs"], cfg["num_wgs"], num_cus=cfg["num_cus"],
                    num_wgs_req=nw, tail_split=1)
    tail, S, _ = sm.split_plan(g)
    assert (cfg["split_tiles"], cfg["split_pieces"]) == (tail, S)
    if cfg["num_cus"] == 256:
        assert tail == 16 and S == (2 if K == 1024 else 4)
    fo = out_bits(f.out)
    assert_close(w, fo, C, "fused")
    for _ in range(2):  # later runs: the same bits
        out = f.op.run(dev.shards, dev.B, dev.bias)
        assert np.array_equal(out_bits(out), fo)
    f.op.close()
    bo = out_bits(run_gpu(w, inp, "baseline", dev_inp=dev, **kw).out)
    assert np.array_equal(fo, bo)
    nosplit = run_gpu(w, inp, "fused", dev_inp=dev, **dict(kw, tail_split=0))
    assert nosplit.config["split_tiles"] == 0
    assert_close(w, out_bits(nosplit.out), C, "fused, no split")
    wi = w.with_(dist="int", name=w.name + "_int")
    inpi = make_inputs(wi)
    _, out16 = oracle_full(wi, inpi)
    assert np.array_equal(out_bits(run_gpu(wi, inpi, "fused", **kw).out), out16)
    assert np.array_equal(out_bits(run_gpu(wi, inpi, "baseline", **kw).out), out16)


GATHER = [
    # (D, M_s, N, K, dtype, bias, block_m (0 = auto), rank, direct_local)
    (2, 136, 264, 1032, "f16", True, 128, 1, True),
    (4, 72, 520, 200, "bf16", False, 64, 0, True),
    (3, 200, 328, 424, "f16", True, 256, 2, False),
    (8, 128, 1024, 1024, "bf16", False, 0, 3, True),
    (1, 296, 136, 72, "bf16", True, 256, 0, True),
]


@pytest.mark.parametrize("D,Ms,N,K,dt,bias,bm,rank,dl", GATHER)
def test_gather_a_parity(D, Ms, N, K, dt, bias, bm, rank, dl):
    """The op that also returns the gathered A ((a, out) = ag_matmul(a_shared, b)): a equals
    the oracle's all_gather bit for bit, and out equals the plain run's output bit for bit
    (same kernels, same K order) and the oracle within tolerance; fused and baseline."""
    import torch
    import all_gather_gemm_amd as A
    import oracle
    from workloads import bits
    w = Workload(f"gather_{D}x{Ms}_{N}_{K}_{dt}", D, D * Ms, N, K, dt, "normal_sqrtk", bias,
                 "k_contiguous", dl, 200 + D + K, rank=rank)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    g = inp.to("cuda")
    A_ref = oracle.all_gather([bits(s) for s in inp.shards])
    C, _ = oracle_full(w, inp)
    tun = {"block_m": bm} if bm else {}
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    for algo in ("fused", "baseline"):
        plain = out_bits(run_gpu(w, inp, algo, dev_inp=g, **tun).out)
        op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=dt, layout="k_contiguous", algo=algo,
                        rank=rank, direct_local=dl, has_bias=bias, gather_a=True, **tun)
        for it in range(2):
            a_out = torch.full((w.M, w.K), float("nan"), dtype=tdt, device="cuda")
            a, out = op.run(g.shards, g.B, g.bias, a_out=a_out)
            torch.cuda.synchronize()
            assert np.array_equal(out_bits(a).reshape(w.M, w.K), A_ref), (algo, it)
            assert np.array_equal(out_bits(out), plain), (algo, it)
        assert_close(w, out_bits(out), C, algo)
        op.close()


def test_gather_a_edge_cases():
    """N = 0 (no output tile, the gathered A is still written), K = 0 (nothing to gather),
    and the entry points refusing the wrong kind of handle."""
    import torch
    import all_gather_gemm_amd as A
    import oracle
    from workloads import bits
    rng = np.random.default_rng(3)
    sh = [torch.from_numpy(rng.standard_normal((64, 72)).astype(np.float16)).cuda() for _ in range(2)]
    A_ref = oracle.all_gather([bits(s.cpu()) for s in sh])
    for algo in ("fused", "baseline"):
        op = A.AgMatmul(2, 128, 0, 72, algo=algo, rank=1, gather_a=True)
        a, out = op.run(sh, torch.zeros((72, 0), dtype=torch.float16, device="cuda"))
        torch.cuda.synchronize()
        assert out.shape == (128, 0)
        assert np.array_equal(out_bits(a).reshape(128, 72), A_ref), algo
        op.close()
    op = A.AgMatmul(2, 128, 64, 0, gather_a=True)
    a, out = op.run([torch.zeros((64, 0), dtype=torch.float16, device="cuda")] * 2,
                    torch.zeros((0, 64), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert a.shape == (128, 0) and not out.float().abs().sum().item()
    op.close()
    # a gather handle refuses ag_matmul_run; a plain handle refuses ag_matmul_run_gather
    B = torch.zeros((72, 64), dtype=torch.float16, device="cuda")
    out = torch.empty((128, 64), dtype=torch.float16, device="cuda")
    a_out = torch.empty((128, 72), dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    ptrs = [t.data_ptr() for t in sh]
    og = A.AgMatmul(2, 128, 64, 72, gather_a=True)
    assert A.ag_matmul_run(og.handle, ptrs, B.data_ptr(), None, out.data_ptr(), s) == -1
    # the gathered A may not alias the output or a shard
    assert A.ag_matmul_run_gather(og.handle, ptrs, B.data_ptr(), None, out.data_ptr(),
                                  sh[0].data_ptr(), s) == -1
    op = A.AgMatmul(2, 128, 64, 72)
    assert A.ag_matmul_run_gather(op.handle, ptrs, B.data_ptr(), None, out.data_ptr(),
                                  a_out.data_ptr(), s) == -1
    torch.cuda.synchronize()
    og.close()
    op.close()


PIPE = [
    # (D, M_s, N, K, dtype, bias, block_m, rank, direct_local, chunks requested)
    (2, 512, 264, 1032, "f16", True, 128, 1, True, 4),
    (4, 128, 520, 200, "bf16", False, 64, 0, True, 2),
    (3, 256, 328, 424, "f16", True, 256, 2, False, 0),
    (8, 128, 1024, 1024, "bf16", False, 64, 3, True, 4),
    (2, 200, 136, 72, "bf16", True, 64, 0, True, 4),     # M_s not a multiple of 64: one chunk
    (1, 512, 136, 264, "f16", False, 128, 0, True, 4),   # D=1: nothing staged
]


@pytest.mark.parametrize("D,Ms,N,K,dt,bias,bm,rank,dl,S", PIPE)
def test_pipelined_parity(D, Ms, N, K, dt, bias, bm, rank, dl, S):
    """The host stream pipeline: output bit-identical to the baseline (same GEMM kernel and K
    order, only the launch schedule differs) and within tolerance of the oracle; chunk
    tables against the model; every chunk's staged rows written (staging poisoned with NaN
    before each run); and with gather_a the gathered A bit-exact."""
    import torch
    import all_gather_gemm_amd as A
    import oracle
    from oracle import schedule_model as sm
    from workloads import bits
    w = Workload(f"pipe_{D}x{Ms}_{N}_{K}_{dt}_{S}", D, D * Ms, N, K, dt, "normal_sqrtk", bias,
                 "k_contiguous", dl, 300 + D + K, rank=rank)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    g = inp.to("cuda")
    C, _ = oracle_full(w, inp)
    base = out_bits(run_gpu(w, inp, "baseline", dev_inp=g, block_m=bm).out)
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=dt, algo="pipelined", rank=rank, direct_local=dl,
                    has_bias=bias, block_m=bm, pipeline_chunks=S)
    cfg = op.config.as_dict()
    geo = sm.Geometry(w.D, w.M, w.N, w.K, cfg["block_m"], cfg["block_n"], cfg["block_k"],
                      cfg["k_per_flag"], rank, dl, cfg["num_fetch_wgs"], cfg["num_wgs"],
                      num_cus=cfg["num_cus"])
    S_model, chunks = sm.pipeline_plan(geo, S)
    assert cfg["pipeline_chunks"] == S_model
    assert cfg["pipeline_streams"] == min(S_model, 4)
    got = op.chunks()
    assert [c[0] for c in got] == [c[0] for c in chunks]
    assert [[x & 0x7FFFFFFF for x in c[1]] for c in got] == [c[1] for c in chunks]
    assert [[bool(x >> 31) for x in c[1]] for c in got] == \
        [[sm.is_direct(geo, t) for t in c[1]] for c in chunks]
    A_bits = np.concatenate([bits(s) for s in inp.shards])
    for it in range(3):
        op.fill_staging(NAN16[dt])
        out = op.run(g.shards, g.B, g.bias)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), base), it
        if cfg["staging_elems"]:
            assert np.array_equal(op.staging(),
                                  sm.expected_staging(geo, A_bits, "k_contiguous", NAN16[dt]))
    assert_close(w, out_bits(out), C, "pipelined")
    op.close()
    # the pipeline with the gathered A returned as well
    opg = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=dt, algo="pipelined", rank=rank, direct_local=dl,
                     has_bias=bias, block_m=bm, pipeline_chunks=S, gather_a=True)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    a_out = torch.full((w.M, w.K), float("nan"), dtype=tdt, device="cuda")
    a, out = opg.run(g.shards, g.B, g.bias, a_out=a_out)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(a).reshape(w.M, w.K), oracle.all_gather(list(map(bits, inp.shards))))
    assert np.array_equal(out_bits(out), base)
    opg.close()


def test_pipelined_back_to_back_on_a_side_stream():
    """Runs enqueued back to back on a non-default caller stream with alternating inputs:
    every run's chunk streams start after the caller's earlier work and the caller's stream
    waits for all of them, so each output matches its own input's baseline."""
    import torch
    import all_gather_gemm_amd as A
    w = Workload("pipe_alt", 4, 4 * 256, 392, 520, "f16", "normal_sqrtk", True, "k_contiguous",
                 True, 61, rank=2)
    sets = [make_inputs(w, seed=s) for s in (61, 62)]
    dev = [s.to("cuda") for s in sets]
    refs = [out_bits(run_gpu(w, s, "baseline", dev_inp=d, block_m=64).out)
            for s, d in zip(sets, dev)]
    op = A.AgMatmul(w.D, w.M, w.N, w.K, algo="pipelined", rank=w.rank, has_bias=True,
                    block_m=64, pipeline_chunks=4)
    side = torch.cuda.Stream()
    outs = [torch.empty((w.M, w.N), dtype=torch.float16, device="cuda") for _ in range(6)]
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for it in range(6):
            i = it % 2
            op.run(dev[i].shards, dev[i].B, dev[i].bias, out=outs[it], stream=side)
    side.synchronize()
    for it in range(6):
        assert np.array_equal(out_bits(outs[it]), refs[it % 2]), it
    op.close()


@pytest.mark.parametrize("Ms,layout", [(8, "k_contiguous"), (8, "m_contiguous"), (1, "m_contiguous"),
                                       (3, "k_contiguous")])
def test_sixty_four_shards(Ms, layout):
    """The most shards the ABI takes (64): every m-tile spans many shards, so the fetch takes
    its per-row shard lookup path. Fused, baseline and pipelined against the full oracle and
    against each other bit for bit."""
    D = 64
    w = Workload(f"d64_{Ms}_{layout}", D, D * Ms, 136, 264, "f16", "normal_sqrtk", True, layout,
                 True, 400 + Ms, rank=37)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    C, _ = oracle_full(w, inp)
    outs = [out_bits(run_gpu(w, inp, algo).out) for algo in ("fused", "baseline", "pipelined")]
    assert_close(w, outs[0], C, "fused")
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
