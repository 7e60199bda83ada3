#!/usr/bin/env python3
"""Benchmark of the fused all-gather + GEMM on one MI355X.

A step is one ag_matmul_run over the resident synthetic inputs of the headline workload
(16384x3584x8192 fp16, D=8 shards of 2048 rows, fp16 bias, m_contiguous staging, local
shard read in place). Warmup steps are untimed; the K timed steps are bracketed by device
synchronizations and timed twice: wall clock over the whole region, and HIP events around
every launch on the launch stream (the fused path is one kernel per step, so the events
time that kernel). TFLOP/s counts 2*M*N*K per step with M the full gathered row count, the
convention of the iris issue's results tables.

Prints ONE JSON line on stdout. Unless --no-extras, the line also carries the other variants
on the same inputs: the copy-barrier-GEMM baseline (runs interleaved with the fused ones,
and "standalone": each timed back to back in alternating blocks, plus cold-cache single
runs, each after 1 GiB of unrelated writes, the two handles taking turns), the baseline's
copy and GEMM phases timed alone (the copy's staging rate against the HBM peak), the shader
clock and socket power sampled under sustained fused load, the host stream pipeline (2, 4, 8
chunks), the variant that also returns the gathered A, the GEMM + all-reduce variants, and
torch.matmul on a pre-gathered A as a yardstick. kernel_resources gives the fused and GEMM
kernels' registers, spills and LDS from the built code object. `--sweep` additionally writes
a table of all five workloads to stderr and, with --out, to a JSON-lines file; `--timeline`
prints the fused kernel's fetch/GEMM overlap from a debug trace instead.
"""
import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + % MFMA peak, fused AG+GEMM 16384x3584x8192 fp16, D=8, 1 GPU"
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # MI355X dense fp16/bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def tflops(M, N, K, seconds):
    """2*M*N*K / t in TFLOP/s (the pages' convention, M = gathered rows)."""
    return 2.0 * M * N * K / seconds / 1e12


def time_runs(op, dev, steps, warmup, torch):
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        op.run(dev.shards, dev.B, dev.bias, out=dev.out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(s)
        op.run(dev.shards, dev.B, dev.bias, out=dev.out, check=False)
        b.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]   # ms
    return wall, per


def interleaved(w, algos, steps, warmup, torch, A, inputs=None, dev=None, **tun):
    """Median ms per op of several variants on the same inputs, their runs alternating on one
    stream (forward, then backward order), so that clock drift, the power limit's state and
    allocator state fall on every variant alike. A variant is an algorithm name, or a tuple
    (name, algorithm, extra tunables). Returns ({name: median_ms}, {name: config}, inputs,
    dev)."""
    from workloads import make_inputs
    inp = inputs if inputs is not None else make_inputs(w)
    if dev is None:
        dev = inp.to("cuda")
        dev.out = torch.empty((w.M, w.N), dtype=w.torch_dtype(), device="cuda")
    ops = []
    for v in algos:
        name, algo, kw = (v, v, {}) if isinstance(v, str) else v
        ops.append((name, A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout,
                                     algo=algo, rank=w.rank, direct_local=w.direct_local,
                                     has_bias=w.has_bias, **{**tun, **kw})))
    for _ in range(warmup):
        for _, op in ops:
            op.run(dev.shards, dev.B, dev.bias, out=dev.out)
    torch.cuda.synchronize()
    ev = {name: [] for name, _ in ops}
    for i in range(steps):
        for a, op in (ops if i % 2 == 0 else ops[::-1]):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            op.run(dev.shards, dev.B, dev.bias, out=dev.out, check=False)
            e1.record()
            ev[a].append((e0, e1))
    torch.cuda.synchronize()
    med = {a: statistics.median(e0.elapsed_time(e1) for e0, e1 in v) for a, v in ev.items()}
    cfgs = {a: op.config.as_dict() for a, op in ops}
    for _, op in ops:
        op.close()
    return med, cfgs, inp, dev


def bench_workload(w, algo, steps, warmup, torch, A, inputs=None, dev=None, **tun):
    from workloads import make_inputs
    inp = inputs if inputs is not None else make_inputs(w)
    if dev is None:
        dev = inp.to("cuda")
        dev.out = torch.empty((w.M, w.N), dtype=w.torch_dtype(), device="cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, algo=algo, rank=w.rank,
                    direct_local=w.direct_local, has_bias=w.has_bias, **tun)
    wall, per = time_runs(op, dev, steps, warmup, torch)
    cfg = op.config.as_dict()
    op.close()
    return {"wall_s": wall, "per_ms": per, "config": cfg, "inputs": inp, "dev": dev}


def gather_variant(w, dev, steps, warmup, torch, A):
    """The op that also returns the gathered A, (a, out) = ag_matmul(a_shared, b), on the
    workload's shape with k_contiguous staging (the caller's [M, K] buffer is the staging):
    median ms of fused and baseline, and of the plain fused run on the same layout, whose
    difference is the cost of also copying the local shard. Runs interleaved on one stream."""
    wk = w.with_(layout="k_contiguous")
    a_out = torch.empty((wk.M, wk.K), dtype=wk.torch_dtype(), device="cuda")
    ops = []
    for key, algo, gather in (("fused_ms", "fused", True), ("baseline_ms", "baseline", True),
                              ("fused_no_gather_ms", "fused", False)):
        ops.append((key, A.AgMatmul(wk.D, wk.M, wk.N, wk.K, dtype=wk.dtype, layout=wk.layout,
                                    algo=algo, rank=wk.rank, direct_local=wk.direct_local,
                                    has_bias=wk.has_bias, gather_a=gather),
                    {"a_out": a_out} if gather else {}))
    for _ in range(warmup):
        for _, op, kw in ops:
            op.run(dev.shards, dev.B, dev.bias, out=dev.out, **kw)
    torch.cuda.synchronize()
    ev = {key: [] for key, _, _ in ops}
    for i in range(steps):
        for key, op, kw in (ops if i % 2 == 0 else ops[::-1]):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            op.run(dev.shards, dev.B, dev.bias, out=dev.out, check=False, **kw)
            e1.record()
            ev[key].append((e0, e1))
    torch.cuda.synchronize()
    res = {"workload": wk.name, "layout": wk.layout}
    for key, op, _ in ops:
        res[key] = round(statistics.median(e0.elapsed_time(e1) for e0, e1 in ev[key]), 5)
        op.close()
    res["fused_speedup"] = round(res["baseline_ms"] / res["fused_ms"], 3)
    del a_out
    torch.cuda.empty_cache()
    return res


def gemm_allreduce_variant(w, steps, warmup, torch, A):
    """One rank's share of GEMM + all-reduce (atomics) on the workload's output shape: A_r
    [M, K/D] @ B_r [K/D, N] added in fp32 into the D result buffers with device atomics.
    Median ms of that share and of the plain GEMM of the same shape (16-bit output, no
    atomics), interleaved on one stream; TFLOP/s of the share and its atomic-add rate
    (D * M * N fp32 adds per share), and the ms of the finalize pass (one buffer to 16 bits).
    Also the per-tile flag variant, all D ranks' shares in one launch, against D shares of
    the atomics variant plus a finalize (the same result on one GPU).
    """
    D, M, N, Kl = w.D, w.M, w.N, w.K // w.D
    tdt = w.torch_dtype()
    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn((M, Kl), generator=g, device="cuda").div_(Kl ** 0.5).to(tdt)
    b = torch.randn((Kl, N), generator=g, device="cuda").to(tdt)
    C = [torch.zeros((M, N), dtype=torch.float32, device="cuda") for _ in range(D)]
    out = torch.empty((M, N), dtype=tdt, device="cuda")
    ar = A.GemmAllReduce(D, w.rank, M, N, Kl, w.dtype)
    plain = A.AgMatmul(1, M, N, Kl, dtype=w.dtype, algo="baseline")
    # the per-tile flag variant: all D ranks' shares (distinct A_r, B_r) in one launch
    a_parts = [a] + [torch.randn((M, Kl), generator=g, device="cuda").div_(Kl ** 0.5).to(tdt)
                     for _ in range(D - 1)]
    b_parts = [b] + [torch.randn((Kl, N), generator=g, device="cuda").to(tdt) for _ in range(D - 1)]
    fl = A.GemmAllReduceFlags(D, M, N, Kl, w.dtype)
    runs = {"share_ms": lambda: ar.run(a, b, C, check=False),
            "plain_gemm_ms": lambda: plain.run([a], b, None, out=out, check=False),
            "finalize_ms": lambda: ar.finalize(C[0], None, out=out),
            "flags_all_ranks_ms": lambda: fl.run(a_parts, b_parts, None, out=out, check=False)}
    for _ in range(warmup):
        for f in runs.values():
            f()
    torch.cuda.synchronize()
    ev = {k: [] for k in runs}
    keys = list(runs)
    for i in range(steps):
        for k in (keys if i % 2 == 0 else keys[::-1]):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            runs[k]()
            e1.record()
            ev[k].append((e0, e1))
    torch.cuda.synchronize()
    res = {"D": D, "M": M, "N": N, "K_local": Kl, "dtype": w.dtype}
    for k in keys:
        res[k] = round(statistics.median(e0.elapsed_time(e1) for e0, e1 in ev[k]), 5)
    res["share_tflops"] = round(tflops(M, N, Kl, res["share_ms"] * 1e-3), 1)
    res["atomic_adds_per_s"] = round(D * M * N / (res["share_ms"] * 1e-3), 0)
    res["atomic_GBps"] = round(D * M * N * 4 / (res["share_ms"] * 1e-3) / 1e9, 1)
    res["flags_all_ranks_tflops"] = round(tflops(M, N, D * Kl, res["flags_all_ranks_ms"] * 1e-3), 1)
    res["atomics_all_ranks_ms"] = round(D * res["share_ms"] + res["finalize_ms"], 5)
    ar.close()
    plain.close()
    fl.close()
    del a, b, C, out, a_parts, b_parts
    torch.cuda.empty_cache()
    return res


def yardstick_matmul(w, dev, steps, warmup, torch):
    """torch.matmul on a pre-gathered A (library GEMM, context only)."""
    Ag = torch.cat(dev.shards, 0)
    for _ in range(warmup):
        torch.matmul(Ag, dev.B)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        torch.matmul(Ag, dev.B)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


TRAFFIC_FILE = "profiles/agmm_persistent_fused_16384x3584x8192_f16_hbm_traffic.md"
RESOURCES_FILE = "all_gather_gemm_amd/kernel_resources.json"


def kernel_resources():
    """The built library's per-kernel registers, spills and LDS (written by the build from the
    gfx950 code object's metadata), or None when the build did not write them."""
    try:
        with open(os.path.join(ROOT, RESOURCES_FILE)) as fh:
            return json.load(fh)
    except (OSError, ValueError):
        return None


def kernel_entry(res, block_m, dtype, fused, layout_k, row_wait):
    """Resources of one agmm_persistent instance (by its mangled template arguments)."""
    if not res:
        return None
    dt = 1 if dtype == "bf16" else 0
    tag = "agmm_persistentILi%dELi%dELb%dELb%dELb%dELi0EE" % (block_m, dt, int(fused),
                                                             int(layout_k), int(row_wait))
    for k, v in res["kernels"].items():
        if tag in k:
            return dict(v, symbol=k)
    return None


def measured_traffic(workload_name, algo):
    """HBM bytes per launch of the fused kernel from the committed counter summary (rocprofv3
    FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when that summary was taken on other
    machine code (the hash of the fused kernel's instructions it records differs from the
    built kernel's) or another workload."""
    if workload_name != "ag_16384x3584x8192_d8_f16_bias" or algo != "fused":
        return None
    res = kernel_resources()
    if not res:
        return None
    kv = {}
    try:
        with open(os.path.join(ROOT, TRAFFIC_FILE)) as fh:
            for line in fh:
                if ":" in line and not line.startswith(("|", "#", "-")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
    except OSError:
        return None
    ent = kernel_entry(res, 256, "f16", True, False, False)
    if not ent or kv.get("kernel_code_sha256") != ent.get("code_sha256"):
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def sample_sclk(n=4, gap_s=0.3):
    """Shader clock (MHz, rocm-smi) and socket power (W, amd-smi), read n times gap_s apart
    (None where unreadable)."""
    import re
    import subprocess
    out = []
    for i in range(n):
        clk = pw = None
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                               text=True, timeout=20)
            m = re.search(r'"sclk clock speed:":\s*"\((\d+)Mhz\)"', r.stdout)
            clk = int(m.group(1)) if m else None
        except Exception:
            pass
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "--json"],
                               capture_output=True, text=True, timeout=20)
            m = re.search(r'"socket_power":\s*\{\s*"value":\s*(\d+)', r.stdout)
            pw = int(m.group(1)) if m else None
        except Exception:
            pass
        out.append((clk, pw))
        time.sleep(gap_s)
    return out


def clock_under_load(op, dev, torch, seconds=2.0):
    """Median shader clock and socket power while the op runs back to back for about
    `seconds`."""
    import threading
    samples = []
    th = threading.Thread(target=lambda: samples.extend(sample_sclk(4, seconds / 6)))
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            op.run(dev.shards, dev.B, dev.bias, out=dev.out, check=False)
        torch.cuda.synchronize()
    th.join()
    med = lambda v: sorted(v)[len(v) // 2] if v else None
    clk = [c for c, _ in samples]
    pw = [p for _, p in samples]
    return {"sclk_mhz_samples": clk, "sclk_mhz_median": med([c for c in clk if c]),
            "socket_power_w_samples": pw, "socket_power_w_median": med([p for p in pw if p])}


def block_times(w, ops, dev, torch, blocks, per):
    """Median ms per run of each op, each timed back to back in blocks of `per` runs, the
    blocks of the ops alternating (order reversed every other round): every op runs in its
    own sustained state, and drift falls on all of them alike."""
    res = {n: [] for n, _ in ops}
    for blk in range(blocks):
        for n, op in (ops if blk % 2 == 0 else ops[::-1]):
            for _ in range(2):
                op.run(dev.shards, dev.B, dev.bias, out=dev.out, check=False)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(per):
                op.run(dev.shards, dev.B, dev.bias, out=dev.out, check=False)
            e1.record()
            torch.cuda.synchronize()
            res[n].append(e0.elapsed_time(e1) / per)
    return {n: statistics.median(v) for n, v in res.items()}


def standalone_ops(w, A, tun):
    """Handles timed in sustained blocks against each other: the fused run (fetchers in the
    grid), the barrier baseline, and the fused run with its fetch as a kernel of its own
    beside the grid (fetch_kernel=1; 'fetch_kernel')."""
    mk = lambda algo, **kw: A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout,
                                       algo=algo, rank=w.rank, direct_local=w.direct_local,
                                       has_bias=w.has_bias, **{**tun, **kw})
    return [("fused", mk("fused", fetch_kernel=-1)), ("baseline", mk("baseline")),
            ("fetch_kernel", mk("fused", fetch_kernel=1))]


def cold_times(ops, dev, torch, reps, flush_bytes=1 << 30):
    """Median ms of single runs of each op, each run after 1 GiB of unrelated writes (untimed)
    have pushed the op's working set out of the caches. The ops take turns, so that the
    clock's drift over the series (the first runs after a pause are slow) falls on all of
    them alike."""
    junk = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    per = {n: [] for n, _ in ops}
    for i in range(reps):
        for n, op in (ops if i % 2 == 0 else ops[::-1]):
            junk.fill_(7)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            op.run(dev.shards, dev.B, dev.bias, out=dev.out, check=False)
            e1.record()
            torch.cuda.synchronize()
            per[n].append(e0.elapsed_time(e1))
    del junk
    torch.cuda.empty_cache()
    return {n: statistics.median(v) for n, v in per.items()}


def baseline_parts(w, dev, torch, A, reps=20):
    """The barrier baseline's two phases timed alone (debug entry point): the staging copy
    (its HBM rate against the peak) and the GEMM over the staged A."""
    import all_gather_gemm_amd as AA
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, algo="baseline",
                    rank=w.rank, direct_local=w.direct_local, has_bias=w.has_bias)
    out = {}
    for name, part in (("copy", AA.PART_COPY), ("gemm", AA.PART_GEMM)):
        for _ in range(3):
            op.run_part(part, dev.shards, dev.B, dev.bias, out=dev.out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            op.run_part(part, dev.shards, dev.B, dev.bias, out=dev.out)
        e1.record()
        torch.cuda.synchronize()
        out[name + "_ms"] = e0.elapsed_time(e1) / reps
    op.close()
    staged = 2 * (w.M - (w.M_s if w.direct_local else 0)) * w.K * 2
    return {"copy_ms": round(out["copy_ms"], 5), "staging_bytes": staged,
            "copy_gbs": round(staged / (out["copy_ms"] * 1e-3) / 1e9, 1),
            "copy_frac_of_hbm_peak": round(staged / (out["copy_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "gemm_ms": round(out["gemm_ms"], 5),
            "gemm_tflops": round(tflops(w.M, w.N, w.K, out["gemm_ms"] * 1e-3), 1)}


def mfma_ceiling(torch, A, iters=20000):
    """TFLOP/s of a register-only MFMA loop (ag_matmul_debug_mfma_loop), fp16, per grid size
    and operand kind, best of 3 launches: the rate the chip sustains with no memory traffic, at
    the clock its power limit allows for that switching activity."""
    sink = torch.empty(512 * 256, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    res = {}
    for vary in (False, True):
        for grid in (64, 256, 512):
            A.ag_matmul_debug_mfma_loop(A.F16, vary, grid, 2000, sink.data_ptr(), s)
            torch.cuda.synchronize()
            best = None
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                rc = A.ag_matmul_debug_mfma_loop(A.F16, vary, grid, iters, sink.data_ptr(), s)
                e1.record()
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError(f"ag_matmul_debug_mfma_loop: {rc}")
                ms = e0.elapsed_time(e1)
                tf = grid * 4 * iters * 16 * 32768.0 / (ms * 1e-3) / 1e12
                best = tf if best is None else max(best, tf)
            res[f"{'rotating' if vary else 'fixed'}_operands_grid{grid}_tflops"] = round(best, 1)
    res["peak_tflops"] = PEAK_TFLOPS["f16"]
    return res


def graph_replay(w, torch, A, runs=20, reps=5, **tun):
    """Per-run time of `runs` fused runs issued from the host one by one (each through the
    Python binding and the C ABI) against the same runs captured once into a HIP graph and
    replayed: wall clock from the first enqueue to the end of the stream work, best of `reps`.
    The kernels count run epochs on the device, so a captured run replays correctly."""
    import time
    from workloads import make_inputs
    dev = make_inputs(w).to("cuda")
    out = torch.empty((w.M, w.N), dtype=w.torch_dtype(), device="cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, rank=w.rank,
                    direct_local=w.direct_local, has_bias=w.has_bias, **tun)
    run = lambda: op.run(dev.shards, dev.B, dev.bias, out=out)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ref = out.clone()

    def wall(fn):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) * 1e3 / runs
            best = dt if best is None else min(best, dt)
        return best

    eager = wall(lambda: [run() for _ in range(runs)])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(runs):
            run()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, ref))
    replay = wall(g.replay)
    del g
    op.close()
    return {"workload": w.name, "runs": runs, "eager_ms_per_run": round(eager, 5),
            "graph_ms_per_run": round(replay, 5), "graph_output_bit_identical": same}


def timeline(w, torch, A, runs=3, **tun):
    """Fetch-vs-GEMM overlap of the fused kernel from its debug trace (per-workgroup fetch,
    tile and wait records, 100 MHz timestamps) on the last of `runs` runs. Debug runs record
    every event, so absolute times run somewhat longer than timed runs."""
    from workloads import make_inputs
    inp = make_inputs(w)
    dev = inp.to("cuda")
    op = A.AgMatmul(w.D, w.M, w.N, w.K, dtype=w.dtype, layout=w.layout, rank=w.rank,
                    direct_local=w.direct_local, has_bias=w.has_bias, debug=True, trace_cap=64,
                    **tun)
    for _ in range(runs):
        op.run(dev.shards, dev.B, dev.bias)
        torch.cuda.synchronize()
    counts, recs = op.trace()
    cfg = op.config.as_dict()
    direct = {int(e & 0x7FFFFFFF) for e in op.mtiles() if e >> 31}
    ev = []
    for wg in range(len(counts)):
        for r in recs[wg, :min(int(counts[wg]), recs.shape[1])]:
            ev.append((wg, int(r["event"]), int(r["a"]), int(r["t0"]), int(r["t1"])))
    op.close()
    t0 = min(e[3] for e in ev)
    us = lambda t: (t - t0) * 1e-2
    fetch = [e for e in ev if e[1] == 1]
    gemm = [e for e in ev if e[1] == 2]
    wait = [e for e in ev if e[1] == 3]
    span = us(max(e[4] for e in ev))
    res = {"workload": w.name, "block_m": cfg["block_m"], "fetch_wgs": cfg["num_fetch_wgs"],
           "wgs": cfg["num_wgs"], "k_per_flag": cfg["k_per_flag"], "row_wait": cfg["row_wait"],
           "span_us": round(span, 1)}
    q = lambda v, f: sorted(v)[int(f * (len(v) - 1))]
    if fetch:
        fe = [us(e[4]) for e in fetch]
        res.update({"units": len(fetch), "fetch_end_us": round(max(fe), 1),
                    "fetch_end_frac": round(max(fe) / span, 3),
                    "unit_us_median": round(statistics.median((e[4] - e[3]) * 1e-2 for e in fetch), 2)})
        # MFMA work that ran while the fetch was still going: tile time inside [0, fetch end]
        fend = max(e[4] for e in fetch)
        overl = sum(max(0, min(e[4], fend) - e[3]) for e in gemm) * 1e-2
        res["tile_us_during_fetch"] = round(overl, 1)
        res["tile_us_total"] = round(sum((e[4] - e[3]) * 1e-2 for e in gemm), 1)
    st = [(e[4] - e[3]) * 1e-2 for e in gemm if e[2] not in direct]
    dr = [(e[4] - e[3]) * 1e-2 for e in gemm if e[2] in direct]
    if st:
        res["staged_tile_us_median"] = round(statistics.median(st), 1)
    if dr:
        res["direct_tile_us_median"] = round(statistics.median(dr), 1)
    starts = [us(min(e[3] for e in gemm if e[0] == wg)) for wg in {e[0] for e in gemm}]
    ends = [us(max(e[4] for e in gemm if e[0] == wg)) for wg in {e[0] for e in gemm}]
    res["wg_first_tile_start_us_p50_p90_max"] = [round(q(starts, f), 1) for f in (0.5, 0.9, 1.0)]
    res["wg_last_tile_end_us_min_p50_max"] = [round(q(ends, f), 1) for f in (0.0, 0.5, 1.0)]
    per = {}
    for e in gemm:
        per[e[0]] = per.get(e[0], 0) + 1
    hist = {}
    for n in per.values():
        hist[n] = hist.get(n, 0) + 1
    res["tiles_per_wg"] = {str(k): v for k, v in sorted(hist.items())}
    if wait:
        res["waits"] = len(wait)
        res["wait_us_total"] = round(sum((e[4] - e[3]) * 1e-2 for e in wait), 1)
    return res


def cpu_baseline(w, inp, gpu_out, target_s):
    """The oracle, as it stands, on a bounded sample of output rows of the same workload."""
    import numpy as np
    import oracle
    from workloads import bits
    sh = [bits(s) for s in inp.shards]
    Bb = bits(inp.B)
    bias = bits(inp.bias) if inp.bias is not None else None
    thr = oracle.max_threads()
    rows = max(1, min(w.M, 2 * thr))
    t0 = time.perf_counter()
    C, _, used = oracle.agmm(w.dtype, sh, Bb, bias, 0, rows)
    t = time.perf_counter() - t0
    # grow the sample until it takes about target_s (small samples run below the threads'
    # full rate, so one extrapolation undershoots)
    while t < target_s / 2 and rows < w.M:
        rows = int(min(w.M, max(rows + 1, rows * 0.9 * target_s / max(t, 1e-3))))
        t0 = time.perf_counter()
        C, _, used = oracle.agmm(w.dtype, sh, Bb, bias, 0, rows)
        t = time.perf_counter() - t0
    got = gpu_out[:rows].detach().cpu().contiguous().view(__import__("torch").int16).numpy()
    chk = oracle.check(w.dtype, got.view(np.uint16), C)
    return {"value": round(tflops(rows, w.N, w.K, t), 6), "unit": "TFLOP/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"output rows 0..{rows - 1} of {w.M} ({rows}x{w.N}x{w.K}), {t:.2f} s, "
                      f"fp64 C oracle, OpenMP over rows",
            "parity_rows_bad": int(chk["bad"]), "parity_max_err_over_tol": chk["max_ratio"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ag_16384x3584x8192_d8_f16_bias")
    ap.add_argument("--algo", default="fused", choices=["fused", "baseline", "pipelined"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the requested algorithm (for profiler runs)")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--out", default=None)
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--fetch-wgs", type=int, default=0)
    ap.add_argument("--k-per-flag", type=int, default=0)
    ap.add_argument("--fetch-kernel", action="store_true",
                    help="fused: run the fetch as a kernel of its own beside the GEMM grid")
    ap.add_argument("--timeline", action="store_true",
                    help="only print the fused kernel's fetch/GEMM timeline from a debug trace "
                         "(for each of --workload, or of all five workloads with --sweep)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the MFMA rate with pseudo-random register operands (no "
                         "memory traffic), one set or four rotating, on 64, 256 and 512 workgroups")
    ap.add_argument("--graph", action="store_true",
                    help="only time fused runs issued one by one against the same runs captured "
                         "in a HIP graph and replayed (for each of --workload, or of all five "
                         "workloads with --sweep)")
    ap.add_argument("--yardstick", action="store_true",
                    help="only time torch.matmul (hipBLASLt) on a pre-gathered A of --workload: "
                         "--warmup untimed and --steps timed launches, for counter runs beside "
                         "the library's GEMM kernel")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times): the "
                         "known-size reference for the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the "
              "multi-GPU pull over xGMI is designed but not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import all_gather_gemm_amd as A
    from workloads import BY_NAME, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                          "dispatches": 3}), flush=True)
        return
    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling(torch, A)), flush=True)
        return
    if args.timeline:
        for w in (WORKLOADS if args.sweep else [BY_NAME[args.workload]]):
            print(json.dumps(timeline(w, torch, A)), flush=True)
        return
    if args.graph:
        for w in (WORKLOADS if args.sweep else [BY_NAME[args.workload]]):
            print(json.dumps(graph_replay(w, torch, A)), flush=True)
        return
    if args.yardstick:
        from workloads import make_inputs
        w = BY_NAME[args.workload]
        ms = yardstick_matmul(w, make_inputs(w).to("cuda"), args.steps, args.warmup, torch)
        print(json.dumps({"workload": w.name, "yardstick_torch_matmul_pregathered_ms": round(ms, 5),
                          "tflops": round(tflops(w.M, w.N, w.K, ms / 1e3), 3)}), flush=True)
        return
    tun = {}
    if args.block_m:
        tun["block_m"] = args.block_m
    if args.fetch_wgs:
        tun["num_fetch_wgs"] = args.fetch_wgs
    if args.k_per_flag:
        tun["k_per_flag"] = args.k_per_flag
    if args.fetch_kernel:
        tun["fetch_kernel"] = 1

    if args.sweep:
        rows = []
        # the 4096^3 cube also with its own shard staged like the others (direct-local off),
        # beside the default in-place read
        cube = BY_NAME["square_4096_d8_bf16"]
        extra = [dataclasses.replace(cube, name=cube.name + "_direct_local_off", direct_local=False)]
        for w in list(WORKLOADS) + extra:
            med, cfgs, _, dev = interleaved(w, ("fused", "baseline", "pipelined"), args.steps,
                                            args.warmup, torch, A, **tun)
            ym = yardstick_matmul(w, dev, args.steps, args.warmup, torch)
            mf, mb, mp = med["fused"], med["baseline"], med["pipelined"]
            bops = standalone_ops(w, A, tun)
            bt = block_times(w, bops, dev, torch, 6, 10)
            for _, op in bops:
                op.close()
            row = {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "D": w.D,
                   "dtype": w.dtype, "layout": w.layout,
                   "fused_ms_median": mf,
                   "baseline_ms_median": mb, "speedup": mb / mf,
                   "fused_ms_standalone": bt["fused"], "baseline_ms_standalone": bt["baseline"],
                   "speedup_standalone": bt["baseline"] / bt["fused"],
                   "fetch_kernel_ms_standalone": bt["fetch_kernel"],
                   "pipelined_ms_median": mp,
                   "pipelined_chunks": cfgs["pipelined"]["pipeline_chunks"],
                   "fused_tflops": tflops(w.M, w.N, w.K, mf / 1e3),
                   "baseline_tflops": tflops(w.M, w.N, w.K, mb / 1e3),
                   "pct_peak": 100 * tflops(w.M, w.N, w.K, mf / 1e3) / PEAK_TFLOPS[w.dtype],
                   "torch_matmul_pregathered_ms": ym, "block_m": cfgs["fused"]["block_m"],
                   "fetch_wgs": cfgs["fused"]["num_fetch_wgs"], "wgs": cfgs["fused"]["num_wgs"]}
            rows.append(row)
            print("| {workload} | {fused_ms_median:.4f} | {baseline_ms_median:.4f} | "
                  "{pipelined_ms_median:.4f} (S={pipelined_chunks}) | "
                  "{speedup:.2f}x | {fused_ms_standalone:.4f} | {baseline_ms_standalone:.4f} | "
                  "{speedup_standalone:.3f}x | {fused_tflops:.1f} | {pct_peak:.1f}% | "
                  "{torch_matmul_pregathered_ms:.4f} | {block_m} |".format(**row),
                  file=sys.stderr, flush=True)
            del dev
            torch.cuda.empty_cache()
        if args.out:
            with open(args.out, "w") as fh:
                for r in rows:
                    fh.write(json.dumps(r) + "\n")

    w = BY_NAME[args.workload]
    r = bench_workload(w, args.algo, args.steps, args.warmup, torch, A, **tun)
    per = r["per_ms"]
    ms_step = r["wall_s"] * 1e3 / args.steps
    value = tflops(w.M, w.N, w.K, r["wall_s"] / args.steps)
    avg_ms = sum(per) / len(per)
    achieved = tflops(w.M, w.N, w.K, avg_ms / 1e3)
    peak = PEAK_TFLOPS[w.dtype]
    res = {
        "metric": METRIC if w.name == "ag_16384x3584x8192_d8_f16_bias" and args.algo == "fused" else
                  f"TFLOP/s + % MFMA peak, {args.algo} AG+GEMM {w.M}x{w.N}x{w.K} {w.dtype}, D={w.D}, 1 GPU",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; see workloads.py)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "D": w.D,
                   "shard_rows": w.M_s, "layout": w.layout, "bias": w.has_bias,
                   "direct_local": w.direct_local, "rank": w.rank, "algo": args.algo,
                   "block_m": r["config"]["block_m"], "block_k": r["config"]["block_k"],
                   "k_per_flag": r["config"]["k_per_flag"],
                   "fetch_wgs": r["config"]["num_fetch_wgs"], "wgs": r["config"]["num_wgs"]},
        "pct_mfma_peak": round(100 * value / peak, 2),
        "latency_ms": {"median": round(statistics.median(per), 5), "min": round(min(per), 5),
                       "p90": round(sorted(per)[int(0.9 * (len(per) - 1))], 5)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.name, args.algo),
                     "kernel": "agmm_persistent (fused)" if args.algo == "fused" else
                               "agmm_copy + agmm_persistent (gemm only)",
                     "per_launch_flops": 2.0 * w.M * w.N * w.K,
                     "avg_launch_ms": round(avg_ms, 5)},
    }
    kr = kernel_resources()
    cfg = r["config"]
    lk = w.layout == "k_contiguous"
    res["kernel_resources"] = {
        "code_object_sha256": kr["code_object_sha256"] if kr else None,
        "fused": kernel_entry(kr, cfg["block_m"], w.dtype, True, lk, cfg["row_wait"]),
        "baseline_gemm": kernel_entry(kr, cfg["block_m"], w.dtype, False, True, False)}
    if not args.no_cpu_baseline:   # before the extras reuse the output buffer
        res["cpu_baseline"] = cpu_baseline(w, r["inputs"], r["dev"].out, args.cpu_seconds)
    if not args.no_extras:
        # the other algorithm, timed interleaved with this one (runs alternating on one
        # stream), so the ratio does not depend on which ran first
        other = "baseline" if args.algo == "fused" else "fused"
        pipes = [(f"pipelined_{S}", "pipelined", {"pipeline_chunks": S}) for S in (2, 4, 8)]
        med, cfgs, _, _ = interleaved(w, [args.algo, other] + pipes, args.steps, args.warmup,
                                      torch, A, inputs=r["inputs"], dev=r["dev"], **tun)
        mb = med[other]
        res[f"{other}_variant"] = {"median_ms": round(mb, 5),
                                   "tflops": round(tflops(w.M, w.N, w.K, mb / 1e3), 3),
                                   "interleaved_median_ms_this": round(med[args.algo], 5),
                                   "fused_speedup": round((mb / med[args.algo])
                                                          if other == "baseline" else
                                                          (med[args.algo] / mb), 3)}
        if args.algo == "fused":
            bops = standalone_ops(w, A, tun)
            bt = block_times(w, bops, r["dev"], torch, 6, 10)
            ct = cold_times(bops[:2], r["dev"], torch, 10)
            res["standalone"] = {"fused_ms": round(bt["fused"], 5),
                                 "baseline_ms": round(bt["baseline"], 5),
                                 "fused_speedup": round(bt["baseline"] / bt["fused"], 3),
                                 "fetch_kernel_ms": round(bt["fetch_kernel"], 5),
                                 "cold_fused_ms": round(ct["fused"], 5),
                                 "cold_baseline_ms": round(ct["baseline"], 5)}
            res["clock"] = clock_under_load(bops[0][1], r["dev"], torch)
            for _, op in bops:
                op.close()
            res["baseline_parts"] = baseline_parts(w, r["dev"], torch, A)
        ym = yardstick_matmul(w, r["dev"], args.steps, args.warmup, torch)
        res["yardstick_torch_matmul_pregathered"] = {
            "median_ms": round(ym, 5), "tflops": round(tflops(w.M, w.N, w.K, ym / 1e3), 3)}
        res["gather_a_variant"] = gather_variant(w, r["dev"], args.steps, args.warmup, torch, A)
        res["gemm_allreduce_variant"] = gemm_allreduce_variant(w, args.steps, args.warmup, torch, A)
        # the host stream pipeline (chunked copy + GEMM-only kernels rotating over 4
        # streams), from the same interleaved runs
        pv = {f"chunks_{cfgs[n]['pipeline_chunks']}_median_ms": round(med[n], 5)
              for n, _, _ in pipes}
        fused_med = med["fused"]
        pv["fused_speedup_vs_best"] = round(min(med[n] for n, _, _ in pipes) / fused_med, 3)
        res["pipelined_variant"] = pv
        # staging traffic of the fused step: 2 * (staged rows) * K * 2 bytes (read + write)
        staged_bytes = 2 * (w.M - (w.M_s if w.direct_local else 0)) * w.K * 2
        res["staging"] = {"bytes_per_step": staged_bytes,
                          "gbs_over_step": round(staged_bytes / (avg_ms / 1e3) / 1e9, 1),
                          "peak_gbs": PEAK_HBM_GBS}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
