"""CPU-only checks of the C-ABI library: it loads, exports every function include/agmm.h
declares, and its host-side logic (defaults, validation, workspace sizing, error strings)
behaves as documented. Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "all_gather_gemm_amd", "libagmm.so")


@pytest.fixture(scope="module")
def A():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "agmm_build", os.path.join(ROOT, "all_gather_gemm_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import all_gather_gemm_amd
    return all_gather_gemm_amd


def header_functions():
    with open(os.path.join(ROOT, "include", "agmm.h")) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ag_(?:matmul|gemm_ar)_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(A):
    names = header_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in agmm.h but not exported"
    assert set(names) == set(A.EXPORTED)


def test_desc_defaults(A):
    d = A.ag_matmul_desc_init()
    assert (d.D, d.rank, d.dtype, d.layout, d.algo, d.direct_local, d.has_bias, d.debug) == \
        (1, 0, A.F16, A.K_CONTIGUOUS, A.ALGO_FUSED, 1, 0, 0)
    assert d.debug_skip_unit == -1 and d.block_m == 0 and d.spin_limit == 0


def test_strerror(A):
    assert A.strerror(0) == "ok"
    for code in range(-7, 0):
        assert A.strerror(code) and A.strerror(code) != "unknown error code"
    assert A.strerror(-99) == "unknown error code"


def _ws(A, **kw):
    return A.ag_matmul_workspace_bytes(A.ag_matmul_desc_init(**kw))


def test_validation_errors(A):
    INV, UNS = -1, -2
    assert _ws(A, D=0, M=8, N=8, K=8) == INV
    assert _ws(A, D=65, M=65 * 8, N=8, K=8) == INV
    assert _ws(A, D=2, rank=2, M=8, N=8, K=8) == INV
    assert _ws(A, D=3, M=8, N=8, K=8) == INV            # M % D
    assert _ws(A, D=1, M=-1, N=8, K=8) == INV
    assert _ws(A, D=1, M=8, N=12, K=8) == UNS          # N % 8
    assert _ws(A, D=1, M=8, N=8, K=12) == UNS          # K % 8
    assert _ws(A, D=2, M=2 * 5, N=8, K=8, layout=A.M_CONTIGUOUS) == UNS  # M % 8
    assert _ws(A, D=1, M=8, N=8, K=8, block_m=96) == INV
    assert _ws(A, D=1, M=8, N=8, K=8, dtype=2) == INV
    assert _ws(A, D=1, M=1 << 23, N=8, K=8) == UNS
    assert _ws(A, D=1, M=8, N=1 << 22, K=8) == UNS        # 256 output rows past 2^31 bytes
    assert _ws(A, D=1, M=8, N=8, K=1 << 22) == UNS        # 256 K-major rows likewise
    assert _ws(A, D=1, M=8, N=(1 << 22) - 8, K=(1 << 22) - 8) > 0
    assert _ws(A, D=1, M=8, N=8, K=8, has_bias=2) == INV
    assert _ws(A, D=1, M=8, N=8, K=8, tail_split=2) == INV
    assert _ws(A, D=1, M=8, N=8, K=8, gather_a=2) == INV
    assert _ws(A, D=1, M=8, N=8, K=8, fetch_kernel=2) == INV
    assert _ws(A, D=1, M=8, N=8, K=8, fetch_kernel=-2) == INV
    assert _ws(A, D=2, M=16, N=8, K=8, fetch_kernel=1) > 0
    assert _ws(A, D=2, M=16, N=8, K=8, fetch_kernel=-1) > 0
    # a queue entry holds the tile id in 24 bits: 4096 x 4096 tiles of 64 fit, 4097 x 4096 not
    assert _ws(A, D=1, M=(1 << 18) + 64, N=1 << 18, K=8, block_m=64) == UNS
    assert _ws(A, D=1, M=1 << 18, N=1 << 18, K=8, block_m=64) > 0
    assert _ws(A, D=2, M=16, N=8, K=8, gather_a=1, layout=A.M_CONTIGUOUS) == UNS
    assert _ws(A, D=1, M=8, N=8, K=8, algo=3) == INV
    assert _ws(A, D=1, M=8, N=8, K=8, algo=A.ALGO_PIPELINED, pipeline_chunks=-1) == INV
    assert _ws(A, D=1, M=8, N=8, K=8, algo=A.ALGO_PIPELINED, pipeline_chunks=65) == INV
    # create rejects before touching a device
    with pytest.raises(A.AgmmError) as e:
        A.ag_matmul_create(A.ag_matmul_desc_init(D=0))
    assert e.value.code == INV
    # NULL handles
    assert A.ag_matmul_destroy(None) == 0
    assert A.lib.ag_matmul_run(None, None, None, None, None, None) == INV
    assert A.lib.ag_matmul_run_gather(None, None, None, None, None, None, None) == INV


def test_workspace_bytes_large(A):
    # 16384x3584x8192, D=8, tile 256 (sized for 256 compute units), k-groups of 512 columns
    # (the default once K >= 4096, so G = 16): staging M*K fp16, flags T_m*G, counters (a done word and status words, the fetch-piece counter and 9 queue
    # counters, each on its own 128-byte line), 128 split-tile counters (896 tiles = 3 rounds of 256 + 128, split in 2 along
    # K), 56 staged m-tiles x 16 k-groups of 8-byte unit records, 64 m-tile records, 768 + 2 *
    # 128 queue entries, 2 * 128 fp32 partial tiles; 256-byte aligned pieces.
    al = lambda x: (x + 255) & ~255
    exp = (al(16384 * 8192 * 2) + al(64 * 16 * 4) + al((96 + 9 * 32) * 4) + al(128 * 4)
           + al(56 * 16 * 8) + al(64 * 4) + al(1024 * 4) + al(256 * 256 * 256 * 4) + 0 + al(4))
    got = _ws(A, D=8, M=16384, N=3584, K=8192, block_m=256, layout=A.M_CONTIGUOUS, has_bias=1,
              tail_split=1)
    assert got == exp
    # direct_local off: all 64 m-tiles staged
    got2 = _ws(A, D=8, M=16384, N=3584, K=8192, block_m=256, direct_local=0, tail_split=1)
    assert got2 - got == al(64 * 16 * 8) - al(56 * 16 * 8)
    # no tail split (the default): no counters, partial slots or extra queue entries
    got3 = _ws(A, D=8, M=16384, N=3584, K=8192, block_m=256, layout=A.M_CONTIGUOUS, has_bias=1)
    assert got - got3 == al(128 * 4) - al(4) + al(1024 * 4) - al(896 * 4) + al(256 * 256 * 256 * 4)
    # D=1 with direct reads: nothing staged, no staging buffer
    assert _ws(A, D=1, M=1024, N=1024, K=1024, block_m=128) < 1 << 16
    # gather_a: the caller's buffer is the staging (none in the workspace), and the local
    # shard's 8 m-tiles x 16 k-groups join the unit records
    got4 = _ws(A, D=8, M=16384, N=3584, K=8192, block_m=256, gather_a=1)
    got5 = _ws(A, D=8, M=16384, N=3584, K=8192, block_m=256)
    assert got5 - got4 == al(16384 * 8192 * 2) + al(56 * 16 * 8) - al(64 * 16 * 8)
    # the host stream pipeline (4 chunks): a counter block per chunk, and the chunk tables
    # (896 staged units of 2 words, 64 m-tiles, 896 queue entries)
    got6 = _ws(A, D=8, M=16384, N=3584, K=8192, block_m=256, algo=A.ALGO_PIPELINED)
    assert got6 - got5 == al(4 * (96 + 9 * 32) * 4) + al(896 * 2 * 4) + al(64 * 4) + al(896 * 4)


def test_struct_layout_matches_header(A, tmp_path):
    """The ctypes mirrors of agmm_desc / agmm_config / agmm_trace_rec have the C layout:
    compile a probe against include/agmm.h with the host C compiler and compare offsets."""
    import subprocess
    structs = {"agmm_desc": A.agmm_desc, "agmm_config": A.agmm_config,
               "agmm_trace_rec": A.agmm_trace_rec}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "agmm.h"', "int main(void){"]
    for sname, cls in structs.items():
        lines.append(f'printf("{sname} size %zu\\n", sizeof({sname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{sname} {f} %zu\\n", offsetof({sname}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line.strip():
            sname, f, v = line.split()
            got[(sname, f)] = int(v)
    for sname, cls in structs.items():
        assert got[(sname, "size")] == ctypes.sizeof(cls), sname
        for f, _ in cls._fields_:
            assert got[(sname, f)] == getattr(cls, f).offset, (sname, f)


def test_one_hip_runtime_whatever_the_import_order():
    """The package binds the library to torch's HIP runtime: imported before torch, it must
    not load a second libamdhip64 (the library's calls then report no device while torch's
    work)."""
    import subprocess
    import sys
    code = ("import all_gather_gemm_amd, torch; "
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))), timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip() == "1", r.stdout


def test_planner_defaults_at_the_measured_shapes(A):
    """The planner's automatic choices at the shapes whose timings chose them (256 compute
    units, fp16, N = 3584, K = 8192): tile rows, k-group size in K-tiles of 32, fetchers, wait
    mode."""
    def cfg(**kw):
        return A.ag_matmul_plan_query(A.ag_matmul_desc_init(N=3584, K=8192, **kw), 256)["config"]
    # 16384 rows, 8 shards: 256-row tiles, k-groups of 512 columns, 32 fetchers, per-k-group waits
    c = cfg(D=8, M=16384, layout=A.M_CONTIGUOUS, has_bias=1)
    assert (c.block_m, c.k_per_flag, c.num_fetch_wgs, c.row_wait) == (256, 16, 32, 0)
    # 4096 rows, 4 shards: one round of 224 tiles beside 32 fetchers, k-groups of 256 columns
    c = cfg(D=4, M=4096)
    assert (c.block_m, c.k_per_flag, c.num_fetch_wgs, c.num_tiles) == (256, 8, 32, 224)
    # 1024 rows: one round of 224 tiles of 128 rows, k-groups of 512 columns
    for D in (2, 4, 8):
        c = cfg(D=D, M=1024)
        assert (c.block_m, c.k_per_flag, c.num_fetch_wgs, c.num_tiles) == (128, 16, 32, 224), D
    # the baseline's copy units follow the same k-groups (512 columns once K >= 4096)
    c = cfg(D=8, M=16384, algo=A.ALGO_BASELINE)
    assert c.k_per_flag == 16
