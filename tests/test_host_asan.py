"""The library's host code under AddressSanitizer, on the CPU.

The C ABI's host side (argument checks, the planner and its tables, workspace sizing, the
claim order of the per-tile flag all-reduce) is rebuilt with AddressSanitizer: host code only,
the gfx950 kernels are linked in as built. The host-only tests are then run against that
build: the planner against the schedule model over random problems, the ABI's refusals and
workspace sizes, and the all-reduce claim order. Any out-of-bounds access or use after free
in those paths fails the run. Needs the objects that the regular build leaves in
all_gather_gemm_amd/csrc.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "all_gather_gemm_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
HOST_TESTS = ["test_plan_model.py", "test_ar_flags_order.py", "test_abi.py"]


def _asan_runtime():
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return found[0] if found else None


@pytest.fixture(scope="module")
def asan_pkg(tmp_path_factory):
    objs = [os.path.join(CSRC, "agmm_kernels.o"), os.path.join(CSRC, "agmm_static.o")]
    if not os.path.exists(HIPCC) or _asan_runtime() is None:
        pytest.skip("no hipcc or no AddressSanitizer runtime")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library has not been built here (no kernel objects)")
    d = tmp_path_factory.mktemp("asan")
    pkg = d / "pkg" / "all_gather_gemm_amd"
    pkg.mkdir(parents=True)
    api = str(d / "agmm_api_asan.o")
    # the sanitizer applies to the host pass only (-Xarch_host before each option)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    "-c", os.path.join(CSRC, "agmm_api.cpp"), "-o", api],
                   check=True, capture_output=True, timeout=600)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-o", str(pkg / "libagmm.so"), api] + objs,
                   check=True, capture_output=True, timeout=600)
    shutil.copy(os.path.join(ROOT, "all_gather_gemm_amd", "__init__.py"), pkg)
    return str(d / "pkg")


def _env(pkg):
    return dict(os.environ, LD_PRELOAD=_asan_runtime(),
                ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=77",
                PYTHONPATH=os.pathsep.join([pkg, ROOT]))


def test_asan_build_is_the_one_loaded(asan_pkg):
    r = subprocess.run([sys.executable, "-c",
                        "import all_gather_gemm_amd as A; print(A.LIB_PATH)"],
                       capture_output=True, text=True, timeout=300, env=_env(asan_pkg),
                       cwd=os.path.dirname(asan_pkg))
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().startswith(asan_pkg), r.stdout


def test_host_paths_clean_under_asan(asan_pkg):
    # (run from outside the repository, so that the sanitized package comes first on the path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "--rootdir", ROOT] +
                       [os.path.join(HERE, t) for t in HOST_TESTS],
                       capture_output=True, text=True, timeout=900, env=_env(asan_pkg),
                       cwd=os.path.dirname(asan_pkg))
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
