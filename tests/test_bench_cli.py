"""bench.py's command-line contract on a host without a GPU.

More than one GPU is refused with exit status 2 and a message before anything touches a
device; with no GPU visible the run stops with status 1 and says so, printing no JSON line.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT, env=env)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _bench("--gpus", n)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_visible_stops_without_a_result_line():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    r = _bench("--steps", "1", "--warmup", "0", env=env)
    assert r.returncode == 1, (r.returncode, r.stderr[-2000:])
    assert "no GPU visible" in r.stderr
    assert r.stdout.strip() == ""
