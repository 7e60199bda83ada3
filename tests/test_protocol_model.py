"""The fetch/flag protocol as a CPU thread model (tests/protocol_model.cpp) under
ThreadSanitizer: the protocol as built (release publish, relaxed polls, one acquire) runs
race-free and every read sees the current run's data, also with fetchers delayed at random; a
dropped publish surfaces as a bounded-wait timeout on exactly that unit; a double publish is
detected (the flag passes the epoch); and the same model with a relaxed publish and no
acquire is reported as a data race, which shows the check can see one."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("protocol") / "protocol_model")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
           os.path.join(HERE, "protocol_model.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


def _run(exe, mode):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=0 exitcode=66 report_signal_unsafe=0")
    return subprocess.run([exe, mode], capture_output=True, text=True, timeout=120, env=env)


@pytest.mark.parametrize("mode", ["ok", "delay"])
def test_protocol_race_free_and_fresh(model, mode):
    r = _run(model, mode)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ThreadSanitizer" not in r.stderr
    assert "timeouts=0 over_epoch=0 stale=0" in r.stdout


def test_dropped_publish_times_out(model):
    r = _run(model, "drop")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "timeouts=1 over_epoch=0 stale=0" in r.stdout
    assert "ThreadSanitizer" not in r.stderr


def test_double_publish_is_detected(model):
    r = _run(model, "double")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "over_epoch=1" in r.stdout


def test_relaxed_protocol_is_reported_as_a_race(model):
    r = _run(model, "race")
    assert r.returncode == 66, r.stdout + r.stderr       # TSan's exit code for a report
    assert "WARNING: ThreadSanitizer: data race" in r.stderr
