"""CPU model of the decoupled look-back protocol, run under ThreadSanitizer.

``lookback_model.hip`` is built for the host only: it includes the library's
own status-word code (publish, read, poll decision) and drives it from one
thread per tile, with random interleavings, stale words from an earlier call,
two-word values written one word at a time, the one-word short form and the
tag wrap that clears the status array. Every call's tile prefixes are checked
against a serial scan of the same steps.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "linear_recurrence_scan_coefficient_amd", "csrc")


def _hipcc():
    for path in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if path and os.path.exists(path):
            return path
    return None


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("lookback") / "lookback_model")
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g",
           "-Xarch_host", "-fsanitize=thread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(HERE, "lookback_model.hip"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 second_deadlock_stack=1")
    return subprocess.run([exe, *args], capture_output=True, text=True,
                          timeout=600, env=env)


@pytest.mark.parametrize("seed", [1, 2])
def test_lookback_protocol_under_tsan(model, seed):
    r = _run(model, "--trials", "150", "--seed", str(seed))
    out = r.stdout + r.stderr
    assert "ThreadSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert r.stdout.startswith("ok"), out[-4000:]
    # the trials must have crossed the tag wrap at least once, and some
    # walks must have folded aggregates over more than one window
    assert " 0 tag wraps" not in r.stdout, r.stdout
    assert " 0 walks over several windows" not in r.stdout, r.stdout
