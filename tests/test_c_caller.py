"""librlscan from plain C: ``c_caller.c`` includes only ``include/rlscan.h``
and the HIP runtime API, is compiled as C11 by gcc (so the header must be
valid C, not only C++) and linked against ``librlscan.so`` and the oracle's C
source.

* ``checks`` (CPU): version and status strings, ``rlscan_plan``, and the
  status codes of invalid calls, which are refused before anything is
  enqueued.
* ``gpu``: hipMalloc'd buffers and calls on a stream the program creates --
  GAE on 64 x 512 (the README's usage shape), GAE with truncation on
  5 x 300001 (look-back, ragged tail), the prefix sum on 3 x 700001 and one
  ``rlscan_group`` launch -- compared with the float64 oracle to
  1e-4 * (1 + |ref|), the integer prefix sum exactly.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "linear_recurrence_scan_coefficient_amd")
LIB = os.path.join(PKG, "librlscan.so")
ROCM = "/opt/rocm"


@pytest.fixture(scope="module")
def c_caller(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    if not os.path.exists(LIB):
        pytest.fail("librlscan.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path_factory.mktemp("c_caller") / "c_caller")
    cmd = [gcc, "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_caller.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-o", exe, "-L", PKG, "-lrlscan", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-lm", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    return exe


def _run(exe, mode, timeout):
    run = subprocess.run([exe, mode], capture_output=True, text=True, timeout=timeout)
    print(run.stdout)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert run.stdout.strip().splitlines()[-1] == f"ok {mode}"


def test_c_caller_host_checks(c_caller):
    _run(c_caller, "checks", 120)


@pytest.mark.gpu
def test_c_caller_on_gpu(c_caller):
    _run(c_caller, "gpu", 300)
