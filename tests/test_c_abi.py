"""The library from plain C: tests/c/thd_worked_example.c includes only
include/thd_cp.h and the HIP runtime's C API and runs the worked example of
"Packed Sequence 与上下文并行" §3 through pack, route build, both swaps and the
zigzag roll, comparing with the values that page prints.  The host mode
checks argument handling without a GPU; the gpu mode runs the example.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "context_packed_sequence_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(PKG, "libthdcp.so")):
        pytest.fail("libthdcp.so is not built")
    exe = str(tmp_path / "thd_worked_example")
    cmd = [cc, "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", f"-I{ROOT}/include", f"-I{ROCM}/include",
           "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "c", "thd_worked_example.c"), "-o", exe,
           f"-L{PKG}", "-lthdcp", f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


def test_c_caller_host_checks(tmp_path):
    exe = _build(tmp_path)
    res = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("OK")


@pytest.mark.gpu
def test_c_caller_worked_example(tmp_path):
    exe = _build(tmp_path)
    print("c caller: worked example", flush=True)
    res = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("OK")
