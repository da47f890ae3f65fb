"""include/kda.h from plain C: tests/c_abi_client.c is compiled with gcc (as C99, host only) and
linked against libkda.so and the HIP runtime.  Without a GPU it only runs far enough to print the
library version; on a GPU it runs a prefill, checks the state hand-off between two calls, a
decode step and two rejected calls."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "gated_delta_rule_94_amd")
ROCM_LIB = "/opt/rocm/lib"


def build_client(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libkda.so")):
        pytest.skip("libkda.so not built")
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM_LIB, "libamdhip64.so")):
        pytest.skip("gcc or the HIP runtime library is missing")
    exe = str(tmp_path / "c_abi_client")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Werror", os.path.join(ROOT, "tests", "c_abi_client.c"),
           "-I", os.path.join(ROOT, "include"), "-L", LIBDIR, "-lkda", "-L", ROCM_LIB, "-lamdhip64", "-lm",
           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + ROCM_LIB, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_client_builds_and_loads(tmp_path):
    exe = build_client(tmp_path)
    r = subprocess.run([exe, "--version"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "libkda version" in r.stdout


@pytest.mark.gpu
def test_c_client_runs(tmp_path):
    exe = build_client(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c client ok" in r.stdout
