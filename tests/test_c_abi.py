"""The public header is plain C: a C99 program that includes include/fa.h
and links libfa.so builds with -Wall -Wextra -pedantic -Werror and gets the
documented answers from the calls that never reach the device (CPU only)."""
import os
import shutil
import subprocess

import pytest

import io_aware_exact_20_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_client_builds_and_runs(tmp_path):
    lib = fa.LIB_PATH
    if not os.path.exists(lib):
        pytest.fail("libfa.so is not built: %s" % lib)
    exe = str(tmp_path / "c_abi_client")
    libdir = os.path.dirname(lib)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_client.c"), "-o", exe,
                    "-L", libdir, "-l:" + os.path.basename(lib), "-Wl,-rpath," + libdir],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
