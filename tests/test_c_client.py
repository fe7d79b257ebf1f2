"""The public header is plain C: a C99 program compiled with gcc against
include/adaln.h links libadaln.so and calls its host-only entry points."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c99_client(tmp_path):
    import adaln_fwd_amd as A
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    libdir = os.path.dirname(A.LIB_PATH)
    exe = tmp_path / "abi_client"
    subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
         "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "tests", "c", "abi_client.c"),
         "-L", libdir, "-ladaln", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
        check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count("ok:") >= 17
