"""The C ABI from plain C (CPU only): include/qknorm.h compiles as C99 with
warnings as errors, links against libqknorm.so, and its calls behave as
documented without a GPU (ABI version, plan description, argument errors)."""

import os
import shutil
import subprocess

import pytest

import layerwise_qk_norm_qknorm_amd as qk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_and_library_from_c(tmp_path):
    lib = qk.library_path()
    assert os.path.exists(lib), "build the library first"
    exe = tmp_path / "abi_from_c"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", str(exe), lib,
           "-Wl,-rpath," + os.path.dirname(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan: fused bf16 path=16B" in r.stdout and "error: qknorm_fused:" in r.stdout
