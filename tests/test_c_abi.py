"""The C ABI from plain C: tests/c_abi/abi_check.c is compiled with gcc against
include/flashblock.h, linked to the built library, and run (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

import cached_kv_prefix_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_c_program_uses_the_abi(tmp_path):
    lib_dir = os.path.dirname(fb.LIB_PATH)
    assert os.path.exists(fb.LIB_PATH), "build the library first"
    exe = str(tmp_path / "abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), "-L", lib_dir, "-lflashblock",
           "-Wl,-rpath," + lib_dir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout
