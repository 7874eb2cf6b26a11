"""The C ABI from plain C on the GPU: tests/c_abi/gpu_step.c is compiled with gcc against
include/flashblock.h and HIP only (no PyTorch in the process), then run: a fresh step,
the three passes separately, a reuse step, the threshold rule and a refused call."""
import os
import shutil
import subprocess

import pytest

import cached_kv_prefix_amd as fb
from tests.gpu_util import say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.gpu


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_c_program_runs_a_step(tmp_path):
    lib_dir = os.path.dirname(fb.LIB_PATH)
    assert os.path.exists(fb.LIB_PATH), "build the library first"
    exe = str(tmp_path / "gpu_step")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi", "gpu_step.c"), "-L", lib_dir, "-lflashblock",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    say("[c abi] gpu_step")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=90)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout
