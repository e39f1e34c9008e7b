"""Host-side check of how the row pass splits a position's tiles over its
workgroups (ranges, record slots); see
tests/host/flat_split_check.cpp.  Runs on the CPU: the checked functions are
host-callable and the program is built without device code."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_flat_split_invariants(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    exe = tmp_path / "flat_split_check"
    cmd = [hipcc, "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "rejection_sampling_verify_sv_amd", "csrc"),
           "-o", str(exe), os.path.join(HERE, "host", "flat_split_check.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, cwd=str(tmp_path))
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok")
