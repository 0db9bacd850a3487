"""Workspace-layout invariant, checked on the host (no GPU): the region that must be
zero at launch depends on B and K only, so one workspace serves every V of a (B, K)
without being cleared again; it holds every unit a call can publish; and the layout
fits in spec_workspace_bytes.  (A queue sized by V once let stale scratch of a
smaller-V call be read as queue entries.)"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_sampling_verification_row_amd", "csrc")


def test_zero_region_is_independent_of_V(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "layout_check")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", exe, "-x", "hip"]
    # the source must be compiled as HIP (it includes the kernel file)
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "hip", os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 violations" in out.stdout
