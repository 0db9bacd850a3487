"""Workspace-layout invariant, checked on the host (no GPU): every region a call
indexes with its own slice and sub-tile counts stays inside its region, regions do
not overlap, and the layout fits in spec_workspace_bytes for every V.  (A region
sized by V once let one call read another call's leftovers.)  Also the static
schedules: the phase-0 split deals each slice once, and the gamma row chunks make
every row a job of exactly one slot with its target row before it."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_sampling_verification_row_amd", "csrc")


def test_workspace_regions_fit_every_shape(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "layout_check")
    # the source must be compiled as HIP (it includes the kernel file)
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "hip", os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "layouts, 0 violations" in out.stdout
    assert "schedules, 0 violations" in out.stdout
    assert "row-chunk partitions, 0 violations" in out.stdout
