"""Compile libspecverify.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m speculative_sampling_verification_row_amd.build [--asm]

Flags: -O3 for gfx950 only; packed-fp32 instructions are disabled
(-target-feature -packed-fp32-ops) so the compiler never emits them.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = [os.path.join(CSRC, "spec_verify.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def common_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source into one shared library; returns its path."""
    tmp = out + ".tmp"
    cmd = [hipcc()] + common_flags() + [f"-D{d}" for d in defines] + ["-shared"] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


def dump_asm(out_dir: str) -> None:
    """Device assembly and register usage of the kernels (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    cmd = [hipcc()] + common_flags() + ["--cuda-device-only", "-S", SOURCES[0], "-o",
                                        os.path.join(out_dir, "spec_verify.s"),
                                        "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    sys.stdout.write(res.stderr)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed")


if __name__ == "__main__":
    if "--asm" in sys.argv:
        dump_asm(os.path.join(ROOT, "_work", "asm"))
    else:
        print(build(verbose=True))
