"""Compile libspecverify.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m speculative_sampling_verification_row_amd.build [--asm OUT_DIR]

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
# the streaming-read probe that measures the read ceiling (a library of its own)
PROBE_LIB = os.path.join(PKG, "libstreamprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "stream_probe.hip")]
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
    """Compile the verification library (and the streaming-read probe beside it); returns
    the verification library's path."""
    path = _build_one(SOURCES, out, defines, verbose)
    if out == LIB:
        _build_one(PROBE_SOURCES, PROBE_LIB, (), verbose)
    return path


def _build_one(sources, out, defines, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc()] + common_flags() + [f"-D{d}" for d in defines] + ["-shared"] + sources + ["-o", tmp]
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
        i = sys.argv.index("--asm")
        if i + 1 >= len(sys.argv):
            raise SystemExit("--asm needs an output directory")
        dump_asm(sys.argv[i + 1])
    else:
        print(build(verbose=True))
