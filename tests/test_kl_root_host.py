"""The exact-KL Cactus gamma* solver and divergence of the HIP source, compiled for the host,
against the oracle over a wide grid of (c, delta): candidate probabilities from 1e-300 to
1 - 1e-12, budgets from 1e-300 to 700, both clip edges.  No GPU is touched."""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_sampling_verification_row_amd", "csrc")


@pytest.fixture(scope="module")
def solver(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("kl") / "kl_root_check")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "hip", os.path.join(ROOT, "tests", "kl_root_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]

    def run(pairs, mode=None):
        text = "".join(f"{float(c).hex()} {float(d).hex()}\n" for c, d in pairs)
        argv = [exe] + ([mode] if mode else [])
        out = subprocess.run(argv, input=text, capture_output=True, text=True, check=True).stdout.split("\n")
        got = [ln.split() for ln in out if ln.strip()]
        assert len(got) == len(pairs)
        if mode == "div":
            return np.array([float.fromhex(g[0]) for g in got])
        return np.array([float.fromhex(g) for g, _ in got]), np.array([int(s) for _, s in got])
    return run


def grid():
    rng = np.random.default_rng(20)
    cs = list(10.0 ** rng.uniform(-300, 0, 200)) + list(rng.uniform(0, 1, 200)) + \
        [1e-300, 1e-30, 1e-8, 0.5, 1 - 1e-6, 1 - 1e-12, 0.0, 1.0]
    pairs = []
    for c in cs:
        for d in [1e-300, 1e-30, 1e-12, 1e-6, 1e-3, 0.02, 0.3, 1.0, 3.0, 40.0, 700.0,
                  float(10 ** rng.uniform(-8, 1))]:
            pairs.append((min(c, 1.0), d))
    # budgets just below and at the clip edge -ln c
    for c in [1e-5, 0.01, 0.3, 0.9, 0.999]:
        e = -math.log(c)
        pairs += [(c, e), (c, e * (1 - 1e-9)), (c, e * (1 - 1e-3))]
    return pairs


def test_solver_matches_oracle_bisection(solver):
    pairs = grid()
    got, steps = solver(pairs)
    ref = np.array([oracle.cactus_gamma_star_kl(c, d) for c, d in pairs])
    cs = np.array([c for c, _ in pairs])
    # a few ulps, or 1e-13 of the smaller of gamma and 1 - gamma (the scale of the other tokens
    # is (1 - gamma) / (1 - c)), or a tiny fraction of the gap gamma - c
    tol = 8 * np.spacing(np.maximum(ref, 1e-300)) + 1e-13 * np.minimum(ref, 1.0 - ref) + 1e-12 * (ref - cs)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), [(pairs[i], got[i], ref[i]) for i in np.flatnonzero(bad)[:5]]
    assert np.all((got >= cs) & (got <= 1.0))
    # the steps stay few: Newton from the Taylor start, bisection only as a fallback
    assert steps.max() <= 60, steps.max()
    assert np.median(steps[steps > 0]) <= 8


def test_solver_edges(solver):
    got, steps = solver([(0.3, 0.0), (0.0, 1.0), (1.0, 0.2), (0.5, math.log(2.0)), (0.5, 0.69)])
    assert got[0] == 0.3 and got[1] == 0.0 and got[2] == 1.0 and got[3] == 1.0
    assert 0.5 < got[4] < 1.0
    assert steps[:4].max() == 0


def test_divergence_matches_oracle(solver):
    """kl_divergence (the accept test's divergence of r pd(n)) against the oracle's, g in [c, 1)."""
    rng = np.random.default_rng(21)
    pairs = []
    for _ in range(3000):
        c = float(10 ** rng.uniform(-300, 0)) * 0.9999
        if rng.random() < 0.5:
            g = c * (1.0 + float(10 ** rng.uniform(-14, 3)))
        else:
            g = c + (1.0 - c) * float(rng.random())
        if g < 1.0:
            pairs.append((g, c))
    pairs += [(0.5, 0.5), (0.3, 0.1), (1 - 1e-12, 0.5), (0.9999999, 0.9999)]
    got = solver(pairs, "div")
    ref = np.array([oracle.cactus_kl(g, c) for g, c in pairs])
    assert np.all(np.abs(got - ref) <= 1e-13 * ref + 1e-300), np.max(np.abs(got - ref) / np.maximum(ref, 1e-300))
