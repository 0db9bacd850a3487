"""The C ABI library loads and exports every function include/spec_verify.h declares;
argument validation returns the documented status codes before any launch.

Runs without a GPU: only host-side calls are made (status strings, workspace
sizes, and calls whose arguments are rejected before anything is launched).
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
LIB = os.path.join(ROOT, "speculative_sampling_verification_row_amd", "libspecverify.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libspecverify.so is not built (run __graft_entry__.build())")
    from speculative_sampling_verification_row_amd import binding
    return binding.load(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["spec_verify", "spec_cactus_verify", "spec_cactus_kl_verify", "spec_counterfactual_gamma",
              "spec_tree_gamma", "spec_tree_workspace_bytes", "hedge_update", "hedge_exp_update",
              "spec_acceptance_loss", "hedge_queue_update", "hedge_censored_update",
              "spec_workspace_bytes", "spec_workspace_init", "spec_status_str"]:
        assert n in names, names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in [0, -1, -2, -3, -4, -5, -6, -7]:
        assert lib.spec_status_str(code)
    assert lib.spec_status_str(0) == b"ok"


def test_workspace_bytes_layout(lib):
    assert lib.spec_workspace_bytes(0, 5, 1) == 0
    a = lib.spec_workspace_bytes(64, 5, 1)
    b = lib.spec_workspace_bytes(64, 8, 21)
    assert a % 256 == 0 and b % 256 == 0 and b > a
    # statistics words of 2K+1 rows x 64 slices x 4 waves + draw slice totals (64 readers x 64 slices)
    assert a >= 8 * 64 * 11 * 64 * 4 + 8 * 64 * 64 * 64
    # gamma: (K+1 + N K) rows of statistics words + gamma partial sums (K N x 64 slices x 4 waves)
    assert b >= 8 * 64 * (9 + 21 * 8) * 64 * 4 + 8 * 64 * 8 * 21 * 64 * 4


P = ctypes.c_void_p


def fake(addr):
    return P(addr)


def verify_args(**kw):
    a = dict(target=fake(4096), ts=128, draft=fake(8192), ds=128, tok=fake(256), r=fake(512), u=fake(768),
             B=2, K=3, V=100, T=1.0, A=fake(1024), o=fake(1280), m=None, ws=fake(1 << 20), wsb=16,
             stream=None)
    # wsb=16 is always too small, so even a call whose other arguments are all valid is
    # rejected (SPEC_ERR_WORKSPACE) before anything could be launched on these fake pointers.
    a.update(kw)
    return a


def call_verify(lib, a):
    return lib.spec_verify(a["target"], a["ts"], a["draft"], a["ds"], a["tok"], a["r"], a["u"], a["B"], a["K"],
                           a["V"], a["T"], a["A"], a["o"], a["m"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(K=0), -2), (dict(K=65), -2), (dict(V=0), -2), (dict(V=(1 << 20) + 1), -2),
    (dict(T=0.0), -3), (dict(T=-1.0), -3), (dict(T=float("inf")), -3), (dict(T=float("nan")), -3),
    (dict(target=None), -1), (dict(draft=None), -1), (dict(tok=None), -1), (dict(A=None), -1),
    (dict(ts=99), -2), (dict(ts=100), -2), (dict(ds=50), -2),
    (dict(target=fake(4098)), -4), (dict(draft=fake(8200)), -4),
    (dict(ws=None), -5), (dict(ws=fake((1 << 20) + 8)), -5), (dict(), -5),
])
def test_verify_validation(lib, kw, code):
    assert call_verify(lib, verify_args(**kw)) == code


def test_cactus_validation(lib):
    a = verify_args()
    args = [a["target"], a["ts"], a["draft"], a["ds"], a["tok"], a["r"], a["u"], a["B"], a["K"], a["V"]]
    tail = [a["A"], a["o"], None, None, a["ws"], a["wsb"], None]
    assert lib.spec_cactus_verify(*args, -0.5, 1.0, *tail) == -3
    assert lib.spec_cactus_verify(*args, float("nan"), 1.0, *tail) == -3
    assert lib.spec_cactus_verify(*args, 0.5, 0.0, *tail) == -3
    for delta, T, code in [(-0.5, 1.0, -3), (float("nan"), 1.0, -3), (float("inf"), 1.0, -3), (0.5, 0.0, -3),
                           (0.5, 1.0, -5)]:   # the last: valid, rejected only by the tiny workspace
        assert lib.spec_cactus_kl_verify(*args, delta, T, *tail) == code


def test_gamma_validation(lib):
    def call(**kw):
        a = dict(t=fake(4096), ts=128, tr=3, d=fake(8192), ds=128, dstr=128 * 6, traj=fake(256), B=2, K=3,
                 N=4, V=100, T=1.0, g=fake(512), e=fake(768), l=fake(1024), sel=None, tok=None, r=None,
                 u=None, A=None, o=None, m=None, ws=fake(1 << 20), wsb=64)  # wsb too small: never launches
        a.update(kw)
        return lib.spec_counterfactual_gamma(a["t"], a["ts"], a["tr"], a["d"], a["ds"], a["dstr"], a["traj"],
                                             a["B"], a["K"], a["N"], a["V"], a["T"], a["g"], a["e"], a["l"],
                                             a["sel"], a["tok"], a["r"], a["u"], a["A"], a["o"], a["m"], a["ws"],
                                             a["wsb"], None)
    assert call(N=0) == -2 and call(N=65) == -2
    assert call(tr=2) == -2                       # fewer target rows than K
    assert call(sel=fake(64), tok=fake(64), r=fake(64), u=fake(64), A=fake(64), o=fake(64)) == -2  # fused needs K+1
    assert call(sel=fake(64)) == -1               # fused without its buffers
    assert call(dstr=130) == -2 and call(dstr=0) == -2
    assert call(g=None) == -1 and call(traj=None) == -1
    assert call(wsb=64) == -5


def test_hedge_validation(lib):
    ok = [fake(4096), fake(8192), fake(1024), None, 0.2, None, None, 4, 7, None]  # never called as is
    bad_n = list(ok)
    bad_n[8] = 65
    assert lib.hedge_update(*bad_n) == -2
    bad_scale = list(ok)
    bad_scale[4] = float("nan")
    assert lib.hedge_update(*bad_scale) == -3
    no_sel = list(ok)
    no_sel[5] = fake(64)
    assert lib.hedge_update(*no_sel) == -1
    no_state = list(ok)
    no_state[0] = None
    assert lib.hedge_update(*no_state) == -1


def test_product_path_refuses_without_library(tmp_path):
    from speculative_sampling_verification_row_amd import binding
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            binding.load(str(tmp_path / "missing.so"))
    finally:
        binding._lib = saved


def test_package_imports_no_oracle():
    import subprocess
    import sys
    code = ("import sys; import speculative_sampling_verification_row_amd as p; "
            "from speculative_sampling_verification_row_amd import binding, inputs, hedge; "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)


def test_tree_workspace_and_validation(lib):
    assert lib.spec_tree_workspace_bytes(4, 5, 7, 1000, 0) == 0 and lib.spec_tree_workspace_bytes(4, 5, 7, 1000, 65) == 0
    assert lib.spec_tree_workspace_bytes(4, 5, 7, 0, 8) == 0 and lib.spec_tree_workspace_bytes(4, 5, 7, (1 << 20) + 1, 8) == 0
    a = lib.spec_tree_workspace_bytes(32, 5, 7, 128256, 8)
    # records: 32 pieces of 4096 tokens x 8 per row; statistics words of the K target rows
    assert a % 256 == 0 and a >= 8 * 32 * 5 * 7 * 32 * 8 + 8 * 32 * 5 * 64 * 4
    assert lib.spec_tree_workspace_bytes(32, 5, 7, 128256, 16) > a
    assert lib.spec_tree_workspace_bytes(32, 5, 7, 1000, 8) < a

    def call(**kw):
        a = dict(t=fake(4096), ts=128, tr=3, d=fake(8192), ds=128, dstr=128 * 6, B=2, K=3, N=4, V=100, topk=8,
                 T=1.0, g=fake(512), ws=fake(1 << 20), wsb=64)   # wsb too small: never launches
        a.update(kw)
        return lib.spec_tree_gamma(a["t"], a["ts"], a["tr"], a["d"], a["ds"], a["dstr"], a["B"], a["K"], a["N"],
                                   a["V"], a["topk"], a["T"], a["g"], a["ws"], a["wsb"], None)
    assert call(topk=0) == -3 and call(topk=65) == -3
    assert call(N=0) == -2 and call(tr=2) == -2 and call(ds=50) == -2 and call(dstr=130) == -2
    assert call(g=None) == -1 and call(t=None) == -1
    assert call(T=0.0) == -3
    assert call(d=fake(8200)) == -4
    assert call() == -5


def test_hedge_exp_and_loss_validation(lib):
    ok = [fake(4096), fake(8192), fake(1024), None, 0.2, 0.5, None, None, 4, 7, None]  # never called as is
    for pos, val, code in [(9, 65, -2), (8, 0, -2), (4, float("nan"), -3), (5, -1.0, -3), (5, float("inf"), -3),
                           (0, None, -1), (2, None, -1), (6, fake(64), -1)]:
        a = list(ok)
        a[pos] = val
        assert lib.hedge_exp_update(*a) == code, (pos, val)
    assert lib.spec_acceptance_loss(fake(64), fake(128), 0, 5, 7, None) == -2
    assert lib.spec_acceptance_loss(fake(64), fake(128), 2, 65, 7, None) == -2
    assert lib.spec_acceptance_loss(None, fake(128), 2, 5, 7, None) == -1


def test_hedge_censored_validation(lib):
    P_ = fake(4096)
    # state, weights, qloss, qtok, round, loss, alen, K, learner, eta, scale, v, sel, hist, B, N, Q, T, stream
    base = [P_, P_, P_, P_, P_, P_, P_, 5, 0, 0.0, 0.2, P_, P_, P_, 4, 7, 6, 100, None]  # never called as is
    for pos, val, code in [(14, 0, -2), (15, 65, -2), (7, 0, -2), (7, 65, -2), (16, 5, -2), (16, 257, -2),
                           (17, 0, -2), (8, 2, -3), (9, -1.0, -3), (9, float("inf"), -3), (10, float("nan"), -3),
                           (0, None, -1), (6, None, -1), (11, None, -1), (13, None, -1)]:
        a = list(base)
        a[pos] = val
        assert lib.hedge_censored_update(*a) == code, (pos, val)


def test_hedge_queue_validation(lib):
    P_ = fake(4096)
    base = [P_, P_, P_, P_, P_, P_, P_, 0.2, P_, P_, P_, 4, 7, 12, 100, None]  # never called as is
    for pos, val, code in [(11, 0, -2), (12, 65, -2), (13, 1, -2), (13, 257, -2), (14, 0, -2), (7, float("nan"), -3),
                           (0, None, -1), (4, None, -1), (10, None, -1)]:
        a = list(base)
        a[pos] = val
        assert lib.hedge_queue_update(*a) == code, (pos, val)
