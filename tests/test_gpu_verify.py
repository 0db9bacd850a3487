"""GPU parity: spec_verify, spec_cactus_verify and spec_cactus_kl_verify against the
float64 oracle.

Every case feeds the same seeded bf16 rows, tokens and uniforms to the HIP path
(through the C ABI) and to the oracle, and compares element by element under
the rules of tests/parity.py.
"""

import numpy as np
import pytest
from scipy import stats

import oracle
from speculative_sampling_verification_row_amd import inputs as gen

from gpu_util import banner, bf16_bits_from_f64, dev_bf16, dev_f32, dev_i32
from parity import assert_rel, compare_verify, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def B():
    from speculative_sampling_verification_row_amd import binding
    binding.load()
    return binding


def run_verify(binding, x, T=1.0, delta=None, ws=None, kl=False):
    t, d = dev_bf16(x["target"]), dev_bf16(x["draft"])
    tok, r, u = dev_i32(x["draft_tokens"]), dev_f32(x["r"]), dev_f32(x["u"])
    B_, K1 = x["target"].shape[:2]
    if ws is None:
        ws = binding.make_workspace(B_, K1 - 1, 1)
    if delta is None:
        A, o, m = binding.spec_verify(t, d, tok, r, u, T, workspace=ws)
        g = None
    else:
        fn = binding.spec_cactus_kl_verify if kl else binding.spec_cactus_verify
        A, o, m, g = fn(t, d, tok, r, u, delta, T, workspace=ws)
    torch.cuda.synchronize()
    assert binding.workspace_fault(ws) == 0, "kernel reported an internal consistency fault"
    # every word the call published was cleared by its last reader
    assert int(ws.count_nonzero().item()) == 0, "workspace not left zero"
    return to_np(A), to_np(o), to_np(m), to_np(g)


def oracle_verify(x, T=1.0, delta=None, kl=False):
    if delta is None:
        return oracle.spec_verify(x["target"], x["draft"], x["draft_tokens"], x["r"], x["u"], T)
    return oracle.spec_cactus_verify(x["target"], x["draft"], x["draft_tokens"], x["r"], x["u"], delta, T,
                                     exact_kl=kl)


def sps_case(B_, K, V, seed=0, T=1.0, sigma_t=2.5, sigma_d=0.8, peak=0.01):
    w = gen.SpsWorkload("test", B=B_, K=K, V=V, target_sigma=sigma_t, draft_sigma=sigma_d, peak_frac=peak,
                        temperature=T, config_id=90)
    return gen.make_sps_inputs(w, seed=seed)


def worked_example_rows(Bn, seed):
    """bf16(log p), bf16(log q) of the tutorial's cat/dog/fish example, K = 1."""
    p = np.array([0.6, 0.3, 0.1])
    q = np.array([0.4, 0.5, 0.1])
    tb = bf16_bits_from_f64(np.log(p))
    db = bf16_bits_from_f64(np.log(q))
    pt = oracle.softmax_t(oracle.widen_bf16(tb), 1.0)
    pd = oracle.softmax_t(oracle.widen_bf16(db), 1.0)
    rng = np.random.default_rng(seed)
    return {
        "target": np.broadcast_to(tb, (Bn, 2, 3)).copy(),
        "draft": np.broadcast_to(db, (Bn, 1, 3)).copy(),
        "draft_tokens": rng.choice(3, size=(Bn, 1), p=pd).astype(np.int32),
        "r": rng.random((Bn, 1), dtype=np.float32),
        "u": rng.random((Bn, 2), dtype=np.float32),
    }, pt, pd


def test_worked_example_exact(B):
    banner("worked example V=3 B=4096 exact")
    x, pt, pd = worked_example_rows(4096, seed=1)
    A, o, m, _ = run_verify(B, x)
    ref = oracle_verify(x)
    stats_ = compare_verify(ref, A, o, m, "worked")
    assert stats_["excluded_sequences"] == 0


def test_worked_example_lossless_mc(B):
    """Tutorial §5.2: the first emitted token follows the target.  One million GPU trials."""
    banner("worked example lossless MC 1M")
    counts = np.zeros(3)
    for rep in range(16):
        x, pt, pd = worked_example_rows(1 << 16, seed=100 + rep)
        A, o, _, _ = run_verify(B, x)
        first = np.where(A == 1, x["draft_tokens"][:, 0], o)
        counts += np.bincount(first, minlength=3)
    n = counts.sum()
    assert stats.chisquare(counts, n * pt).pvalue > 1e-4, (counts / n, pt)
    # and it is not the draft's law, nor the wrong-resample law (P(cat) = 0.52)
    assert abs(counts[0] / n - pt[0]) < 2e-3 and abs(counts[0] / n - 0.52) > 0.05


@pytest.mark.parametrize("V", [1, 2, 3, 7, 8, 9, 100, 511, 512, 513, 2047, 2048, 2049, 4096, 4097, 6143, 10000])
def test_ragged_vocab(B, V):
    banner(f"ragged V={V}")
    K = 3
    x = sps_case(8, K, V, seed=V)
    A, o, m, _ = run_verify(B, x)
    compare_verify(oracle_verify(x), A, o, m, f"V={V}")
    assert np.all((o >= 0) & (o < V))


def test_several_tiles(B):
    banner("B=16 K=5 V=5000 sigma 2.5/0.8")
    x = sps_case(16, 5, 5000, seed=3)
    A, o, m, _ = run_verify(B, x)
    print(compare_verify(oracle_verify(x), A, o, m, "tiles"))


@pytest.mark.parametrize("T", [0.7, 1.6])
def test_temperature(B, T):
    banner(f"temperature {T}")
    x = sps_case(16, 4, 3000, seed=5, T=T)
    A, o, m, _ = run_verify(B, x, T=T)
    compare_verify(oracle_verify(x, T=T), A, o, m, f"T={T}")


def test_peaked_rows(B):
    banner("peaked rows 50%")
    x = sps_case(32, 5, 7000, seed=7, peak=0.5)
    A, o, m, _ = run_verify(B, x)
    compare_verify(oracle_verify(x), A, o, m, "peaked")


def test_masked_logits(B):
    """-inf logits (masked tokens): zero mass, never drawn."""
    banner("masked logits")
    rng = np.random.default_rng(11)
    x = sps_case(16, 4, 3001, seed=11)
    neg = np.uint16(0xFF80)
    for b in range(16):
        for k in range(5):
            x["target"][b, k, rng.choice(3001, 800, replace=False)] = neg
        for k in range(4):
            x["draft"][b, k, rng.choice(3001, 800, replace=False)] = neg
    # drafted tokens must have draft mass: redraw from the masked draft rows
    x["draft_tokens"] = gen.sample_tokens(x["draft"], 1.0, seed=12, config_id=91)
    A, o, m, _ = run_verify(B, x)
    ref = oracle_verify(x)
    compare_verify(ref, A, o, m, "masked")
    for b in range(16):
        a = int(A[b])
        row = x["target"][b, a] if a == 4 else None
        if row is not None:
            assert row[o[b]] != neg


def test_equal_rows_always_accept(B):
    """Tutorial §7.2: q = p never rejects; the bonus comes from target row K."""
    banner("equal rows")
    x = sps_case(16, 5, 4000, seed=13)
    x["draft"] = x["target"][:, :5].copy()
    x["draft_tokens"] = gen.sample_tokens(x["draft"], 1.0, seed=14, config_id=92)
    A, o, m, _ = run_verify(B, x)
    assert np.all(A == 5) and np.all(m == 1)
    compare_verify(oracle_verify(x), A, o, m, "equal")


def test_disjoint_always_reject(B):
    """Tutorial §7.3: disjoint supports reject at once; the residual is the target itself."""
    banner("disjoint support")
    V = 2000
    x = sps_case(16, 3, V, seed=15)
    neg = np.uint16(0xFF80)
    x["target"][:, :, : V // 2] = neg
    x["draft"][:, :, V // 2:] = neg
    x["draft_tokens"] = gen.sample_tokens(x["draft"], 1.0, seed=16, config_id=93)
    A, o, m, _ = run_verify(B, x)
    assert np.all(A == 0) and np.all(m == 0) and np.all(o >= V // 2)
    compare_verify(oracle_verify(x), A, o, m, "disjoint")


def test_invalid_token_reports_minus_one(B):
    banner("invalid token ids")
    x = sps_case(4, 3, 1000, seed=17)
    x["draft_tokens"][1, 2] = 1000
    x["draft_tokens"][3, 0] = -5
    A, o, m, _ = run_verify(B, x)
    assert A[1] == -1 and o[1] == -1 and A[3] == -1 and o[3] == -1
    assert m[1, 2] == 0 and m[3, 0] == 0
    ref = oracle_verify({k: (v[[0, 2]] if isinstance(v, np.ndarray) else v) for k, v in x.items()})
    compare_verify(ref, A[[0, 2]], o[[0, 2]], m[[0, 2]], "valid rows")


def test_full_llama_vocab_config(B):
    """The benchmarked workload: B=64, K=5, V=128256, 1% peaked rows; every sequence checked."""
    banner("full B=64 K=5 V=128256")
    x = gen.make_sps_inputs(gen.LLAMA_SPS)
    A, o, m, _ = run_verify(B, x)
    ref = oracle_verify(x)
    print(compare_verify(ref, A, o, m, "full c2"))


@pytest.mark.parametrize("Bn,V,delta", [(16, 1 << 20, None), (64, 400000, None), (64, 400000, 0.5)])
def test_units_of_several_slices(B, Bn, V, delta):
    """More sequence slices than the grid has workgroups (B S > 512 on MI355X): a
    sequence gets fewer draw units than slices, each streaming several slices (V = 2^20:
    S = 64, 16 sequences, units of 2 slices; V = 400,000: S = 25, 64 sequences, units of
    3-4 slices), and a crossing in a unit's earlier slice is found from a re-read tile.
    Every sequence is checked, for SpS and for Cactus."""
    banner(f"several slices per draw unit B={Bn} V={V} delta={delta}")
    x = sps_case(Bn, 3, V, seed=31 + Bn, peak=0.0)
    A, o, m, g = run_verify(B, x, delta=delta)
    ref = oracle_verify(x, delta=delta)
    print(compare_verify(ref, A, o, m, f"several slices B={Bn} V={V}"))
    if delta is not None:
        valid = x["draft_tokens"] >= 0
        assert_rel(g[valid], ref["gamma_star"][valid], label="gamma* (several slices)")
    # where the tokens fell, with the draw units a 512-workgroup grid gives
    S = -(-V // 16384)
    P1 = max(1, min(S, 512 // Bn))
    earlier = sum(1 for t in o if t >= 0 and (t // 16384) + P1 < S)
    print(f"tokens in a slice that is not its unit's last: {earlier} of {Bn}")


@pytest.mark.parametrize("Bn,V", [(64, 128256), (16, 1 << 20), (64, 400000)])
def test_bonus_row_at_references_of_its_own(B, Bn, V):
    """Every draft accepted (draft rows equal to the target's), so every sequence draws
    its bonus from target row K, a row with no statistics of its own: each wave of a draw
    unit weighs its share of a slice at its own reference and the slices meet at a common
    one ([LT] §9.1: the bonus token from the target's last row).  Each bonus row puts two
    slices 40 above the rest, so that the mass splits between them, every other slice 200
    below (about 290 binary orders, past fp32's range), one wave's share of a top slice
    30 below its slice, and a run of masked (-inf) tokens in the other top slice.  Units of
    one slice (V = 128,256) and of several (V = 2^20 and 400,000); every sequence checked."""
    banner(f"bonus draws at their own references B={Bn} V={V}")
    K = 4
    x = sps_case(Bn, K, V, seed=41 + Bn, peak=0.0)
    x["draft"] = x["target"][:, :K].copy()
    x["draft_tokens"] = gen.sample_tokens(x["draft"], 1.0, seed=42, config_id=94)
    rng = np.random.default_rng(43 + Bn)
    S = -(-V // 16384)
    tops = []
    for b in range(Bn):
        z = oracle.widen_bf16(x["target"][b, K]).astype(np.float64)
        top = rng.choice(S, size=2, replace=False)
        off = np.full(S, -200.0)
        off[top] = 40.0 + 0.5 * rng.random(2)
        z = z + np.repeat(off, 16384)[:V]
        for q in range(8):  # wave 2's share of the first top slice: 512 tokens of each tile
            lo = int(top[0]) * 16384 + q * 2048 + 2 * 512
            z[lo:min(lo + 512, V)] -= 30.0
        bits = bf16_bits_from_f64(z)
        lo = int(top[1]) * 16384 + 300
        bits[lo:min(lo + 700, V)] = np.uint16(0xFF80)
        x["target"][b, K] = bits
        tops.append(sorted(int(t) for t in top))
    A, o, m, _ = run_verify(B, x)
    assert np.all(A == K) and np.all(m == 1)
    ref = oracle_verify(x)
    print(compare_verify(ref, A, o, m, f"bonus B={Bn} V={V}"))
    # the draws did land in both top slices across the batch
    slices = [int(t) // 16384 for t in o]
    assert all(s in tp for s, tp in zip(slices, tops))
    first = sum(1 for s, tp in zip(slices, tops) if s == tp[0])
    print(f"tokens in the lower-indexed top slice: {first} of {Bn}")
    assert 0 < first < Bn


def test_repeat_deterministic_one_workspace(B):
    """100 back-to-back calls on one workspace (its words must return to zero each time)
    give bit-identical results; then the same workspace serves another V."""
    banner("repeat 100x on one workspace")
    from speculative_sampling_verification_row_amd import binding
    x = sps_case(16, 5, 9000, seed=19)
    ws = binding.make_workspace(16, 5, 1)
    first = run_verify(B, x, ws=ws)
    for _ in range(99):
        again = run_verify(B, x, ws=ws)
        for a, b in zip(first[:3], again[:3]):
            np.testing.assert_array_equal(a, b)
    compare_verify(oracle_verify(x), *first[:3], "repeat")
    y = sps_case(16, 5, 40000, seed=20)
    got = run_verify(B, y, ws=ws)
    compare_verify(oracle_verify(y), *got[:3], "same workspace, V=40000")
    # every call leaves the workspace zero: a smaller B and K reuse it without clearing
    z = sps_case(8, 3, 20000, seed=21)
    got = run_verify(B, z, ws=ws)
    compare_verify(oracle_verify(z), *got[:3], "same workspace, B=8 K=3")
    assert int(ws.count_nonzero().item()) == 0


# ---------------------------------------------------------------------------
# Cactus
# ---------------------------------------------------------------------------

def test_cactus_delta0_bit_identical_to_sps(B):
    banner("cactus delta=0 == spec_verify")
    x = sps_case(32, 6, 6000, seed=21, sigma_t=3.0, sigma_d=1.0, peak=0.0)
    a = run_verify(B, x)
    c = run_verify(B, x, delta=0.0)
    for u, v in zip(a[:3], c[:3]):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("delta", [0.0, 0.5, 1.0])
def test_cactus_parity(B, delta):
    banner(f"cactus delta={delta} B=16 m=20 V=4000")
    x = sps_case(16, 20, 4000, seed=23, sigma_t=3.0, sigma_d=1.0, peak=0.0)
    A, o, m, g = run_verify(B, x, delta=delta)
    ref = oracle_verify(x, delta=delta)
    compare_verify(ref, A, o, m, f"cactus {delta}")
    valid = x["draft_tokens"] >= 0
    assert_rel(g[valid], ref["gamma_star"][valid], label="gamma*")


# ---------------------------------------------------------------------------
# Cactus with gamma* the exact root of the KL budget
# ---------------------------------------------------------------------------

def test_cactus_kl_delta0_bit_identical_to_sps(B):
    banner("cactus-kl delta=0 == spec_verify")
    x = sps_case(32, 6, 6000, seed=31, sigma_t=3.0, sigma_d=1.0, peak=0.0)
    a = run_verify(B, x)
    c = run_verify(B, x, delta=0.0, kl=True)
    for u, v in zip(a[:3], c[:3]):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("delta", [0.02, 0.5, 1.0, 3.0])
def test_cactus_kl_parity(B, delta):
    """delta = 3 clips gamma* to 1 wherever c >= e^-3, delta = 0.02 keeps it near c."""
    banner(f"cactus-kl delta={delta} B=16 m=20 V=4000")
    x = sps_case(16, 20, 4000, seed=33, sigma_t=3.0, sigma_d=1.0, peak=0.0)
    A, o, m, g = run_verify(B, x, delta=delta, kl=True)
    ref = oracle_verify(x, delta=delta, kl=True)
    compare_verify(ref, A, o, m, f"cactus-kl {delta}")
    valid = x["draft_tokens"] >= 0
    assert_rel(g[valid], ref["gamma_star"][valid], label="gamma* kl")


def test_cactus_kl_ragged_and_peaked(B):
    """A ragged vocabulary over several slices, peaked rows (c near 1 and near 0)."""
    banner("cactus-kl B=8 m=7 V=20001 peaked delta=0.3")
    x = sps_case(8, 7, 20001, seed=35, sigma_t=2.5, sigma_d=0.8, peak=0.2)
    A, o, m, g = run_verify(B, x, delta=0.3, kl=True)
    ref = oracle_verify(x, delta=0.3, kl=True)
    compare_verify(ref, A, o, m, "cactus-kl ragged")
    assert_rel(g, ref["gamma_star"], label="gamma* kl ragged")


def test_cactus_kl_not_below_taylor_where_corollary6_applies(B):
    """Corollary 6: where the Taylor gamma* is <= 0.5 it keeps the budget, so the exact root is
    at least as large there, position by position, on the same launch inputs."""
    banner("cactus-kl >= taylor where taylor <= 0.5")
    x = sps_case(16, 20, 4000, seed=37, sigma_t=3.0, sigma_d=1.0, peak=0.0)
    _, _, _, gt = run_verify(B, x, delta=0.5)
    _, _, _, gk = run_verify(B, x, delta=0.5, kl=True)
    sel = gt <= 0.5
    assert sel.sum() > 100
    assert np.all(gk[sel] >= gt[sel] * (1 - 1e-6))


@pytest.mark.parametrize("delta", [1e-6, 40.0])
def test_cactus_kl_extreme_budgets(B, delta):
    """A tiny budget keeps gamma* within rounding of c (the small-x series of the divergence);
    delta = 40 clips gamma* to 1 for every candidate with c >= e^-40."""
    banner(f"cactus-kl delta={delta} B=8 m=6 V=9000")
    x = sps_case(8, 6, 9000, seed=39, sigma_t=3.0, sigma_d=1.0, peak=0.0)
    A, o, m, g = run_verify(B, x, delta=delta, kl=True)
    ref = oracle_verify(x, delta=delta, kl=True)
    compare_verify(ref, A, o, m, f"cactus-kl extreme {delta}")
    assert_rel(g, ref["gamma_star"], label=f"gamma* kl {delta}")
