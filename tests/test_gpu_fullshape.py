"""GPU parity at the full sizes of the evaluation workloads, every sequence checked.

The oracle runs row-parallel on the host cores (tests/oracle_pool.py) so that
the whole batch of each workload is compared, not a sample:
  * HedgeSpec evaluation, B=32, K=5, N=7, V=128256, fused with the verification
    of each sequence's selected drafter (the launch the HedgeSpec rounds use);
  * Cactus, B=64, m=20, V=151936, at delta 0, 0.5 and 1 (Taylor gamma*) and at
    delta 1 with the exact-KL gamma*;
  * the 21-drafter pool, B=64, K=8, N=21, V=151936, in one fused launch;
  * 256 HedgeSpec rounds at the evaluation size with the censoring delay, the
    learner consuming the device's own losses and accepted lengths;
  * an estimator whose K (N + 1) rows exceed one pass of its row buffer
    (K=20, N=21), so that it runs in chunks of positions.
Comparison rules: tests/parity.py.
"""

import numpy as np
import pytest

import oracle
from speculative_sampling_verification_row_amd import inputs as gen

from gpu_util import banner, dev_bf16, dev_f32, dev_i32
from oracle_pool import OraclePool
from parity import assert_loss, assert_rel, compare_verify, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def binding():
    from speculative_sampling_verification_row_amd import binding as b
    b.load()
    return b


def gamma_call(binding, x, fused):
    kw = {}
    if fused:
        kw = dict(sel=dev_i32(x["sel"]), draft_tokens=dev_i32(x["draft_tokens"]), r_accept=dev_f32(x["r"]),
                  u_resample=dev_f32(x["u"]))
    N, B, K = x["drafts"].shape[:3]
    ws = binding.make_workspace(B, K, N)
    out = binding.spec_counterfactual_gamma(dev_bf16(x["target"]), dev_bf16(x["drafts"]), dev_i32(x["traj"]),
                                            workspace=ws, **kw)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0, "workspace not left zero"
    return {k: to_np(v) for k, v in out.items()}


def check_gamma(got, ref, label):
    wg = assert_rel(got["gamma"], ref["gamma"], label=f"{label} gamma")
    we = assert_rel(got["est_len"], ref["est_len"], label=f"{label} est")
    wl = assert_loss(got["loss"], ref["loss"], ref["gamma"].shape[1], label=label)
    print(f"{label}: max rel err gamma {wg:.2e} est {we:.2e} loss {wl:.2e}")


@pytest.fixture(scope="module")
def hedge_eval_inputs():
    import dataclasses
    return gen.make_gamma_inputs(dataclasses.replace(gen.HEDGE_EVAL, fused=True))


@pytest.mark.timeout(900)
def test_hedge_eval_all_sequences_fused(binding, hedge_eval_inputs):
    """B=32, K=5, N=7, V=128256: gamma, estimator and loss of every (sequence, drafter), and the
    fused verification of every sequence's selected drafter."""
    banner("full c3: B=32 K=5 N=7 V=128256 fused")
    x = hedge_eval_inputs
    got = gamma_call(binding, x, fused=True)
    B, K = x["target"].shape[0], x["drafts"].shape[2]
    with OraclePool(x) as pool:
        ref = pool.gamma(range(B), K)
        vref = pool.verify(range(B), draft="drafts", drafters=x["sel"])
    check_gamma(got, ref, "c3")
    print(compare_verify(vref, got["accepted_len"], got["out_token"], got["accept_mask"], "c3 fused verify"))


@pytest.fixture(scope="module")
def qwen_inputs():
    return gen.make_sps_inputs(gen.QWEN_CACTUS)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("delta,kl", [(0.0, False), (0.5, False), (1.0, False), (1.0, True)])
def test_qwen_cactus_all_sequences(binding, qwen_inputs, delta, kl):
    """B=64, m=20, V=151936: every sequence's decisions, accepted length, token and gamma*."""
    banner(f"full c4: B=64 m=20 V=151936 delta={delta} exact_kl={kl}")
    x = qwen_inputs
    B, m1 = x["target"].shape[:2]
    ws = binding.make_workspace(B, m1 - 1, 1)
    fn = binding.spec_cactus_kl_verify if kl else binding.spec_cactus_verify
    A, o, msk, g = fn(dev_bf16(x["target"]), dev_bf16(x["draft"]), dev_i32(x["draft_tokens"]), dev_f32(x["r"]),
                      dev_f32(x["u"]), delta, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0
    with OraclePool(x) as pool:
        ref = pool.verify(range(B), delta=delta, exact_kl=kl)
    print(compare_verify(ref, A, o, msk, f"c4 delta={delta} kl={kl}"))
    assert_rel(to_np(g), ref["gamma_star"], label="gamma*")


@pytest.mark.timeout(900)
def test_pool21_all_sequences_fused(binding):
    """B=64, K=8, N=21, V=151936 (3.4 GB of logits) in one launch: gamma, estimator and loss of
    all 21 drafters and the verification of each sequence's selected drafter, every sequence."""
    banner("full c5: B=64 K=8 N=21 V=151936 fused")
    x = gen.make_gamma_inputs(gen.POOL21)
    got = gamma_call(binding, x, fused=True)
    B, K = x["target"].shape[0], x["drafts"].shape[2]
    with OraclePool(x) as pool:
        ref = pool.gamma(range(B), K)
        vref = pool.verify(range(B), draft="drafts", drafters=x["sel"])
    check_gamma(got, ref, "c5")
    print(compare_verify(vref, got["accepted_len"], got["out_token"], got["accept_mask"], "c5 fused verify"))


def test_estimator_in_chunks_of_positions(binding):
    """K=20 positions of N=21 drafters: K (N + 1) = 440 rows exceed the estimator's row buffer
    (256), so it merges the statistics and forms the estimate in chunks of 11 positions."""
    banner("estimator chunks: B=3 K=20 N=21 V=4000")
    w = gen.GammaWorkload("chunks", B=3, K=20, N=21, V=4000, target_sigma=2.0, sigma_range=(0.2, 1.5),
                          fused=True, config_id=94)
    x = gen.make_gamma_inputs(w, seed=5)
    got = gamma_call(binding, x, fused=True)
    ref = oracle.spec_counterfactual_gamma(x["target"][:, :20], x["drafts"], x["traj"])
    check_gamma(got, ref, "K=20 N=21")
    vdraft = np.stack([x["drafts"][x["sel"][b], b] for b in range(3)])
    vref = oracle.spec_verify(x["target"], vdraft, x["draft_tokens"], x["r"], x["u"])
    compare_verify(vref, got["accepted_len"], got["out_token"], got["accept_mask"], "K=20 N=21 verify")


@pytest.mark.timeout(900)
def test_hedge_eval_256_censored_rounds(binding, hedge_eval_inputs):
    """256 HedgeSpec rounds at B=32, K=5, N=7, V=128256 from a captured graph: each round the
    device learner (NormalHedge, censoring delay) selects, the fused launch verifies the
    selection and evaluates all drafters, and the learner consumes that launch's own loss and
    accepted length.  The rows are the same every round, so the oracle plays the same rounds
    from its own loss of the rows and its own verification of each drafter; every sequence's
    selections must follow the oracle's until a drawn uniform falls within 1e-4 of a cumulative
    weight or a near-tie verification (after which the two runs may part)."""
    banner("c3 256 rounds censored, graph")
    from speculative_sampling_verification_row_amd.loop import HedgeSpecLoop
    x = hedge_eval_inputs
    N, B, K, V = x["drafts"].shape
    T = 256
    v = gen.hedge_schedule(T, B, K)["v"]
    rows = {"target": dev_bf16(x["target"]), "drafts": dev_bf16(x["drafts"]), "traj": dev_i32(x["traj"]),
            "draft_tokens": dev_i32(x["draft_tokens"]), "r_accept": dev_f32(x["r"]), "u_resample": dev_f32(x["u"])}
    lp = HedgeSpecLoop(rows, dev_f32(v), 1.0 / K)
    lp.step()                  # library set-up outside the capture
    torch.cuda.synchronize()
    lp.reset()
    lp.capture()
    lp.reset()
    for _ in range(T):
        lp.replay()
    lp.check()
    hist = to_np(lp.sel_hist)
    # the oracle's loss of the rows and its verification of every drafter, all sequences
    xo = dict(x)
    with OraclePool(xo) as pool:
        ref = pool.gamma(range(B), K)
        A_by = np.zeros((N, B), dtype=np.int64)
        tie = np.zeros((N, B), dtype=bool)
        for i in range(N):
            vr = pool.verify(range(B), draft="drafts", drafters=np.full(B, i))
            A_by[i] = vr["accepted_len"]
            tie[i] = vr["margin_r"].min(axis=1) < 1e-6
    assert_loss(to_np(lp.out["loss"]), ref["loss"], K, label="round loss")

    def outcome(t, sel):
        return ref["loss"], A_by[sel, np.arange(B)]

    sel_o, _, _, _, W_rounds = oracle.hedge_censored_rounds(outcome, T, B, N, K, K + 1, 1.0 / K, v)
    checked, parted = 0, 0
    for b in range(B):
        for t in range(T):
            w = W_rounds[t, b]
            c = np.cumsum(w) / w.sum()
            if np.min(np.abs(c - float(v[t, b]))) <= 1e-4 or tie[sel_o[t, b], b]:
                parted += 1
                break
            assert hist[t, b] == sel_o[t, b], (t, b)
            checked += 1
    print(f"256 rounds: {checked} selections compared, {parted} sequences parted at a near tie")
    assert parted <= 1 + B // 10 and checked >= 0.9 * T * B
