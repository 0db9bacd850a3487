"""GPU parity of the device-resident HedgeSpec rounds: the delayed-feedback queue kernel
(hedge_queue_update) against the oracle's queue, and whole rounds (queue + fused verify and
gamma) replayed from a captured graph against the same rounds launched eagerly and against the
oracle."""

import numpy as np
import pytest

import oracle
from speculative_sampling_verification_row_amd import inputs as gen

from gpu_util import banner, dev_bf16, dev_f32, dev_i32
from parity import to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def binding():
    from speculative_sampling_verification_row_amd import binding as b
    b.load()
    return b


def test_queue_kernel_matches_oracle_queue(binding):
    """256 rounds, B=32 learners of N=7, delays in [-1, 2K] (-1: never), losses from a seeded
    generator; the queue lives on the device and is driven one round at a time."""
    banner("queue kernel 256 rounds")
    T, B, N, K = 256, 32, 7, 5
    Q = 2 * K + 2
    losses = gen.synthetic_losses(T, B, N, K).astype(np.float32)
    rng = np.random.default_rng(50)
    delays = rng.integers(-1, 2 * K + 1, (T, B)).astype(np.int32)
    v = rng.random((T, B), dtype=np.float32)
    sel_o, R_o, W_o = oracle.hedge_delayed_rounds_rule(losses, delays, v, 1.0 / K, eta=None)
    dev = "cuda"
    R = torch.zeros((B, N), dtype=torch.float64, device=dev)
    W = torch.full((B, N), 1.0 / N, dtype=torch.float64, device=dev)
    ql = torch.zeros((B, Q, N), dtype=torch.float64, device=dev)
    qd = torch.full((B, Q), -1, dtype=torch.int32, device=dev)
    rnd = torch.zeros(B, dtype=torch.int32, device=dev)
    loss = torch.zeros((B, N), dtype=torch.float32, device=dev)
    d_dev, v_dev = dev_i32(delays), dev_f32(v)
    sel = torch.zeros(B, dtype=torch.int32, device=dev)
    hist = torch.zeros((T, B), dtype=torch.int32, device=dev)
    lib = binding.load()
    P = binding._ptr
    for t in range(T):
        if t > 0:
            loss.copy_(dev_f32(losses[t - 1]))
        st = lib.hedge_queue_update(P(R), P(W), P(ql), P(qd), P(rnd), P(loss), P(d_dev), 1.0 / K, P(v_dev), P(sel),
                                    P(hist), B, N, Q, T, binding._stream())
        assert st == 0
    torch.cuda.synchronize()
    # the oracle also applies the losses of round T-1 and earlier that are usable at round T-1 only
    np.testing.assert_array_equal(to_np(hist), sel_o)
    np.testing.assert_allclose(to_np(R), R_o, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(to_np(W), W_o, rtol=1e-9, atol=1e-12)
    assert int(to_np(rnd).min()) == T


def loop_rows(x):
    return {"target": dev_bf16(x["target"]), "drafts": dev_bf16(x["drafts"]), "traj": dev_i32(x["traj"]),
            "draft_tokens": dev_i32(x["draft_tokens"]), "r_accept": dev_f32(x["r"]), "u_resample": dev_f32(x["u"])}


def small_inputs(seed, big=False):
    # big: 64 sequences of 151,936-token rows (10 slices each), more draw units than
    # the grid holds, so the fused kernel's units of several slices run
    w = (gen.GammaWorkload("loop", B=64, K=2, N=2, V=151936, target_sigma=2.0, sigma_range=(0.3, 2.0), fused=True,
                           draft_from="drafter0", config_id=96) if big else
         gen.GammaWorkload("loop", B=4, K=3, N=3, V=3000, target_sigma=2.0, sigma_range=(0.3, 2.0), fused=True,
                           draft_from="drafter0", config_id=97))
    return w, gen.make_gamma_inputs(w, seed=seed)


def small_loop(binding, T=24, seed=0, scheduled=False, sets=1, fused=True, eta=None, big=False):
    from speculative_sampling_verification_row_amd.loop import HedgeSpecLoop
    w, x = small_inputs(seed, big)
    xs = [x] + [small_inputs(seed + 100 + j, big)[1] for j in range(sets - 1)]
    rng = np.random.default_rng(seed + 60)
    delays = rng.integers(0, 2 * w.K + 1, (T, w.B)).astype(np.int32)
    v = rng.random((T, w.B), dtype=np.float32)
    rows = [loop_rows(xi) for xi in xs]
    lp = HedgeSpecLoop(rows if sets > 1 else rows[0], dev_f32(v), 1.0 / w.K,
                       delays=dev_i32(delays) if scheduled else None, fused=fused, eta=eta)
    return lp, xs, delays, v


def snapshot(lp):
    torch.cuda.synchronize()
    return [to_np(t).copy() for t in (lp.sel_hist, lp.learner.state, lp.learner.weights, lp.out["gamma"],
                                      lp.out["loss"], lp.out["accepted_len"], lp.out["out_token"])]


@pytest.mark.parametrize("scheduled,sets", [(False, 1), (True, 1), (False, 2)])
def test_loop_graph_replays_equal_eager_rounds(binding, scheduled, sets):
    """Captured rounds replayed T times give bit for bit what T eager rounds give, three
    times over, with eager work and synchronisations between the replays (censoring or
    scheduled delays; one row set, or two alternating row sets with a graph each)."""
    banner(f"loop graph vs eager scheduled={scheduled} sets={sets}")
    T = 24
    lp, _, _, _ = small_loop(binding, T, scheduled=scheduled, sets=sets)
    for _ in range(T):
        lp.step()
    ref = snapshot(lp)
    assert int(lp.ws.count_nonzero().item()) == 0
    lp.reset()
    lp.capture()
    for rep in range(3):
        lp.reset()
        torch.cuda.synchronize()
        for _ in range(T):
            lp.replay()
        got = snapshot(lp)
        for a, b in zip(ref, got):
            np.testing.assert_array_equal(a, b)
        lp.check()
        assert int(lp.ws.count_nonzero().item()) == 0
        junk = torch.randn(1000, device="cuda").sum()   # the program's own eager work between replays
        torch.cuda.synchronize()
        del junk


def oracle_round_outcomes(x):
    """The oracle's loss of every drafter on these rows, and its verification of each drafter
    (accepted length, near-tie flag per sequence)."""
    K = x["drafts"].shape[2]
    ref = oracle.spec_counterfactual_gamma(x["target"][:, :K], x["drafts"], x["traj"])
    N, B = x["drafts"].shape[:2]
    A = np.zeros((N, B), dtype=np.int64)
    tie = np.zeros((N, B), dtype=bool)
    for i in range(N):
        vr = oracle.spec_verify(x["target"], x["drafts"][i], x["draft_tokens"], x["r"], x["u"])
        A[i] = vr["accepted_len"]
        tie[i] = vr["margin_r"].min(axis=1) < 1e-6
    return ref, A, tie


def check_selections_follow_oracle(hist, W_rounds, v, margin=1e-4):
    """hist [T, B] from the device; W_rounds [T, B, N] the oracle learner's weights before each
    round's draw.  Each sequence must match the oracle's draw at every round up to the first
    whose uniform lies within `margin` of a cumulative weight (after which the two runs may
    part).  Returns the number of rounds compared."""
    T, B = hist.shape
    checked = 0
    for b in range(B):
        for t in range(T):
            w = W_rounds[t, b]
            c = np.cumsum(w) / w.sum()
            if np.min(np.abs(c - float(v[t, b]))) <= margin:
                break
            assert hist[t, b] == oracle.normalhedge_select(w, float(v[t, b])), (t, b)
            checked += 1
    return checked


@pytest.mark.parametrize("eta", [None, 0.7])
def test_fused_round_equals_two_launches(binding, eta):
    """One launch per round (spec_hedgespec_round: the learner step inside the gamma
    launch) gives, round after round, bit for bit what the learner's own launch
    followed by the fused gamma launch gives: selections, learner state, gamma, losses,
    accepted lengths and tokens (NormalHedge, and Hedge at rate eta; two row sets)."""
    banner(f"fused round vs two launches eta={eta}")
    T = 24
    a = small_loop(binding, T, sets=2, fused=True, eta=eta)[0]
    b = small_loop(binding, T, sets=2, fused=False, eta=eta)[0]
    assert a.fused and not b.fused
    for t in range(T):
        a.step()
        b.step()
        for x, y in zip(snapshot(a) + [to_np(a.learner.sel), to_np(a.learner.round)],
                        snapshot(b) + [to_np(b.learner.sel), to_np(b.learner.round)]):
            np.testing.assert_array_equal(x, y, err_msg=f"round {t}")
    assert int(a.ws.count_nonzero().item()) == 0 and int(b.ws.count_nonzero().item()) == 0
    a.check()


def test_fused_round_equals_two_launches_multi_slice_units(binding):
    """The same at 64 sequences of 151,936-token rows: 640 draw units for a grid of at
    most 512, so each fused launch runs the instance whose draw units take several
    slices, with the learner steps in its first gamma slot."""
    banner("fused round vs two launches, units of several slices")
    T = 6
    a = small_loop(binding, T, fused=True, big=True)[0]
    b = small_loop(binding, T, fused=False, big=True)[0]
    S = -(-151936 // 16384)
    assert 64 * S > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    for t in range(T):
        a.step()
        b.step()
        for x, y in zip(snapshot(a) + [to_np(a.learner.sel), to_np(a.learner.round)],
                        snapshot(b) + [to_np(b.learner.sel), to_np(b.learner.round)]):
            np.testing.assert_array_equal(x, y, err_msg=f"round {t}")
    assert int(a.ws.count_nonzero().item()) == 0 and int(b.ws.count_nonzero().item()) == 0
    a.check()


def test_loop_censored_rounds_match_oracle(binding):
    """Every round evaluates the same rows, so every round's loss is the oracle's loss of
    those rows and a round's accepted length is the oracle's verification of the drafter it
    selected; the device learner, counting the censoring delay from its own accepted lengths,
    must make the oracle learner's selections (hedge_censored_rounds)."""
    banner("loop censored vs oracle")
    T = 24
    lp, xs, _, v = small_loop(binding, T, seed=1)
    x = xs[0]
    for _ in range(T):
        lp.step()
    hist, S, W, g, l, A, tok = snapshot(lp)
    ref, A_by, tie = oracle_round_outcomes(x)
    assert not tie.any()
    np.testing.assert_allclose(g, ref["gamma"], rtol=1e-5)
    K, N, B = x["drafts"].shape[2], x["drafts"].shape[0], x["drafts"].shape[1]

    def outcome(t, sel):
        return ref["loss"], A_by[sel, np.arange(B)]

    # The learners' arithmetic is checked at 1e-9 where both are fed the same losses
    # (test_gpu_gamma_hedge.py); here the device learner consumes the GPU's own fp32
    # losses, each within the parity bound (1e-5 relative), and 24 rounds of them
    # add up in the state, so the state is held to 1e-4 relative.
    sel_o, S_o, W_o, acc_o, W_rounds = oracle.hedge_censored_rounds(outcome, T, B, N, K, K + 1, 1.0 / K, v)
    checked = check_selections_follow_oracle(hist, W_rounds, v)
    assert checked > 0.9 * T * B, checked
    if checked == T * B:
        np.testing.assert_array_equal(hist, sel_o)
        np.testing.assert_allclose(S, S_o, rtol=1e-4, atol=1e-6)
        np.testing.assert_allclose(W, W_o, rtol=1e-4, atol=1e-6)
        np.testing.assert_array_equal(A, acc_o[T - 1])


def test_loop_scheduled_rounds_match_oracle(binding):
    """As above with the delay schedule given in advance (ScheduledLearner)."""
    banner("loop scheduled vs oracle")
    T = 24
    lp, xs, delays, v = small_loop(binding, T, seed=1, scheduled=True)
    x = xs[0]
    for _ in range(T):
        lp.step()
    hist, R, W, g, l, A, tok = snapshot(lp)
    K = x["drafts"].shape[2]
    ref = oracle.spec_counterfactual_gamma(x["target"][:, :K], x["drafts"], x["traj"])
    losses = np.broadcast_to(ref["loss"], (T,) + ref["loss"].shape)
    sel_o, R_o, W_o = oracle.hedge_delayed_rounds_rule(losses, delays, v, 1.0 / K, eta=None)
    np.testing.assert_allclose(R, R_o, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(W, W_o, rtol=1e-4, atol=1e-6)
    W_rounds = [oracle.hedge_delayed_rounds_rule(losses[: t + 1], delays[: t + 1], v[: t + 1], 1.0 / K)[2]
                for t in range(T)]
    checked = check_selections_follow_oracle(hist, np.array(W_rounds), v)
    assert checked > 0.9 * T * hist.shape[1]
    # the last round's fused verification used drafter hist[T-1][b]
    draft = np.stack([x["drafts"][hist[T - 1, b], b] for b in range(x["target"].shape[0])])
    vref = oracle.spec_verify(x["target"], draft, x["draft_tokens"], x["r"], x["u"])
    ok = vref["margin_r"].min(axis=1) >= 1e-6
    assert np.array_equal(A[ok], vref["accepted_len"][ok])


def test_loop_reads_rows_written_between_rounds(binding):
    """A caller streaming new rows writes them into the loop's inputs between rounds: the
    captured round must verify and evaluate the new rows (no frozen copy)."""
    banner("loop rows rewritten between replays")
    T = 4
    lp, xs, _, v = small_loop(binding, T, seed=2)
    lp.capture()
    lp.reset()
    lp.replay()
    _, x2 = small_inputs(77)
    for key, val in loop_rows(x2).items():
        lp.inputs[0][key].copy_(val)
    lp.replay()
    torch.cuda.synchronize()
    K = x2["drafts"].shape[2]
    ref = oracle.spec_counterfactual_gamma(x2["target"][:, :K], x2["drafts"], x2["traj"])
    np.testing.assert_allclose(to_np(lp.out["gamma"]), ref["gamma"], rtol=1e-5)
    sel = to_np(lp.sel_hist)[1]
    draft = np.stack([x2["drafts"][sel[b], b] for b in range(x2["target"].shape[0])])
    vref = oracle.spec_verify(x2["target"], draft, x2["draft_tokens"], x2["r"], x2["u"])
    ok = vref["margin_r"].min(axis=1) >= 1e-6
    assert np.array_equal(to_np(lp.out["accepted_len"])[ok], vref["accepted_len"][ok])


def test_loop_refuses_inputs_it_would_copy(binding):
    """An input the library cannot read in place (another dtype, a misaligned row base) would
    be copied once and the copy captured: the loop refuses it instead."""
    from speculative_sampling_verification_row_amd.loop import HedgeSpecLoop
    w, x = small_inputs(3)
    rows = loop_rows(x)
    v = dev_f32(np.full((4, w.B), 0.5, dtype=np.float32))
    with pytest.raises(ValueError):
        HedgeSpecLoop(dict(rows, traj=rows["traj"].to(torch.int64)), v, 1.0 / w.K)
    # rows of V = 2999 on a pitch of 3000: the drafts can be read in place, a target starting
    # one element in (2-byte offset) cannot
    shifted = dict(rows, target=rows["target"][..., 1:], drafts=rows["drafts"][..., :2999])
    with pytest.raises(ValueError):
        HedgeSpecLoop(shifted, v, 1.0 / w.K)
    HedgeSpecLoop(dict(rows, target=rows["target"][..., :2999], drafts=rows["drafts"][..., :2999]), v, 1.0 / w.K)


def test_fault_word_is_surfaced_and_cleared(binding):
    """A set fault word (a wait between workgroups that timed out) makes the synchronisation
    point raise, and leaves the workspace zeroed for reuse.  The word is set from the host."""
    banner("fault word surfaced")
    from speculative_sampling_verification_row_amd.binding import WorkspaceFault
    lp, _, _, _ = small_loop(binding, 4, seed=4)
    lp.step()
    lp.check()
    lp.ws[binding.FAULT_WORD_OFFSET] = 1
    with pytest.raises(WorkspaceFault):
        lp.check()
    assert int(lp.ws.count_nonzero().item()) == 0
    lp.step()
    lp.check()
