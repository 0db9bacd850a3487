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


def small_loop(binding, T=24, seed=0):
    from speculative_sampling_verification_row_amd.loop import HedgeSpecLoop
    w = gen.GammaWorkload("loop", B=4, K=3, N=3, V=3000, target_sigma=2.0, sigma_range=(0.3, 2.0), fused=True,
                          draft_from="drafter0", config_id=97)
    x = gen.make_gamma_inputs(w, seed=seed)
    rng = np.random.default_rng(seed + 60)
    delays = rng.integers(0, 2 * w.K + 1, (T, w.B)).astype(np.int32)
    v = rng.random((T, w.B), dtype=np.float32)
    lp = HedgeSpecLoop(dev_bf16(x["target"]), dev_bf16(x["drafts"]), dev_i32(x["traj"]), dev_i32(x["draft_tokens"]),
                       dev_f32(x["r"]), dev_f32(x["u"]), dev_i32(delays), dev_f32(v), 1.0 / w.K)
    return lp, x, delays, v


def snapshot(lp):
    torch.cuda.synchronize()
    return [to_np(t).copy() for t in (lp.sel_hist, lp.R, lp.W, lp.out["gamma"], lp.out["loss"],
                                      lp.out["accepted_len"], lp.out["out_token"])]


def test_loop_graph_replays_equal_eager_rounds(binding):
    """A captured round replayed T times gives bit for bit what T eager rounds give, three
    times over, with eager work and synchronisations between the replays."""
    banner("loop graph vs eager")
    T = 24
    lp, _, _, _ = small_loop(binding, T)
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
        assert binding.workspace_fault(lp.ws) == 0 and int(lp.ws.count_nonzero().item()) == 0
        junk = torch.randn(1000, device="cuda").sum()   # the program's own eager work between replays
        torch.cuda.synchronize()
        del junk


def test_loop_rounds_match_oracle(binding):
    """Every round evaluates the same rows, so every round's loss is the oracle's loss of
    those rows; the learner's selections must follow the oracle queue wherever the drawn
    uniform is not within 1e-4 of a cumulative weight."""
    banner("loop vs oracle")
    T = 24
    lp, x, delays, v = small_loop(binding, T, seed=1)
    for _ in range(T):
        lp.step()
    hist, R, W, g, l, A, tok = snapshot(lp)
    K = x["drafts"].shape[2]
    ref = oracle.spec_counterfactual_gamma(x["target"][:, :K], x["drafts"], x["traj"])
    np.testing.assert_allclose(g, ref["gamma"], rtol=1e-5)
    losses = np.broadcast_to(ref["loss"], (T,) + ref["loss"].shape)
    sel_o, R_o, W_o = oracle.hedge_delayed_rounds_rule(losses, delays, v, 1.0 / K, eta=None)
    np.testing.assert_allclose(R, R_o, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(W, W_o, rtol=1e-4, atol=1e-6)
    # selections: the oracle's own weights before each round decide which draws are clear
    Rb = np.zeros_like(R_o)
    Wb = np.full_like(W_o, 1.0 / W_o.shape[1])
    checked = 0
    for b in range(hist.shape[1]):
        pending = []
        for t in range(T):
            ready = sorted(p for p in pending if p[0] <= t)
            pending = [p for p in pending if p[0] > t]
            for _, s in ready:
                Rb[b], Wb[b] = oracle.normalhedge_step(Rb[b], Wb[b], losses[s, b] * np.float32(1.0 / K))
            c = np.cumsum(Wb[b]) / Wb[b].sum()
            if np.min(np.abs(c - float(v[t, b]))) > 1e-4:
                assert hist[t, b] == oracle.normalhedge_select(Wb[b], float(v[t, b])), (t, b)
                checked += 1
            pending.append((t + 1 + int(delays[t, b]), t))
    assert checked > 0.9 * T * hist.shape[1]
    # the last round's fused verification used drafter hist[T-1][b]
    draft = np.stack([x["drafts"][hist[T - 1, b], b] for b in range(x["target"].shape[0])])
    vref = oracle.spec_verify(x["target"], draft, x["draft_tokens"], x["r"], x["u"])
    ok = vref["margin_r"].min(axis=1) >= 1e-6
    assert np.array_equal(A[ok], vref["accepted_len"][ok])
