"""GPU parity: spec_tree_gamma (draft-tree acceptance probabilities) against the float64
oracle.  The target rows are drawn with a wide spread, so that a child chosen wrongly moves
gamma by far more than the tolerance; quantised drafter logits force ties, which must go to
the smaller token id on both sides."""

import numpy as np
import pytest

import oracle
from speculative_sampling_verification_row_amd import inputs as gen

from gpu_util import banner, bf16_bits_from_f64, dev_bf16
from parity import assert_rel, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def binding():
    from speculative_sampling_verification_row_amd import binding as b
    b.load()
    return b


def tree_case(B, K, N, V, seed, sigma_t=4.0, sigma_d=2.0, quant=None, peak=0.0):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, sigma_t, (B, K + 1, V))
    d = rng.normal(0, sigma_d, (N, B, K, V))
    if quant is not None:
        d = np.round(d / quant) * quant
    if peak > 0:
        hot = rng.random((N, B, K)) < peak
        d[hot, rng.integers(0, V)] += 12.0
    return bf16_bits_from_f64(t), bf16_bits_from_f64(d)


def run_tree(binding, t, d, topk, T=1.0):
    N, B, K, V = d.shape
    ws = binding.make_tree_workspace(B, K, N, V, topk)
    g = binding.spec_tree_gamma(dev_bf16(t), dev_bf16(d), topk, T, workspace=ws)
    torch.cuda.synchronize()
    assert binding.workspace_fault(ws) == 0, "kernel reported an internal consistency fault"
    assert int(ws.count_nonzero().item()) == 0, "workspace not left zero"
    return to_np(g)


@pytest.mark.parametrize("B,K,N,V,topk", [
    (2, 3, 4, 1, 1), (2, 2, 3, 9, 4), (2, 2, 2, 20, 64), (3, 2, 5, 513, 8), (2, 3, 3, 16384, 16),
    (2, 2, 3, 16385, 64), (1, 1, 2, 6000, 64), (4, 5, 7, 40000, 8), (2, 3, 2, 33000, 1), (1, 2, 3, 70001, 33),
])
def test_tree_shapes(binding, B, K, N, V, topk):
    banner(f"tree B={B} K={K} N={N} V={V} topk={topk}")
    t, d = tree_case(B, K, N, V, seed=V + topk)
    got = run_tree(binding, t, d, topk)
    ref = oracle.spec_tree_gamma(t, d, topk)
    w = assert_rel(got, ref, label="tree gamma")
    print(f"max rel err {w:.2e}")


@pytest.mark.parametrize("quant,topk", [(0.5, 8), (1.0, 16), (2.0, 64), (4.0, 3)])
def test_tree_ties_go_to_smaller_id(binding, quant, topk):
    banner(f"tree ties quant={quant} topk={topk}")
    t, d = tree_case(2, 3, 4, 20000, seed=int(quant * 10) + topk, quant=quant)
    got = run_tree(binding, t, d, topk)
    ref = oracle.spec_tree_gamma(t, d, topk)
    assert_rel(got, ref, label="tree gamma ties")


@pytest.mark.parametrize("case,topk", [("negative", 8), ("negative", 64), ("zero", 8), ("zero", 33)])
def test_tree_nonpositive_threshold(binding, case, topk):
    """Pieces whose threshold (the topk-th best lane maximum) is negative or zero, on
    quantised logits so that many tie with it, and with -0 beside +0 in the zero case: the
    kernel ranks such pieces on unpacked values rather than on the raw words."""
    banner(f"tree threshold {case} topk={topk}")
    rng = np.random.default_rng(topk + (1 if case == "zero" else 2))
    B, K, N, V = 2, 2, 3, 20000
    t = bf16_bits_from_f64(rng.normal(0, 4, (B, K + 1, V)))
    if case == "negative":
        d = bf16_bits_from_f64(-np.round(np.abs(rng.normal(0, 2, (N, B, K, V))) / 0.25) * 0.25 - 0.5)
    else:
        d = bf16_bits_from_f64(np.minimum(0.0, np.round(rng.normal(-6, 2, (N, B, K, V)))))
        zeros = d == 0
        d[zeros & (rng.random(d.shape) < 0.5)] = 0x8000  # -0
    got = run_tree(binding, t, d, topk)
    ref = oracle.spec_tree_gamma(t, d, topk)
    assert_rel(got, ref, label=f"tree {case} threshold")


def test_tree_all_equal_drafter_logits(binding):
    """Every logit tied: the children are the first topk ids of the row."""
    banner("tree all-equal drafter rows")
    rng = np.random.default_rng(7)
    V = 40000
    t = bf16_bits_from_f64(rng.normal(0, 4, (2, 2, V)))
    d = np.zeros((3, 2, 2, V), dtype=np.uint16)
    for topk in (1, 5, 64):
        got = run_tree(binding, t, d, topk)
        for b in range(2):
            for k in range(2):
                pt = oracle.softmax_t(oracle.widen_bf16(t[b, k]), 1.0)
                assert_rel(got[b, k], np.full(3, pt[:topk].sum()), label="first ids")


def test_tree_peaked_temperature_and_masked(binding):
    banner("tree peaked rows, T=0.7, masked logits")
    t, d = tree_case(3, 2, 4, 30000, seed=11, peak=0.5)
    d = d.copy()
    d[0, 0, 0, :5000] = 0xFF80              # -inf: never better than a finite logit
    t = t.copy()
    t[1, 1, 100:200] = 0xFF80                # target tokens with no mass
    got = run_tree(binding, t, d, 8, T=0.7)
    ref = oracle.spec_tree_gamma(t, d, 8, 0.7)
    assert_rel(got, ref, label="tree peaked")


def test_tree_repeat_one_workspace(binding):
    """Two calls of different shapes on one workspace: each leaves it zero, results unchanged."""
    banner("tree repeat on one workspace")
    ws = binding.make_tree_workspace(4, 5, 7, 20000, 16)
    t1, d1 = tree_case(4, 5, 7, 20000, seed=3)
    t2, d2 = tree_case(2, 3, 7, 3000, seed=4)
    a = to_np(binding.spec_tree_gamma(dev_bf16(t1), dev_bf16(d1), 16, workspace=ws))
    b = to_np(binding.spec_tree_gamma(dev_bf16(t2), dev_bf16(d2), 16, workspace=ws))
    c = to_np(binding.spec_tree_gamma(dev_bf16(t1), dev_bf16(d1), 16, workspace=ws))
    torch.cuda.synchronize()
    assert binding.workspace_fault(ws) == 0 and int(ws.count_nonzero().item()) == 0
    np.testing.assert_array_equal(a, c)
    assert_rel(b, oracle.spec_tree_gamma(t2, d2, 16), label="tree second shape")


def test_tree_hedge_eval_size_sampled(binding):
    """The HedgeSpec evaluation shape B=32 K=5 N=7 V=128256 with 8 children per node; the
    oracle checks 6 (sequence, position) nodes, all 7 drafters each."""
    banner("tree full B=32 K=5 N=7 V=128256 topk=8")
    x = gen.make_gamma_inputs(gen.HEDGE_EVAL)
    got = run_tree(binding, x["target"], x["drafts"], 8)
    for b, k in [(0, 0), (5, 4), (13, 2), (21, 1), (27, 3), (31, 4)]:
        pt = oracle.softmax_t(oracle.widen_bf16(x["target"][b, k]), 1.0)
        ref = [oracle.tree_gamma(pt, oracle.widen_bf16(x["drafts"][i, b, k]), 8) for i in range(7)]
        assert_rel(got[b, k], np.array(ref), label=f"tree full ({b},{k})")


def test_tree_merge_overflow_bound_at_max_vocab(binding):
    """V = 2^20 (256 pieces of 4096 tokens), every piece holding the same logits: each piece's
    64th best record ties on the logit and loses on the id to piece 0's, so ~16k records reach
    the merge's first bound and the second bound (the 64th best of the pieces' bests) must take
    over.  The children are the best token of pieces 0..63."""
    banner("tree merge overflow V=2^20 topk=64")
    V, topk = 1 << 20, 64
    rng = np.random.default_rng(70)
    piece = rng.normal(0, 2.0, 4096)
    d = bf16_bits_from_f64(np.tile(piece, V // 4096)).reshape(1, 1, 1, V)
    t = bf16_bits_from_f64(rng.normal(0, 4.0, (1, 1, V)))
    got = run_tree(binding, t, d, topk)
    ref = oracle.spec_tree_gamma(t, d, topk)
    assert_rel(got, ref, label="tree merge overflow")
    kids = oracle.tree_children(oracle.widen_bf16(d[0, 0, 0]), topk)
    assert np.all(kids // 4096 < 64) and len(set((kids % 4096).tolist())) == 1


def test_tree_single_drafter_position_max_topk_ragged(binding):
    banner("tree N=1 K=1 V=100003 topk=64 and topk=1")
    t, d = tree_case(3, 1, 1, 100003, seed=71)
    for topk in (1, 64):
        got = run_tree(binding, t, d, topk)
        assert_rel(got, oracle.spec_tree_gamma(t, d, topk), label=f"tree N=1 topk={topk}")
