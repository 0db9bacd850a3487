"""Pins of the oracle's draft-tree gamma ([NB] Key design 1, the tree case; reading R24).

Checked against what does not depend on the oracle's own selection code: a
drafter keeping every token makes gamma 1; a drafter equal to the target keeps
the best k tokens, so gamma is the largest target mass of any k-subset (brute
force over all subsets); one child is numpy's first argmax; equal logits keep
the first k ids; and gamma grows with k.
"""

import itertools

import numpy as np

import oracle
from oracle import spec_oracle as so


def test_all_tokens_kept_gives_one():
    rng = np.random.default_rng(0)
    for V in [1, 2, 5, 17]:
        pt = oracle.softmax_t(rng.normal(0, 2, V), 1.0)
        z = rng.normal(0, 2, V)
        assert abs(oracle.tree_gamma(pt, z, V) - 1.0) < 1e-12
        assert abs(oracle.tree_gamma(pt, z, V + 10) - 1.0) < 1e-12


def test_drafter_equal_to_target_keeps_best_subset():
    rng = np.random.default_rng(1)
    for _ in range(60):
        V = int(rng.integers(2, 9))
        z = np.round(rng.normal(0, 1.5, V), 1)          # rounded: ties happen
        pt = oracle.softmax_t(z, 1.0)
        for k in range(1, V + 1):
            best = max(sum(pt[list(c)]) for c in itertools.combinations(range(V), k))
            assert abs(oracle.tree_gamma(pt, z, k) - best) < 1e-12


def test_single_child_is_first_argmax():
    rng = np.random.default_rng(2)
    for _ in range(200):
        V = int(rng.integers(1, 30))
        z = np.round(rng.normal(0, 1, V), 0)            # many ties
        pt = oracle.softmax_t(rng.normal(0, 1, V), 1.0)
        assert oracle.tree_children(z, 1)[0] == int(np.argmax(z))
        assert oracle.tree_gamma(pt, z, 1) == pt[int(np.argmax(z))]


def test_equal_logits_keep_first_ids_and_gamma_grows_with_k():
    pt = oracle.softmax_t(np.array([0.3, -1.0, 2.0, 0.0, 0.5]), 1.0)
    np.testing.assert_array_equal(oracle.tree_children(np.zeros(5), 3), [0, 1, 2])
    assert abs(oracle.tree_gamma(pt, np.zeros(5), 3) - pt[:3].sum()) < 1e-15
    rng = np.random.default_rng(3)
    for _ in range(50):
        V = int(rng.integers(2, 40))
        pt = oracle.softmax_t(rng.normal(0, 2, V), 1.0)
        z = rng.normal(0, 2, V)
        g = [oracle.tree_gamma(pt, z, k) for k in range(1, V + 1)]
        assert np.all(np.diff(g) >= 0.0) and g[-1] <= 1.0 + 1e-12


def test_children_are_the_k_largest():
    """Every kept logit is at least every dropped one, with ties kept by smaller id."""
    rng = np.random.default_rng(4)
    for _ in range(200):
        V = int(rng.integers(2, 60))
        z = np.round(rng.normal(0, 1, V), 1)
        k = int(rng.integers(1, V + 1))
        kept = set(oracle.tree_children(z, k).tolist())
        assert len(kept) == k
        for a in kept:
            for d in set(range(V)) - kept:
                assert z[a] > z[d] or (z[a] == z[d] and a < d)


def test_batched_layout():
    rng = np.random.default_rng(5)
    B, K, N, V = 2, 3, 4, 50
    t = rng.integers(0, 1 << 16, (B, K + 1, V), dtype=np.uint16) & np.uint16(0x3FFF)  # finite bf16
    d = rng.integers(0, 1 << 16, (N, B, K, V), dtype=np.uint16) & np.uint16(0x3FFF)
    g = oracle.spec_tree_gamma(t, d, 5, 0.8)
    assert g.shape == (B, K, N)
    pt = oracle.softmax_t(oracle.widen_bf16(t[1, 2]), 0.8)
    assert g[1, 2, 3] == oracle.tree_gamma(pt, oracle.widen_bf16(d[3, 1, 2]), 5)


def test_planted_tie_rule_mistake_is_caught(monkeypatch):
    """Ties broken towards the larger id fail the equal-logit pin."""
    def wrong(z, topk):
        z = np.asarray(z, dtype=np.float64)
        order = np.lexsort((-np.arange(z.shape[0]), -z))
        return order[:topk]
    monkeypatch.setattr(so, "tree_children", wrong)
    pt = oracle.softmax_t(np.array([0.3, -1.0, 2.0, 0.0, 0.5]), 1.0)
    assert abs(so.tree_gamma(pt, np.zeros(5), 3) - pt[:3].sum()) > 1e-3
