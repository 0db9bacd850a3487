"""Pins of the oracle's Cactus functions (paper note on Cactus, Key designs 1-3).

Checked against what the note fixes: delta = 0 is plain speculative sampling;
gamma* lies in [q(n), 1] and grows with delta; the bonus is largest at
q(n) = 0.5; Corollary 6 (gamma* <= 0.5 implies KL(h || q) <= delta); the
second-order Taylor origin of gamma* (the KL constraint is tight to first
order in delta); and brute force over a tiny vocabulary.
"""

import math

import numpy as np
from scipy import stats

import oracle
from oracle import spec_oracle as so


def kl(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m = a > 0
    return float(np.sum(a[m] * np.log(a[m] / b[m])))


def rand_rows(rng, V, K, sigma=2.0):
    zt = rng.normal(0, sigma, (K + 1, V))
    zd = zt[:K] + rng.normal(0, 1.0, (K, V))
    return oracle.softmax_t(zt, 1.0), oracle.softmax_t(zd, 1.0)


def test_delta_zero_is_sps_bit_identical():
    """delta = 0 turns Cactus into SpS (Key design 1); reading R16: h == pt bit for bit."""
    rng = np.random.default_rng(0)
    for trial in range(200):
        V, K = int(rng.integers(2, 60)), int(rng.integers(1, 6))
        pt, pd = rand_rows(rng, V, K)
        toks = np.array([rng.choice(V, p=pd[k]) for k in range(K)])
        r = rng.random(K, dtype=np.float32)
        u = rng.random(K + 1, dtype=np.float32)
        a = oracle.sps_sequence(pt, pd, toks, r, u)
        c = oracle.cactus_sequence(pt, pd, toks, r, u, 0.0)
        assert a["A"] == c["A"] and a["token"] == c["token"]
        np.testing.assert_array_equal(a["accept"], c["accept"])
        np.testing.assert_array_equal(a["margin_r"], c["margin_r"])
        assert a["margin_u"] == c["margin_u"]
        h, g = oracle.cactus_target(pt[0], int(toks[0]), 0.0)
        assert np.array_equal(h, pt[0]) and g == pt[0][toks[0]]


def test_gamma_star_range_monotone_and_bonus_peak():
    cs = np.linspace(0.0, 1.0, 401)
    for delta in [0.0, 0.01, 0.1, 0.5, 1.0, 3.0]:
        g = np.array([oracle.cactus_gamma_star(c, delta) for c in cs])
        assert np.all(g >= cs - 1e-15) and np.all(g <= 1.0)
    for c in [0.01, 0.2, 0.5, 0.9]:
        gs = [oracle.cactus_gamma_star(c, d) for d in np.linspace(0, 2, 50)]
        assert np.all(np.diff(gs) >= 0.0)
    # the bonus gamma* - q(n) peaks at q(n) = 0.5 (Key design 3), for a delta small enough not to clip
    bonus = np.array([oracle.cactus_gamma_star(c, 0.02) - c for c in cs])
    assert abs(cs[int(np.argmax(bonus))] - 0.5) < 1e-9
    # c = 1 -> gamma* = 1, c = 0 -> gamma* = 0 for every delta
    assert oracle.cactus_gamma_star(1.0, 0.7) == 1.0 and oracle.cactus_gamma_star(0.0, 0.7) == 0.0


def test_target_h_closed_form_properties():
    """Key design 2 (Theorem 2): h_n = gamma*, the rest is q rescaled; h is a distribution."""
    rng = np.random.default_rng(1)
    for _ in range(100):
        V = int(rng.integers(2, 40))
        pt = oracle.softmax_t(rng.normal(0, 2, V), 1.0)
        n = int(rng.integers(V))
        delta = float(rng.choice([0.0, 0.05, 0.5, 1.0, 4.0]))
        h, g = oracle.cactus_target(pt, n, delta)
        assert abs(h.sum() - 1.0) < 1e-12 and np.all(h >= 0.0)
        assert h[n] == g
        others = np.arange(V) != n
        if g < 1.0:
            # proportional to pt away from n
            ratio = h[others] / pt[others]
            assert np.ptp(ratio) < 1e-12
    # c == 1 (one-hot verifier): h one-hot too (s := 0)
    h, g = oracle.cactus_target(np.array([0.0, 1.0, 0.0]), 1, 0.5)
    np.testing.assert_array_equal(h, [0.0, 1.0, 0.0])


def test_corollary6_kl_within_budget():
    """Corollary 6: when gamma* <= 0.5 the Taylor solution satisfies KL(h || q) <= delta."""
    rng = np.random.default_rng(2)
    checked = 0
    for _ in range(3000):
        V = int(rng.integers(2, 30))
        pt = oracle.softmax_t(rng.normal(0, 2.5, V), 1.0)
        n = int(rng.integers(V))
        delta = float(10 ** rng.uniform(-4, 0.5))
        h, g = oracle.cactus_target(pt, n, delta)
        if g <= 0.5:
            checked += 1
            assert kl(h, pt) <= delta * (1 + 1e-12), (pt[n], delta, kl(h, pt))
    assert checked > 500


def test_taylor_constraint_tight_for_small_delta():
    """gamma* is the second-order expansion of KL(gamma || q(n)) = delta around gamma = q(n)
    (Key design 3), so KL(h || q) / delta -> 1 as delta -> 0."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(3, 30))
        pt = oracle.softmax_t(rng.normal(0, 1.0, V), 1.0)
        n = int(rng.integers(V))
        if not 0.05 < pt[n] < 0.95:
            continue
        delta = 1e-6
        h, g = oracle.cactus_target(pt, n, delta)
        assert abs(kl(h, pt) / delta - 1.0) < 0.02


def test_planted_taylor_mistake_is_caught(monkeypatch):
    """A dropped factor 2 inside the square root fails the tightness pin."""
    monkeypatch.setattr(so, "cactus_gamma_star", lambda c, d: min(c + math.sqrt(d * c * (1.0 - c)), 1.0))
    pt = oracle.softmax_t(np.array([0.1, 0.4, -0.3, 0.0]), 1.0)
    h, g = so.cactus_target(pt, 1, 1e-6)
    assert abs(kl(h, pt) / 1e-6 - 1.0) > 0.2


def _h_alg(pt, pd, delta):
    """Output law of one Cactus position built from the per-candidate targets:
    h_alg(x) = sum_n pd(n) [phi(n) 1[x=n] + (1 - phi(n)) g_n(x)] (reading R15)."""
    V = pt.shape[0]
    law = np.zeros(V)
    for n in range(V):
        if pd[n] == 0:
            continue
        h, gstar = oracle.cactus_target(pt, n, delta)
        phi = min(1.0, gstar / pd[n])
        g = np.maximum(h - pd, 0.0)
        law[n] += pd[n] * phi
        if phi < 1.0:
            law += pd[n] * (1.0 - phi) * g / g.sum()
    return law


def test_brute_force_single_position_law():
    """Monte-Carlo frequencies of the oracle's Cactus position match the exact mixture law."""
    rng = np.random.default_rng(4)
    V, n_mc = 4, 40000
    pt = oracle.softmax_t(rng.normal(0, 1.2, V), 1.0)
    pd = oracle.softmax_t(rng.normal(0, 1.2, V), 1.0)
    for delta in [0.0, 0.3]:
        law = _h_alg(pt, pd, delta)
        assert abs(law.sum() - 1.0) < 1e-12
        if delta == 0.0:
            np.testing.assert_allclose(law, pt, atol=1e-12)   # SpS is lossless
        counts = np.zeros(V)
        rows_t = np.stack([pt, pt])
        for _ in range(n_mc):
            n = int(rng.choice(V, p=pd))
            res = oracle.cactus_sequence(rows_t, pd[None, :], [n], rng.random(1, dtype=np.float32),
                                         rng.random(2, dtype=np.float32), delta)
            counts[n if res["A"] == 1 else res["token"]] += 1
        assert stats.chisquare(counts, n_mc * law).pvalue > 1e-4
        if delta > 0:
            # Theorem 3's second term: the output is no farther from q than the draft is
            assert kl(law, pt) <= kl(pd, pt) + 1e-12
            # and the acceptance rate is higher than SpS's
            acc_c = sum(pd[n] * min(1.0, oracle.cactus_gamma_star(pt[n], delta) / pd[n]) for n in range(V))
            assert acc_c >= oracle.acceptance_mass(pt, pd) - 1e-12


def test_always_reject_when_candidate_has_no_verifier_mass():
    pt = oracle.softmax_t(np.array([-np.inf, 0.0, 0.0]), 1.0)
    pd = oracle.softmax_t(np.array([0.0, -1.0, -1.0]), 1.0)
    res = oracle.cactus_sequence(np.stack([pt, pt]), pd[None, :], [0], [0.0], [0.5, 0.5], 1.0)
    assert res["A"] == 0 and res["gamma_star"][0] == 0.0 and res["token"] in (1, 2)


# ---------------------------------------------------------------------------
# Exact-KL gamma* (Key design 2's root, without Key design 3's Taylor step)
# ---------------------------------------------------------------------------

def _binary_kl_scipy(g, c):
    """The divergence of the two-outcome law (g, 1-g) from (c, 1-c), by scipy's rel_entr."""
    from scipy.special import rel_entr
    return float(rel_entr(g, c) + rel_entr(1.0 - g, 1.0 - c))


def test_exact_kl_inverts_the_divergence():
    """For a chosen gamma in (c, 1), delta := KL((g,1-g) || (c,1-c)) must give gamma back."""
    rng = np.random.default_rng(10)
    for _ in range(800):
        c = float(10 ** rng.uniform(-8, 0)) * 0.999
        g = c + (1.0 - c) * float(rng.uniform(0.001, 0.999))
        delta = _binary_kl_scipy(g, c)
        got = oracle.cactus_gamma_star_kl(c, delta)
        assert abs(got - g) <= 1e-9 * (g - c) + 4e-16, (c, g, delta, got)


def test_exact_kl_full_vocab_divergence_equals_budget():
    """KL(h || pt) over the whole vocabulary, by scipy, is delta when gamma* < 1 and at most
    delta when clipped to 1."""
    from scipy.special import rel_entr
    rng = np.random.default_rng(11)
    clipped = tight = 0
    for _ in range(800):
        V = int(rng.integers(2, 50))
        pt = oracle.softmax_t(rng.normal(0, 2.5, V), 1.0)
        n = int(rng.integers(V))
        delta = float(10 ** rng.uniform(-5, 0.7))
        h, g = oracle.cactus_target(pt, n, delta, exact_kl=True)
        assert abs(h.sum() - 1.0) < 1e-12 and h[n] == g and g >= pt[n]
        d = float(np.sum(rel_entr(h, pt)))
        if g < 1.0:
            tight += 1
            assert abs(d - delta) <= 1e-9 * delta, (pt[n], delta, d)
        else:
            clipped += 1
            assert d <= delta * (1 + 1e-12) and -math.log(pt[n]) <= delta * (1 + 1e-12)
    assert tight > 300 and clipped > 10


def test_exact_kl_is_the_constrained_optimum_brute_force():
    """Key design 1 on a 3-token vocabulary: the largest h_n over a grid of distributions h with
    KL(h || q) <= delta matches gamma* (the grid also tries the splits Theorem 2 rules out)."""
    from scipy.special import rel_entr
    q = np.array([0.25, 0.15, 0.6])
    step = 1.0 / 1500
    grid = np.arange(0.0, 1.0 + step / 2, step)
    hn, ha = np.meshgrid(grid, grid, indexing="ij")
    hb = 1.0 - hn - ha
    ok = hb >= -1e-12
    for n in range(3):
        others = [i for i in range(3) if i != n]
        H = np.zeros(hn.shape + (3,))
        H[..., n], H[..., others[0]], H[..., others[1]] = hn, ha, np.maximum(hb, 0.0)
        D = np.sum(rel_entr(H, q), axis=-1)
        for delta in [0.01, 0.1, 0.4]:
            best = float(hn[ok & (D <= delta)].max())
            g = oracle.cactus_gamma_star_kl(float(q[n]), delta)
            assert g - 2 * step <= best <= g + 1e-12, (n, delta, best, g)


def test_exact_kl_edges_monotone_and_corollary6():
    """delta = 0 and c = 0 give c; -log c <= delta gives 1; gamma* grows with delta; Corollary 6
    (Taylor gamma* <= 0.5 keeps KL <= delta) makes the Taylor value a lower bound there; the
    Taylor step is exact to first order as delta -> 0."""
    assert oracle.cactus_gamma_star_kl(0.3, 0.0) == 0.3
    assert oracle.cactus_gamma_star_kl(0.0, 2.0) == 0.0
    assert oracle.cactus_gamma_star_kl(1.0, 0.5) == 1.0
    assert oracle.cactus_gamma_star_kl(0.7, -math.log(0.7)) == 1.0
    assert oracle.cactus_gamma_star_kl(0.7, 0.999 * -math.log(0.7)) < 1.0
    rng = np.random.default_rng(12)
    below = 0
    for _ in range(400):
        c = float(rng.uniform(1e-6, 1.0))
        ds = np.sort(10 ** rng.uniform(-6, 0.5, 6))
        gs = [oracle.cactus_gamma_star_kl(c, float(d)) for d in ds]
        assert all(c <= g <= 1.0 for g in gs) and np.all(np.diff(gs) >= 0.0)
        for d, g in zip(ds, gs):
            gt = oracle.cactus_gamma_star(c, float(d))
            if gt <= 0.5:
                below += 1
                assert gt <= g * (1 + 1e-15), (c, d, gt, g)
    assert below > 200
    for c in [0.05, 0.3, 0.5, 0.8]:
        ratio = (oracle.cactus_gamma_star_kl(c, 1e-10) - c) / (oracle.cactus_gamma_star(c, 1e-10) - c)
        assert abs(ratio - 1.0) < 1e-3


def test_exact_kl_delta_zero_is_sps():
    rng = np.random.default_rng(13)
    for _ in range(100):
        V, K = int(rng.integers(2, 40)), int(rng.integers(1, 6))
        pt, pd = rand_rows(rng, V, K)
        toks = np.array([rng.choice(V, p=pd[k]) for k in range(K)])
        r = rng.random(K, dtype=np.float32)
        u = rng.random(K + 1, dtype=np.float32)
        a = oracle.sps_sequence(pt, pd, toks, r, u)
        c = oracle.cactus_sequence(pt, pd, toks, r, u, 0.0, exact_kl=True)
        assert a["A"] == c["A"] and a["token"] == c["token"] and a["margin_u"] == c["margin_u"]
        np.testing.assert_array_equal(a["accept"], c["accept"])


def test_exact_kl_law_brute_force():
    """Monte-Carlo frequencies of an exact-KL Cactus position match its mixture law, and its
    acceptance is at least the Taylor one's where Corollary 6 applies."""
    rng = np.random.default_rng(14)
    V, n_mc, delta = 4, 30000, 0.3
    pt = oracle.softmax_t(rng.normal(0, 1.2, V), 1.0)
    pd = oracle.softmax_t(rng.normal(0, 1.2, V), 1.0)
    law = np.zeros(V)
    for n in range(V):
        h, g = oracle.cactus_target(pt, n, delta, exact_kl=True)
        phi = min(1.0, g / pd[n])
        w = np.maximum(h - pd, 0.0)
        law[n] += pd[n] * phi
        if phi < 1.0:
            law += pd[n] * (1.0 - phi) * w / w.sum()
    assert abs(law.sum() - 1.0) < 1e-12
    counts = np.zeros(V)
    rows_t = np.stack([pt, pt])
    for _ in range(n_mc):
        n = int(rng.choice(V, p=pd))
        res = oracle.cactus_sequence(rows_t, pd[None, :], [n], rng.random(1, dtype=np.float32),
                                     rng.random(2, dtype=np.float32), delta, exact_kl=True)
        counts[n if res["A"] == 1 else res["token"]] += 1
    assert stats.chisquare(counts, n_mc * law).pvalue > 1e-4


def test_planted_kl_mistake_is_caught(monkeypatch):
    """Dropping the (1 - g) term of the divergence fails the inversion pin."""
    monkeypatch.setattr(so, "cactus_kl", lambda g, c: g * (math.log(g) - math.log(c)) if g > 0 else 0.0)
    c, g = 0.2, 0.45
    got = so.cactus_gamma_star_kl(c, _binary_kl_scipy(g, c))
    assert abs(got - g) > 1e-3


def _kl_mp(g, c):
    """The two-outcome divergence at 700 significant digits (enough for 1 - g with g ~ 1e-300)."""
    import mpmath
    with mpmath.workdps(700):
        g, c = mpmath.mpf(g), mpmath.mpf(c)
        t1 = g * mpmath.log(g / c) if g > 0 else mpmath.mpf(0)
        t2 = (1 - g) * mpmath.log((1 - g) / (1 - c)) if g < 1 else mpmath.mpf(0)
        return t1 + t2


def _extreme_pairs(rng, n):
    out = []
    for _ in range(n):
        c = float(10 ** rng.uniform(-300, 0)) * 0.9999
        if rng.random() < 0.5:
            g = c * (1.0 + float(10 ** rng.uniform(-12, 3)))   # g near c, or decades above it
        else:
            g = c + (1.0 - c) * float(rng.random())
        out.append((min(g, 1.0), c))
    return out


def test_kl_divergence_matches_high_precision():
    """cactus_kl against 700-digit arithmetic, from c = 1e-300 up, g from c (1 + 1e-12) to 1."""
    rng = np.random.default_rng(15)
    for g, c in _extreme_pairs(rng, 1500):
        ref = float(_kl_mp(g, c))
        if ref == 0.0:
            continue
        assert abs(so.cactus_kl(g, c) - ref) <= 1e-13 * ref, (g, c, so.cactus_kl(g, c), ref)


def test_exact_kl_root_matches_high_precision():
    """delta := the 700-digit divergence of a chosen g gives g back, to a few ulps (or to 1e-12
    of g - c), from c = 1e-300 up."""
    rng = np.random.default_rng(16)
    for g, c in _extreme_pairs(rng, 300):
        if not g < 1.0:
            continue
        delta = float(_kl_mp(g, c))
        if delta == 0.0:
            continue
        got = oracle.cactus_gamma_star_kl(c, delta)
        assert abs(got - g) <= 4 * np.spacing(g) + 1e-12 * (g - c), (g, c, delta, got)
