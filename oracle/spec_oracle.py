"""Plain float64 CPU oracle for batched speculative-sampling verification.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke entry point and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
module imports nothing from the product package: the two share no code.

Everything here is the slow, obviously-correct definition of what the GPU path
computes, in numpy float64.  bf16 logits are widened exactly to float64;
uniforms are float32 values (multiples of 2**-24), also exact in float64.

Sources (cited by page title and section, never by line):

* [LT]  "Speculative Decoding 为什么是 Lossless 的 — 详细证明教程" (a tutorial that
  restates Leviathan et al. 2023, App. A.1 and Chen et al. 2023, Thm 1).
  It uses p = target and q = draft.
* [NB]  Paper note "Not-a-Bandit: Provably No-Regret Drafter Selection in
  Speculative Decoding for LLMs" (HedgeSpec), sections "关键设计" 1-4.
* [CA]  Paper note "Cactus: Accelerating Auto-Regressive Decoding with
  Constrained Acceptance Speculative Sampling", "方法详解" / "关键设计" 1-3.
  Cactus writes p = draft and q = verifier; this module always says
  ``pt`` (target / verifier softmax) and ``pd`` (draft softmax).
* [NH]  NormalHedge: K. Chaudhuri, Y. Freund, D. Hsu, "A parameter-free
  hedging algorithm", NIPS 2009.  [NB] names NormalHedge as its learner but
  does not print the update; it is restated here from that paper.

Readings of points the pages leave open (each is listed again in the design
notes of the repository):

R1  Estimator ([NB] Key design 2; the formula did not survive on the page):
    L = 1 + sum_{k=1..K} gamma_k * prod_{j<k} a_j,  a_j = min(1, pd(x_j)/pt(x_j))
    at the realised trajectory tokens x_j.  It is the only form consistent
    with every stated property (one trajectory, unbiased, range [1, K+1],
    gamma_k is a total acceptance probability, not the realised token's).
R2  Loss ([NB] Key design 3; formula lost): f = (K + 1) - L.
R3  NormalHedge update: [NH], fp64 bisection for the scale c.
R8  Accept comparison is strict: accept iff r < ratio ([LT] §2.2, §5.1).
R9  Resampling is an inverse CDF over ascending token ids: the smallest j
    with C_j > u * sum(w).  Zero-mass tokens are never chosen.
R10 If a position rejects while its residual mass is exactly zero (only
    possible through rounding), sample from that position's target
    distribution with the same uniform.
R11 Bonus token when all K drafts are accepted: inverse CDF of pt at target
    row K with uniform u[K] ([LT] §9.1: the target scores K+1 positions).
R12 Uniform layout: r[K] for the accept tests; u[K+1] where slot A is used
    when the first rejection is at A, slot K for the bonus.
R15 Cactus acceptance phi(n) = min(1, h_n / pd(n)) and recovery
    g = (h - pd)+ / sum(h - pd)+  ([CA] Framework: SpS is the case h = pt).
R16 Cactus: c = 1 gives gamma* = 1 and s := 0; delta = 0 gives s = 1.0
    exactly, so h == pt bit for bit and the position is plain SpS.
R17 Cactus bonus is drawn from pt at row m (h is defined per candidate only).
R25 Acceptance-probability objective ([NB] Key design 3): f = 1 - gamma per
    position; a chunk's K position losses enter the learner as their sum (the
    exponential weights depend on the cumulative loss only).  Censoring delay:
    round s's losses are usable once K more tokens (accepted_len + 1 per round)
    have been verified after round s.
R24 Draft-tree gamma ([NB] Key design 1, the tree case): a drafter's children
    at a node are its topk tokens by logit, ties to the smaller id; gamma is
    the target probability of that set.
R23 Exact-KL Cactus: gamma* is the largest g in [c, 1] whose target h keeps
    KL(h || pt) <= delta ([CA] Key design 1's optimisation, Key design 2's
    root), 1 when even the one-hot target fits the budget (-log c <= delta),
    and c when delta = 0 or c = 0.
"""

from __future__ import annotations

import decimal
import functools
import math
import struct

import numpy as np

__all__ = [
    "widen_bf16",
    "softmax_t",
    "accept_ratio",
    "accept_test",
    "inverse_cdf",
    "cdf_neighbours",
    "residual_weights",
    "acceptance_mass",
    "sps_sequence",
    "spec_verify",
    "cactus_gamma_star",
    "cactus_kl",
    "cactus_gamma_star_kl",
    "cactus_target",
    "cactus_sequence",
    "spec_cactus_verify",
    "realised_ratio",
    "acceptance_length_estimate",
    "spec_counterfactual_gamma",
    "tree_children",
    "tree_gamma",
    "spec_tree_gamma",
    "normalhedge_scale",
    "normalhedge_weights",
    "normalhedge_step",
    "normalhedge_select",
    "hedge_update",
    "hedge_delayed_rounds",
    "acceptance_prob_loss",
    "hedge_exp_step",
    "hedge_exp_update",
    "censored_delays",
    "hedge_delayed_rounds_rule",
    "hedge_censored_rounds",
]


# ---------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------

def widen_bf16(bits) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def softmax_t(z, temperature: float) -> np.ndarray:
    """Temperature softmax over the last axis, float64.

    [LT] §8 Q4: temperature (and any other shaping) must be folded into BOTH
    the target and the draft distribution before any ratio is formed, so the
    same T is applied to every row.
    """
    if not (temperature > 0.0 and math.isfinite(temperature)):
        raise ValueError("temperature must be finite and > 0")
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("every row needs at least one finite logit")
    w = np.exp((z - m) / temperature)
    return w / np.sum(w, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Single-position pieces
# ---------------------------------------------------------------------------

def accept_ratio(pt_t: float, pd_t: float) -> float:
    """p(t)/q(t) for the drafted token t ([LT] §2.2 notation a(x), r).

    A drafted token with zero draft mass has ratio +inf when the target gives
    it mass, else 0 (never accepted).
    """
    if pd_t > 0.0:
        return pt_t / pd_t
    return math.inf if pt_t > 0.0 else 0.0


def accept_test(pt_t: float, pd_t: float, r: float):
    """Accept iff r < p(t)/q(t)  ([LT] §5.1 step 2, strict, reading R8).

    Returns (accept, margin) with margin = |r - ratio| (the distance of the
    decision from a tie; +inf when the ratio is infinite).
    """
    ratio = accept_ratio(pt_t, pd_t)
    margin = math.inf if math.isinf(ratio) else abs(r - ratio)
    return bool(r < ratio), margin


def inverse_cdf(w, u: float):
    """Inverse CDF of the non-negative weights ``w`` at uniform ``u`` (R9).

    Returns (j, margin): j is the smallest index with C_j > u * C_{V-1},
    where C is the sequential running sum in ascending index order; margin is
    min(x - C_{j-1}, C_j - x) / C_{V-1}, the relative distance of the
    threshold x = u * C_{V-1} from the two CDF steps around j.  If rounding
    leaves no qualifying j, the last positive-mass index is returned with
    margin 0.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)  # left-to-right running sum
    total = c[-1]
    if not total > 0.0:
        raise ValueError("inverse_cdf needs positive total mass")
    x = u * total
    j = int(np.searchsorted(c, x, side="right"))  # first C_j > x
    if j >= w.shape[0]:
        return int(np.flatnonzero(w > 0.0)[-1]), 0.0
    prev = c[j - 1] if j > 0 else 0.0
    return j, float(min(x - prev, c[j] - x) / total)


def cdf_neighbours(w, j: int):
    """The positive-mass indices just before and just after j in the inverse-CDF order
    (-1 where there is none): the tokens a draw whose threshold sits within rounding of
    one of j's two CDF steps can land on instead of j (the matching rule's near-tie
    band, reading R13)."""
    pos = np.flatnonzero(np.asarray(w, dtype=np.float64) > 0.0)
    before = pos[pos < j]
    after = pos[pos > j]
    return (int(before[-1]) if before.size else -1), (int(after[0]) if after.size else -1)


def residual_weights(pt, pd) -> np.ndarray:
    """(p - q)+ : the part of the target the draft under-covers ([LT] §2.2, §6.4 Step 3a)."""
    return np.maximum(np.asarray(pt) - np.asarray(pd), 0.0)


def acceptance_mass(pt, pd) -> float:
    """sum_x min(p(x), q(x)) = P(accept) = 1 - TV(p, q)  ([LT] §6.3).

    This is also HedgeSpec's counterfactual acceptance probability of a drafter
    in standard single-draft speculative decoding ([NB] Key design 1).
    """
    return float(np.sum(np.minimum(pt, pd)))


# ---------------------------------------------------------------------------
# Lossless SpS: K-position chain
# ---------------------------------------------------------------------------

def sps_sequence(pt_rows, pd_rows, tokens, r, u):
    """One sequence of standard speculative sampling ([LT] §5.1, §9.1).

    pt_rows [K+1, V] target softmaxes (row K scores the bonus position),
    pd_rows [K, V] draft softmaxes, tokens [K] drafted ids, r [K], u [K+1].

    Every position's accept test is evaluated (position-parallel); the chain
    keeps drafts left to right up to the first rejection A, resamples position
    A from (pt - pd)+ / Z, or draws the bonus from pt at row K when A == K.
    """
    K = len(tokens)
    V = pt_rows.shape[-1]
    accept = np.zeros(K, dtype=bool)
    margin_r = np.zeros(K)
    for k in range(K):
        t = int(tokens[k])
        if not 0 <= t < V:
            raise ValueError("drafted token id out of range")
        accept[k], margin_r[k] = accept_test(pt_rows[k, t], pd_rows[k, t], float(r[k]))
    rejected = np.flatnonzero(~accept)
    A = int(rejected[0]) if rejected.size else K
    if A < K:
        w = residual_weights(pt_rows[A], pd_rows[A])
        if not np.sum(w) > 0.0:  # R10
            w = pt_rows[A]
    else:
        w = pt_rows[K]  # R11 bonus
    token, margin_u = inverse_cdf(w, float(u[A]))
    return {"A": A, "token": token, "accept": accept, "margin_r": margin_r, "margin_u": margin_u,
            "neighbours": cdf_neighbours(w, token)}


def spec_verify(target_bits, draft_bits, draft_tokens, r_accept, u_resample, temperature=1.0):
    """Batched lossless verification, one sequence at a time.

    target_bits [B, K+1, V] uint16 bf16, draft_bits [B, K, V] uint16 bf16,
    draft_tokens [B, K] int, r_accept [B, K] float32, u_resample [B, K+1] float32.
    Returns a dict of arrays: accepted_len [B], out_token [B],
    accept_mask [B, K], margin_r [B, K], margin_u [B].
    """
    B, K1, V = np.shape(target_bits)
    K = K1 - 1
    out = {
        "accepted_len": np.zeros(B, dtype=np.int64),
        "out_token": np.zeros(B, dtype=np.int64),
        "accept_mask": np.zeros((B, K), dtype=bool),
        "margin_r": np.zeros((B, K)),
        "margin_u": np.zeros(B),
        "neighbours": np.zeros((B, 2), dtype=np.int64),
    }
    for b in range(B):
        pt = softmax_t(widen_bf16(target_bits[b]), temperature)
        pd = softmax_t(widen_bf16(draft_bits[b]), temperature)
        res = sps_sequence(pt, pd, draft_tokens[b], r_accept[b], u_resample[b])
        out["accepted_len"][b] = res["A"]
        out["out_token"][b] = res["token"]
        out["accept_mask"][b] = res["accept"]
        out["margin_r"][b] = res["margin_r"]
        out["margin_u"][b] = res["margin_u"]
        out["neighbours"][b] = res["neighbours"]
    return out


# ---------------------------------------------------------------------------
# Cactus constrained acceptance
# ---------------------------------------------------------------------------

def cactus_gamma_star(c: float, delta: float) -> float:
    """gamma* = min{c + sqrt(2 delta c (1 - c)), 1}, c = verifier prob of the candidate.

    [CA] Key design 3: the KL-constrained optimum of Key design 2, expanded to
    second order around gamma = c.
    """
    return min(c + math.sqrt(2.0 * delta * c * (1.0 - c)), 1.0)


def _kl_context(g: float, c: float) -> decimal.Context:
    """A decimal context for the divergence of g from c (0 < c < 1, 0 <= g <= 1).

    Each operation rounds to the context's precision P, so each logarithm
    carries an absolute error of about 10^-P and the sum about (1 + g) 10^-P.
    The divergence is the integral from c to g of (g - t) / (t (1 - t)) dt, so
    it is at least (g - c)^2 / (2 m) with m the largest t (1 - t) between c and
    g.  P is that bound's number of leading zero digits plus 40: the result then
    keeps about 39 correct digits, far more than the float64 it is rounded to.
    """
    d = abs(g - c)
    zeros = 0
    if d > 0.0:
        lo, hi = min(g, c), max(g, c)
        m = 0.25 if lo <= 0.5 <= hi else max(lo * (1.0 - lo), hi * (1.0 - hi))
        bound_log10 = 2.0 * math.log10(d) - math.log10(2.0 * m)
        zeros = max(0, int(math.ceil(-bound_log10)))
    return decimal.Context(prec=40 + zeros, Emin=-decimal.MAX_EMAX, Emax=decimal.MAX_EMAX)


def cactus_kl(g: float, c: float) -> float:
    """KL(h || pt) in nats of the Theorem-2 target h with h_n = g ([CA] Key design 2).

    The tokens other than n keep pt's proportions, so the divergence over the
    vocabulary collapses to the two-outcome one,
        g ln(g / c) + (1 - g) ln((1 - g) / (1 - c)),
    with 0 ln 0 = 0 and +inf where g > 0 meets c = 0 (or g < 1 meets c = 1).
    That definition is evaluated as written, in decimal arithmetic with enough
    digits to survive the cancellation of its two terms near g = c
    (_kl_context), and rounded once to float64.
    """
    if g > 0.0 and c <= 0.0:
        return math.inf
    if g < 1.0 and c >= 1.0:
        return math.inf
    if g == c:
        return 0.0
    ctx = _kl_context(g, c)
    G, C = decimal.Decimal(g), decimal.Decimal(c)
    one = decimal.Decimal(1)
    t1 = ctx.multiply(G, ctx.ln(ctx.divide(G, C))) if g > 0.0 else decimal.Decimal(0)
    G1, C1 = ctx.subtract(one, G), ctx.subtract(one, C)
    t2 = ctx.multiply(G1, ctx.ln(ctx.divide(G1, C1))) if g < 1.0 else decimal.Decimal(0)
    return float(ctx.add(t1, t2))


def _next_double_between(lo: float, hi: float) -> float:
    """The double halfway (in order) between two non-negative doubles lo < hi: the
    midpoint of their bit patterns, which order as integers."""
    a = struct.unpack("<q", struct.pack("<d", lo))[0]
    b = struct.unpack("<q", struct.pack("<d", hi))[0]
    return struct.unpack("<d", struct.pack("<q", (a + b) // 2))[0]


@functools.lru_cache(maxsize=1 << 16)
def cactus_gamma_star_kl(c: float, delta: float) -> float:
    """gamma* as the exact root of the KL constraint, without the Taylor step.

    [CA] Key design 2: gamma* is the root in [c, +inf) of D_KL(h || q) = delta,
    clipped to [c, 1]; Key design 3 notes that this equation (x log x terms)
    has no closed form.  Read as the optimisation of Key design 1: the largest
    g in [c, 1] with cactus_kl(g, c) <= delta.  The divergence grows with g on
    [c, 1], so bisection finds it; the bisection runs over the doubles of the
    bracket themselves (at most 63 halvings) and ends at adjacent doubles, the
    lower of which (inside the budget) is returned.  Reading R23.
    """
    if delta <= 0.0 or c <= 0.0:
        return c            # only g = c keeps the divergence at 0 (or finite, at c = 0)
    if c >= 1.0 or cactus_kl(1.0, c) <= delta:
        return 1.0          # the budget reaches the one-hot target: clipped to 1
    lo, hi = c, 1.0         # cactus_kl(lo) <= delta < cactus_kl(hi)
    while True:
        mid = _next_double_between(lo, hi)
        if mid <= lo or mid >= hi:
            return lo
        if cactus_kl(mid, c) <= delta:
            lo = mid
        else:
            hi = mid


def cactus_target(pt, n: int, delta: float, exact_kl: bool = False):
    """The per-candidate target h of [CA] Key design 2 (Theorem 2 closed form).

    h_n = gamma*, h_i = (1 - gamma*) / (1 - c) * pt_i for i != n.  Reading R16:
    c == 1 forces gamma* = 1 and s := 0.  gamma* is the Taylor form of Key
    design 3, or with ``exact_kl`` the exact root (cactus_gamma_star_kl).
    Returns (h, gamma*).
    """
    pt = np.asarray(pt, dtype=np.float64)
    c = float(pt[n])
    g = cactus_gamma_star_kl(c, delta) if exact_kl else cactus_gamma_star(c, delta)
    s = (1.0 - g) / (1.0 - c) if c < 1.0 else 0.0
    h = s * pt
    h[n] = g
    return h, g


def cactus_sequence(pt_rows, pd_rows, tokens, r, u, delta: float, exact_kl: bool = False):
    """One sequence of Cactus draft-and-verify over m positions.

    Position k accepts its candidate n iff r < gamma*/pd(n) (reading R15: the
    acceptance is min(1, h_n / pd(n))).  At the first rejection A the token is
    drawn from g = (h - pd)+ / Z (R15); if all m are accepted the bonus comes
    from pt at row m (R17).
    """
    m = len(tokens)
    V = pt_rows.shape[-1]
    accept = np.zeros(m, dtype=bool)
    margin_r = np.zeros(m)
    gstar = np.zeros(m)
    for k in range(m):
        n = int(tokens[k])
        if not 0 <= n < V:
            raise ValueError("drafted token id out of range")
        c = float(pt_rows[k, n])
        gstar[k] = cactus_gamma_star_kl(c, delta) if exact_kl else cactus_gamma_star(c, delta)
        accept[k], margin_r[k] = accept_test(gstar[k], pd_rows[k, n], float(r[k]))
    rejected = np.flatnonzero(~accept)
    A = int(rejected[0]) if rejected.size else m
    if A < m:
        h, _ = cactus_target(pt_rows[A], int(tokens[A]), delta, exact_kl)
        w = residual_weights(h, pd_rows[A])
        if not np.sum(w) > 0.0:  # R10, with h as the position's target
            w = h
    else:
        w = pt_rows[m]
    token, margin_u = inverse_cdf(w, float(u[A]))
    return {"A": A, "token": token, "accept": accept, "margin_r": margin_r,
            "margin_u": margin_u, "gamma_star": gstar, "neighbours": cdf_neighbours(w, token)}


def spec_cactus_verify(verifier_bits, draft_bits, draft_tokens, r_accept, u_resample,
                       delta: float, temperature=1.0, exact_kl: bool = False):
    """Batched Cactus verification; same layout as :func:`spec_verify` plus gamma_star [B, m].

    ``exact_kl`` takes gamma* as the exact root of the KL constraint instead of
    its Taylor form."""
    if not (delta >= 0.0 and math.isfinite(delta)):
        raise ValueError("delta must be finite and >= 0")
    B, m1, V = np.shape(verifier_bits)
    m = m1 - 1
    out = {
        "accepted_len": np.zeros(B, dtype=np.int64),
        "out_token": np.zeros(B, dtype=np.int64),
        "accept_mask": np.zeros((B, m), dtype=bool),
        "margin_r": np.zeros((B, m)),
        "margin_u": np.zeros(B),
        "gamma_star": np.zeros((B, m)),
        "neighbours": np.zeros((B, 2), dtype=np.int64),
    }
    for b in range(B):
        pt = softmax_t(widen_bf16(verifier_bits[b]), temperature)
        pd = softmax_t(widen_bf16(draft_bits[b]), temperature)
        res = cactus_sequence(pt, pd, draft_tokens[b], r_accept[b], u_resample[b], delta, exact_kl)
        out["accepted_len"][b] = res["A"]
        out["out_token"][b] = res["token"]
        out["accept_mask"][b] = res["accept"]
        out["margin_r"][b] = res["margin_r"]
        out["margin_u"][b] = res["margin_u"]
        out["gamma_star"][b] = res["gamma_star"]
        out["neighbours"][b] = res["neighbours"]
    return out


# ---------------------------------------------------------------------------
# HedgeSpec full-information evaluation
# ---------------------------------------------------------------------------

def realised_ratio(pt_x: float, pd_x: float) -> float:
    """a = min(1, pd(x)/pt(x)) at a realised token x (reading R1).

    This is the probability that drafter i would have proposed-and-kept the
    realised token, divided by the target's probability of it.  A realised
    token always has pt(x) > 0; pt(x) == 0 is mapped to 1 if pd(x) > 0, else 0.
    """
    if pt_x > 0.0:
        return min(1.0, pd_x / pt_x)
    return 1.0 if pd_x > 0.0 else 0.0


def acceptance_length_estimate(gamma_k, a_k) -> float:
    """One-step counterfactual acceptance length (reading R1 of [NB] Key design 2).

    L = 1 + sum_{k=0}^{K-1} gamma_k * prod_{j<k} a_j.  a_k[K-1] is unused.
    """
    L = 1.0
    prod = 1.0
    for k in range(len(gamma_k)):
        L += float(gamma_k[k]) * prod
        prod *= float(a_k[k])
    return L


def spec_counterfactual_gamma(target_bits, drafts_bits, traj_tokens, temperature=1.0):
    """gamma[b, k, i] = sum_x min(pt_k, pd_{i,k})  ([NB] Key design 1) for all N drafters,
    the estimator est[b, i] (R1) and loss[b, i] = (K + 1) - est (R2).

    target_bits [B, >=K, V] (rows 0..K-1 used), drafts_bits [N, B, K, V],
    traj_tokens [B, K] realised tokens (columns 0..K-2 enter the estimator).
    """
    N, B, K, V = np.shape(drafts_bits)
    gamma = np.zeros((B, K, N))
    est = np.zeros((B, N))
    for b in range(B):
        pt = softmax_t(widen_bf16(target_bits[b][:K]), temperature)
        for i in range(N):
            pd = softmax_t(widen_bf16(drafts_bits[i][b]), temperature)
            a = np.ones(K)
            for k in range(K):
                gamma[b, k, i] = acceptance_mass(pt[k], pd[k])
                x = int(traj_tokens[b][k])
                if k < K - 1:
                    if not 0 <= x < V:
                        raise ValueError("trajectory token id out of range")
                    a[k] = realised_ratio(pt[k, x], pd[k, x])
            est[b, i] = acceptance_length_estimate(gamma[b, :, i], a)
    return {"gamma": gamma, "est_len": est, "loss": (K + 1.0) - est}


# ---------------------------------------------------------------------------
# HedgeSpec acceptance under a greedy draft tree
# ---------------------------------------------------------------------------

def tree_children(z_draft, topk: int) -> np.ndarray:
    """Children a drafter keeps at a tree node: its topk most likely tokens.

    [NB] Key design 1 (the draft-tree case, its Theorem 2) names the children
    that the drafter builds or prunes at the node; reading R24 takes them as the
    drafter's topk tokens by logit (its softmax keeps the order at any
    temperature), ties to the smaller token id.  Token ids, best first.
    """
    z = np.asarray(z_draft, dtype=np.float64)
    order = np.lexsort((np.arange(z.shape[0]), -z))   # logit descending, then id ascending
    return order[:min(int(topk), z.shape[0])]


def tree_gamma(pt, z_draft, topk: int) -> float:
    """Acceptance probability at a greedy draft-tree node ([NB] Key design 1, its
    Theorem 2 case): the target's total probability on the node's children."""
    pt = np.asarray(pt, dtype=np.float64)
    return float(np.sum(pt[tree_children(z_draft, topk)]))


def spec_tree_gamma(target_bits, drafts_bits, topk: int, temperature=1.0):
    """gamma[b, k, i] = tree_gamma(pt_{b,k}, drafter i's logits at (b, k), topk).

    target_bits [B, >=K, V], drafts_bits [N, B, K, V] (bf16 bits)."""
    N, B, K, V = np.shape(drafts_bits)
    gamma = np.zeros((B, K, N))
    for b in range(B):
        for k in range(K):
            pt = softmax_t(widen_bf16(target_bits[b, k]), temperature)
            for i in range(N):
                gamma[b, k, i] = tree_gamma(pt, widen_bf16(drafts_bits[i, b, k]), topk)
    return gamma


# ---------------------------------------------------------------------------
# NormalHedge [NH]
# ---------------------------------------------------------------------------

NH_BISECT_ITERS = 64


def normalhedge_scale(rplus) -> float:
    """The scale c > 0 solving (1/N) sum_i exp(rplus_i^2 / (2c)) = e  ([NH]).

    Bisection in float64 on [M^2 / (2 (1 + ln N)), M^2 / 2], M = max rplus:
    at the left end the largest term alone reaches N e, at the right end every
    term is at most e, and the left side is decreasing in c.
    """
    rplus = np.asarray(rplus, dtype=np.float64)
    N = rplus.shape[0]
    M = float(np.max(rplus))
    lo = M * M / (2.0 * (1.0 + math.log(N)))
    hi = M * M / 2.0
    for _ in range(NH_BISECT_ITERS):
        mid = 0.5 * (lo + hi)
        if np.mean(np.exp(rplus * rplus / (2.0 * mid))) > math.e:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def normalhedge_weights(R) -> np.ndarray:
    """w_i proportional to (R_i+ / c) exp(R_i+^2 / (2c)); uniform when no regret is positive."""
    R = np.asarray(R, dtype=np.float64)
    rplus = np.maximum(R, 0.0)
    if not np.any(rplus > 0.0):
        return np.full(R.shape[0], 1.0 / R.shape[0])
    c = normalhedge_scale(rplus)
    w = (rplus / c) * np.exp(rplus * rplus / (2.0 * c))
    return w / np.sum(w)


def normalhedge_step(R, w, loss):
    """One full-information round: learner loss lhat = sum w_i l_i; R_i += lhat - l_i."""
    R = np.asarray(R, dtype=np.float64)
    loss = np.asarray(loss, dtype=np.float64)
    lhat = float(np.sum(np.asarray(w, dtype=np.float64) * loss))
    R = R + (lhat - loss)
    return R, normalhedge_weights(R)


def normalhedge_select(w, v: float) -> int:
    """Draw the next drafter from the weights by inverse CDF with uniform v (reading R5)."""
    j, _ = inverse_cdf(w, v)
    return j


def hedge_update(cum_regret, weights, loss, has_loss, loss_scale, v_select=None):
    """Batched per-sequence NormalHedge (reading R7: one learner per sequence).

    cum_regret [B, N] float64, weights [B, N] float64 (state), loss [B, N],
    has_loss [B] bool or None (all), loss_scale multiplies the loss first
    (e.g. 1/K maps length losses in [0, K] onto [0, 1]).  Returns the new
    (cum_regret, weights, sel) with sel [B] or None.
    """
    R = np.array(cum_regret, dtype=np.float64, copy=True)
    W = np.array(weights, dtype=np.float64, copy=True)
    B = R.shape[0]
    for b in range(B):
        if has_loss is None or has_loss[b]:
            scaled = np.asarray(loss[b], dtype=np.float64) * float(np.float32(loss_scale))
            R[b], W[b] = normalhedge_step(R[b], W[b], scaled)
    sel = None
    if v_select is not None:
        sel = np.array([normalhedge_select(W[b], float(v_select[b])) for b in range(B)], dtype=np.int64)
    return R, W, sel


def hedge_delayed_rounds(losses, delays, v_select, loss_scale):
    """T rounds of per-sequence NormalHedge under delayed feedback ([NB] Key design 3).

    losses [T, B, N]: the loss vector each round produces (after its chunk is
    verified); delays [T, B] integers in [0, 2K] (reading R4: a seeded
    schedule standing in for the chunk-completion delay); v_select [T, B].

    The loss of round s becomes usable for the selection of round
    s + 1 + delays[s]; before each round's selection every usable, not yet
    applied loss is applied one at a time in order of (usable round, origin
    round) -- the feedback queue of the stochastic-setting reduction the note
    describes.  Round 0 selects from uniform weights.  Returns (sel [T, B],
    cum_regret [B, N], weights [B, N]).
    """
    losses = np.asarray(losses, dtype=np.float64)
    T, B, N = losses.shape
    R = np.zeros((B, N))
    W = np.full((B, N), 1.0 / N)
    sel = np.zeros((T, B), dtype=np.int64)
    scale = float(np.float32(loss_scale))
    for b in range(B):
        pending = []  # (usable round, origin round)
        for t in range(T):
            ready = sorted(p for p in pending if p[0] <= t)
            pending = [p for p in pending if p[0] > t]
            for _, s in ready:
                R[b], W[b] = normalhedge_step(R[b], W[b], losses[s, b] * scale)
            sel[t, b] = normalhedge_select(W[b], float(v_select[t][b]))
            pending.append((t + 1 + int(delays[t][b]), t))
    return sel, R, W


# ---------------------------------------------------------------------------
# Acceptance-probability objective with exponential-weights Hedge
# ---------------------------------------------------------------------------

def acceptance_prob_loss(gamma):
    """[NB] Key design 3's loss when the acceptance probability is optimised:
    f = 1 - gamma at every position (reading R25: a chunk's losses, its K
    positions, enter the learner together, as their sum).  gamma [B, K, N] ->
    loss [B, N] in [0, K]."""
    g = np.asarray(gamma, dtype=np.float64)
    return np.sum(1.0 - g, axis=1)


def hedge_exp_step(L, loss, eta: float):
    """One exponential-weights (Hedge) update, [NB] Key design 3's other learner:
    cumulative loss L += loss, weights proportional to exp(-eta L) (computed
    against min L, which leaves them unchanged).  Returns (L, w)."""
    L = np.asarray(L, dtype=np.float64) + np.asarray(loss, dtype=np.float64)
    u = np.exp(-float(eta) * (L - L.min()))
    return L, u / u.sum()


def hedge_exp_update(cum_loss, weights, loss, has_loss, loss_scale, eta, v_select=None):
    """Batched per-sequence Hedge, as hedge_update but with exponential weights
    (learning rate eta >= 0).  cum_loss [B, N] float64 and weights [B, N]
    float64 are the state.  Returns (cum_loss, weights, sel or None)."""
    L = np.array(cum_loss, dtype=np.float64, copy=True)
    W = np.array(weights, dtype=np.float64, copy=True)
    scale = float(np.float32(loss_scale))
    e = float(np.float32(eta))
    for b in range(L.shape[0]):
        if has_loss is None or has_loss[b]:
            L[b], W[b] = hedge_exp_step(L[b], np.asarray(loss[b], dtype=np.float64) * scale, e)
    sel = None
    if v_select is not None:
        sel = np.array([normalhedge_select(W[b], float(v_select[b])) for b in range(L.shape[0])], dtype=np.int64)
    return L, W, sel


def censored_delays(accepted_len, K: int):
    """Delays that censoring causes ([NB] Key design 3): round s's chunk is only
    fully scored once K more tokens have been verified after it.  Round r
    verifies accepted_len[r] + 1 tokens, so round s's loss waits d rounds, d the
    smallest with sum_{r = s+1 .. s+d} (accepted_len[r] + 1) >= K (reading R25;
    d <= K <= 2K, the note's bound).  Rounds whose window runs past the last
    never complete (delay -1).  accepted_len [T, B] -> delays [T, B]."""
    A = np.asarray(accepted_len, dtype=np.int64)
    T, B = A.shape
    d = np.full((T, B), -1, dtype=np.int64)
    for b in range(B):
        for s in range(T):
            got = 0
            for r in range(s + 1, T):
                got += int(A[r, b]) + 1
                if got >= K:
                    d[s, b] = r - s
                    break
    return d


def hedge_delayed_rounds_rule(losses, delays, v_select, loss_scale, eta=None):
    """hedge_delayed_rounds with the learner chosen: NormalHedge (eta None) or
    exponential-weights Hedge with learning rate eta.  A delay of -1 never
    arrives.  Returns (sel [T, B], state [B, N] (regret or cumulative loss),
    weights [B, N])."""
    losses = np.asarray(losses, dtype=np.float64)
    T, B, N = losses.shape
    S = np.zeros((B, N))
    W = np.full((B, N), 1.0 / N)
    sel = np.zeros((T, B), dtype=np.int64)
    scale = float(np.float32(loss_scale))
    e = None if eta is None else float(np.float32(eta))
    for b in range(B):
        pending = []
        for t in range(T):
            ready = sorted(p for p in pending if p[0] <= t)
            pending = [p for p in pending if p[0] > t]
            for _, s in ready:
                if e is None:
                    S[b], W[b] = normalhedge_step(S[b], W[b], losses[s, b] * scale)
                else:
                    S[b], W[b] = hedge_exp_step(S[b], losses[s, b] * scale, e)
            sel[t, b] = normalhedge_select(W[b], float(v_select[t][b]))
            if int(delays[t][b]) >= 0:
                pending.append((t + 1 + int(delays[t][b]), t))
    return sel, S, W


def hedge_censored_rounds(round_outcome, T: int, B: int, N: int, K: int, Q: int, loss_scale, v_select, eta=None):
    """T rounds of per-sequence learning with the delay that censoring causes, run online
    ([NB] Key design 3; reading R25): round s's loss is usable once K more tokens have
    been verified after round s, a round verifying its accepted length plus one token
    (none when the accepted length is negative: nothing was verified).

    round_outcome(t, sel) plays round t with drafters sel [B] and returns its
    (losses [B, N], accepted_len [B]).  Before each round's selection, the learner
    of sequence b first counts the previous round's tokens for every queued loss,
    applies (oldest round first) those that have reached K, then queues the previous
    round's loss; a loss still queued Q rounds after its round is dropped (it never
    arrives; only rounds that verified nothing can keep one waiting that long).  The
    learner is NormalHedge (eta None) or exponential-weights Hedge with rate eta.
    Returns (sel [T, B], state [B, N], weights [B, N], accepted_len [T, B],
    weights before each round's draw [T, B, N]).
    """
    S = np.zeros((B, N))
    W = np.full((B, N), 1.0 / N)
    W_before = np.zeros((T, B, N))
    sel = np.zeros((T, B), dtype=np.int64)
    acc = np.zeros((T, B), dtype=np.int64)
    scale = float(np.float32(loss_scale))
    e = None if eta is None else float(np.float32(eta))
    queued = [[] for _ in range(B)]   # per sequence: [origin round, tokens verified since]
    losses = {}
    for t in range(T):
        for b in range(B):
            if t > 0:
                a = int(acc[t - 1, b])
                for q in queued[b]:
                    q[1] += a + 1 if a >= 0 else 0
                ready = sorted(q[0] for q in queued[b] if q[1] >= K)
                for s in ready:
                    if e is None:
                        S[b], W[b] = normalhedge_step(S[b], W[b], losses[s][b] * scale)
                    else:
                        S[b], W[b] = hedge_exp_step(S[b], losses[s][b] * scale, e)
                queued[b] = [q for q in queued[b] if q[1] < K and q[0] > (t - 1) - Q]
                queued[b].append([t - 1, 0])
            W_before[t, b] = W[b]
            sel[t, b] = normalhedge_select(W[b], float(v_select[t][b]))
        loss_t, acc_t = round_outcome(t, sel[t].copy())
        losses[t] = np.asarray(loss_t, dtype=np.float64)
        acc[t] = np.asarray(acc_t, dtype=np.int64)
    return sel, S, W, acc, W_before
