"""Comparison rules between the HIP path and the float64 oracle.

Decisions, accepted lengths and tokens must be bit-exact, with these exclusions
(counted, bounded and reported, never dropped silently):
  * an accept bit whose oracle margin |r - ratio| < 1e-6;
  * a sequence's accepted length and token when such a near-tie sits at a
    position <= the oracle's accepted length;
  * a token whose oracle inverse-CDF margin < 1e-6 may differ from the oracle's,
    but only by being the positive-mass token just before or just after it in
    the CDF (the neighbour whose step the threshold sits within rounding of).
The excluded sequences may be at most MAX_EXCLUDED_FRACTION of the batch (plus
one): a near tie at 1e-6 is rare, so many of them means a systematic error.
Acceptance masses and estimators: within 1e-5 relative (fp32 outputs).  Losses:
within 1e-5 relative or 1e-6 (K + 1) absolute, whichever is larger -- the loss is
(K + 1) - L, so its absolute error is the estimator's, a sum of K products of
acceptance masses each good to about 1e-7, which no relative bound holds where
the loss itself is 0 (a drafter equal to the target).
"""

from __future__ import annotations

import numpy as np

TIE = 1e-6
REL = 1e-5
MAX_EXCLUDED_FRACTION = 0.02


def to_np(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().numpy()
    except ImportError:
        pass
    return np.asarray(x)


def compare_verify(ref: dict, A, tok, mask, label: str = "") -> dict:
    """ref: oracle dict (accepted_len, out_token, accept_mask, margin_r, margin_u, neighbours)."""
    A, tok, mask = to_np(A), to_np(tok), to_np(mask)
    B, K = ref["accept_mask"].shape
    near_r = ref["margin_r"] < TIE
    if mask is not None:
        ok = (mask.astype(bool) == ref["accept_mask"]) | near_r
        bad = np.argwhere(~ok)
        assert bad.size == 0, f"{label} accept_mask mismatch at {bad[:10].tolist()}"
    n_seq_excl = 0
    n_tok_excl = 0
    for b in range(B):
        Ao = int(ref["accepted_len"][b])
        upto = min(Ao, K - 1)
        if near_r[b, : upto + 1].any():
            n_seq_excl += 1
            continue
        assert int(A[b]) == Ao, f"{label} accepted_len[{b}] gpu {int(A[b])} oracle {Ao}"
        if int(tok[b]) != int(ref["out_token"][b]):
            nb = tuple(int(v) for v in ref["neighbours"][b])
            assert ref["margin_u"][b] < TIE and int(tok[b]) in nb, (
                f"{label} out_token[{b}] gpu {int(tok[b])} oracle {int(ref['out_token'][b])} "
                f"margin_u {ref['margin_u'][b]:.3g} neighbours {nb}")
            n_tok_excl += 1
    limit = 1 + int(MAX_EXCLUDED_FRACTION * B)
    assert n_seq_excl + n_tok_excl <= limit, (
        f"{label} {n_seq_excl} sequences and {n_tok_excl} tokens excluded as near ties (limit {limit})")
    if n_seq_excl or n_tok_excl:
        print(f"{label}: near-tie exclusions: {n_seq_excl} sequences, {n_tok_excl} tokens")
    return {"near_tie_positions": int(near_r.sum()), "excluded_sequences": n_seq_excl,
            "excluded_tokens": n_tok_excl}


def assert_rel(gpu, ref, rel=REL, label=""):
    gpu = to_np(gpu).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-30)
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert np.all((err <= rel) | (np.isnan(gpu) & np.isnan(ref))), f"{label} max rel err {worst:.3g}"
    return worst


def assert_loss(gpu, ref, K, label=""):
    gpu = to_np(gpu).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = np.maximum(REL * np.abs(ref), 1e-6 * (K + 1.0))
    err = np.abs(gpu - ref)
    ok = (err <= tol) | (np.isnan(gpu) & np.isnan(ref))
    assert np.all(ok), f"{label} loss max err {float(np.nanmax(err)):.3g}"
    return float(np.nanmax(err / np.maximum(np.abs(ref), 1e-30))) if err.size else 0.0
