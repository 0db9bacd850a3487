"""Comparison rules between the HIP path and the float64 oracle.

Decisions, accepted lengths and tokens must be bit-exact, with these exclusions
(reported as counts, never dropped silently):
  * an accept bit whose oracle margin |r - ratio| < 1e-6;
  * a sequence's accepted length and token when such a near-tie sits at a
    position <= the oracle's accepted length;
  * a token whose oracle inverse-CDF margin < 1e-6 may differ from the oracle's,
    but must still be a token the oracle gives positive mass.
Acceptance masses, estimators and losses: within 1e-5 relative (fp32 outputs).
"""

from __future__ import annotations

import numpy as np

TIE = 1e-6
REL = 1e-5


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
    """ref: oracle dict (accepted_len, out_token, accept_mask, margin_r, margin_u)."""
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
            assert ref["margin_u"][b] < TIE, (
                f"{label} out_token[{b}] gpu {int(tok[b])} oracle {int(ref['out_token'][b])} "
                f"margin_u {ref['margin_u'][b]:.3g}")
            n_tok_excl += 1
    return {"near_tie_positions": int(near_r.sum()), "excluded_sequences": n_seq_excl,
            "excluded_tokens": n_tok_excl}


def assert_rel(gpu, ref, rel=REL, label=""):
    gpu = to_np(gpu).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-30)
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert np.all((err <= rel) | (np.isnan(gpu) & np.isnan(ref))), f"{label} max rel err {worst:.3g}"
    return worst
