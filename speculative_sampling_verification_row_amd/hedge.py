"""Per-sequence NormalHedge or Hedge learners under delayed feedback.

HedgeSpec note, Key design 3: a round's loss is only known once its chunk has
been verified, so feedback reaches the learner late; the stochastic-setting
reduction the note adopts keeps a feedback queue and applies each loss as it
becomes available.  Here the loss of round s becomes usable for the selection
of round s + 1 + d_s (d_s in [0, 2K] per sequence, supplied by the caller);
before each selection, every usable loss is applied one at a time in order of
(usable round, origin round).

The learner is NormalHedge (``eta`` None) or exponential-weights Hedge with
learning rate ``eta`` (the note names both).  A delay of -1 never arrives: a
round whose chunk is never followed by K more verified tokens
(``censored_delays``).

This module is host-side bookkeeping only: it keeps the queue, builds the
per-step loss matrices and counts delays; every learner update and every
selection runs in the ``hedge_update`` / ``hedge_exp_update`` kernels on the
device, with the learner state resident there.
"""

from __future__ import annotations

import torch

from . import binding


def censored_delays(accepted_len, K: int):
    """Delays from censoring ([NB] Key design 3): round s's losses wait d rounds, d
    the smallest with sum_{r = s+1 .. s+d} (accepted_len[r] + 1) >= K (each round
    verifies its accepted drafts plus one token); -1 when the rounds run out.
    accepted_len [T][B] integers (host) -> list of T lists of B ints."""
    T = len(accepted_len)
    B = len(accepted_len[0]) if T else 0
    out = [[-1] * B for _ in range(T)]
    for b in range(B):
        for s in range(T):
            got = 0
            for r in range(s + 1, T):
                got += int(accepted_len[r][b]) + 1
                if got >= K:
                    out[s][b] = r - s
                    break
    return out


class DelayedHedge:
    def __init__(self, B: int, N: int, loss_scale: float, eta=None, device="cuda"):
        self.B, self.N = B, N
        self.loss_scale = float(loss_scale)
        self.eta = None if eta is None else float(eta)
        self.device = device
        # NormalHedge: cumulative regret; Hedge: cumulative loss
        self.cum_regret = torch.zeros((B, N), dtype=torch.float64, device=device)
        self.weights = torch.full((B, N), 1.0 / N, dtype=torch.float64, device=device)
        self._pending = [[] for _ in range(B)]   # per sequence: (usable round, origin round)
        self._loss = {}                          # origin round -> [B, N] float32 device tensor
        self._zero = torch.zeros((B, N), dtype=torch.float32, device=device)

    def push(self, origin_round: int, loss: torch.Tensor, delays) -> None:
        """Queue round `origin_round`'s loss [B, N]; delays[b] in [0, 2K], or -1 (never)."""
        self._loss[origin_round] = loss.to(torch.float32).contiguous()
        for b in range(self.B):
            if int(delays[b]) >= 0:
                self._pending[b].append((origin_round + 1 + int(delays[b]), origin_round))

    def select(self, round_: int, v: torch.Tensor) -> torch.Tensor:
        """Apply every loss usable at `round_`, then draw the next drafter per sequence."""
        ready = []
        for b in range(self.B):
            r = sorted(p for p in self._pending[b] if p[0] <= round_)
            self._pending[b] = [p for p in self._pending[b] if p[0] > round_]
            ready.append([s for _, s in r])
        steps = max((len(r) for r in ready), default=0)
        for step in range(steps):
            rows, mask = [], []
            for b in range(self.B):
                if step < len(ready[b]):
                    rows.append(self._loss[ready[b][step]][b])
                    mask.append(1)
                else:
                    rows.append(self._zero[b])
                    mask.append(0)
            loss = torch.stack(rows)
            has = torch.tensor(mask, dtype=torch.uint8).to(self.device, non_blocking=False)
            self._update(loss, has)
        still_needed = {s for b in range(self.B) for _, s in self._pending[b]}
        for s in list(self._loss):
            if s not in still_needed:
                del self._loss[s]
        no_loss = torch.zeros(self.B, dtype=torch.uint8, device=self.device)
        return self._update(self._zero, no_loss, v.to(torch.float32))

    def _update(self, loss, has, v=None):
        if self.eta is None:
            return binding.hedge_update(self.cum_regret, self.weights, loss, self.loss_scale, has_loss=has, v_select=v)
        return binding.hedge_exp_update(self.cum_regret, self.weights, loss, self.loss_scale, self.eta,
                                        has_loss=has, v_select=v)


# the NormalHedge learner under its earlier name
DelayedNormalHedge = DelayedHedge
