"""Per-sequence NormalHedge learners under delayed feedback.

HedgeSpec note, Key design 3: a round's loss is only known once its chunk has
been verified, so feedback reaches the learner late; the stochastic-setting
reduction the note adopts keeps a feedback queue and applies each loss as it
becomes available.  Here the loss of round s becomes usable for the selection
of round s + 1 + d_s (d_s in [0, 2K] per sequence, supplied by the caller);
before each selection, every usable loss is applied one at a time in order of
(usable round, origin round).

This class is host-side bookkeeping only: it keeps the queue and builds the
per-step loss matrices; every learner update and every selection runs in the
``hedge_update`` kernel on the device, with the learner state resident there.
"""

from __future__ import annotations

import torch

from . import binding


class DelayedNormalHedge:
    def __init__(self, B: int, N: int, loss_scale: float, device="cuda"):
        self.B, self.N = B, N
        self.loss_scale = float(loss_scale)
        self.device = device
        self.cum_regret = torch.zeros((B, N), dtype=torch.float64, device=device)
        self.weights = torch.full((B, N), 1.0 / N, dtype=torch.float64, device=device)
        self._pending = [[] for _ in range(B)]   # per sequence: (usable round, origin round)
        self._loss = {}                          # origin round -> [B, N] float32 device tensor
        self._zero = torch.zeros((B, N), dtype=torch.float32, device=device)

    def push(self, origin_round: int, loss: torch.Tensor, delays) -> None:
        """Queue round `origin_round`'s loss [B, N]; delays[b] in [0, 2K]."""
        self._loss[origin_round] = loss.to(torch.float32).contiguous()
        for b in range(self.B):
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
            binding.hedge_update(self.cum_regret, self.weights, loss, self.loss_scale, has_loss=has)
        still_needed = {s for b in range(self.B) for _, s in self._pending[b]}
        for s in list(self._loss):
            if s not in still_needed:
                del self._loss[s]
        no_loss = torch.zeros(self.B, dtype=torch.uint8, device=self.device)
        return binding.hedge_update(self.cum_regret, self.weights, self._zero, self.loss_scale,
                                    has_loss=no_loss, v_select=v.to(torch.float32))
