"""Per-sequence drafter learners whose delayed-feedback queue lives on the device.

HedgeSpec note, Key design 3: a round's loss is only known once its chunk has
been verified, and the stochastic-setting reduction the note adopts keeps a
feedback queue and applies each loss once it is available.  Both classes here
hold the learner state, the queue and the round counters as device tensors and
advance a round with one kernel launch; they do no queue arithmetic on the host.

* ``CensoredLearner`` -- the delay that censoring causes: round s's loss is
  usable once K more tokens have been verified after round s, counted on the
  device from the rounds' accepted lengths (``hedge_censored_update``).  The
  learner is NormalHedge or exponential-weights Hedge (``eta``).
* ``ScheduledLearner`` -- NormalHedge with a delay schedule given in advance
  (``hedge_queue_update``): round s's loss usable at round s + 1 + delays[s].

Each ``step`` call is one round: it takes the previous round's loss (and, for
the censored learner, its accepted lengths), applies whatever has become usable,
and draws this round's drafter into ``sel`` (and ``sel_hist[t]``).
"""

from __future__ import annotations

import torch

from . import binding


class _DeviceLearner:
    def __init__(self, B: int, N: int, T: int, Q: int, v_select, device):
        self.B, self.N, self.T, self.Q = B, N, T, Q
        self.v = v_select.to(torch.float32).contiguous()
        if tuple(self.v.shape) != (T, B):
            raise ValueError("v_select must be [T, B]")
        self.state = torch.zeros((B, N), dtype=torch.float64, device=device)
        self.weights = torch.full((B, N), 1.0 / N, dtype=torch.float64, device=device)
        self.queue_loss = torch.zeros((B, Q, N), dtype=torch.float64, device=device)
        self.round = torch.zeros(B, dtype=torch.int32, device=device)
        self.sel = torch.zeros(B, dtype=torch.int32, device=device)
        self.sel_hist = torch.zeros((T, B), dtype=torch.int32, device=device)

    def _reset_common(self) -> None:
        """Device fills (no memset nodes), so that a graph may record them."""
        self.state.zero_()
        self.weights.fill_(1.0 / self.N)
        self.queue_loss.zero_()
        self.round.zero_()
        self.sel.zero_()
        self.sel_hist.zero_()


class CensoredLearner(_DeviceLearner):
    """NormalHedge (eta None) or Hedge with rate eta, under the censoring delay."""

    def __init__(self, B: int, N: int, K: int, T: int, loss_scale: float, v_select, eta=None,
                 queue_slots=None, device="cuda"):
        Q = int(queue_slots) if queue_slots is not None else K + 1
        super().__init__(B, N, T, Q, v_select, device)
        self.K = K
        self.loss_scale = float(loss_scale)
        self.learner = binding.LEARNER_NORMALHEDGE if eta is None else binding.LEARNER_HEDGE
        self.eta = 0.0 if eta is None else float(eta)
        self.queue_tokens = torch.full((B, Q), -1, dtype=torch.int32, device=device)

    def reset(self) -> None:
        self._reset_common()
        self.queue_tokens.fill_(-1)

    def step(self, loss, accepted_len, stream=None) -> torch.Tensor:
        """One round: loss [B, N] float32 and accepted_len [B] int32 of the previous round
        (read only from the second round on).  Returns sel [B] (this round's drafters)."""
        binding.hedge_censored_update(self.state, self.weights, self.queue_loss, self.queue_tokens, self.round,
                                      loss, accepted_len, self.K, self.learner, self.eta, self.loss_scale, self.v,
                                      self.sel, self.sel_hist, stream)
        return self.sel


class ScheduledLearner(_DeviceLearner):
    """NormalHedge with delays fixed in advance: delays [T, B] in [-1, Q-2] (-1: never)."""

    def __init__(self, B: int, N: int, K: int, T: int, loss_scale: float, v_select, delays,
                 queue_slots=None, device="cuda"):
        Q = int(queue_slots) if queue_slots is not None else 2 * K + 2
        super().__init__(B, N, T, Q, v_select, device)
        self.loss_scale = float(loss_scale)
        self.delays = delays.to(torch.int32).contiguous()
        if tuple(self.delays.shape) != (T, B):
            raise ValueError("delays must be [T, B]")
        self.queue_due = torch.full((B, Q), -1, dtype=torch.int32, device=device)

    def reset(self) -> None:
        self._reset_common()
        self.queue_due.fill_(-1)

    def step(self, loss, accepted_len=None, stream=None) -> torch.Tensor:
        """One round: loss [B, N] float32 of the previous round.  Returns sel [B]."""
        binding.hedge_queue_update(self.state, self.weights, self.queue_loss, self.queue_due, self.round, loss,
                                   self.delays, self.loss_scale, self.v, self.sel, self.sel_hist, stream)
        return self.sel
