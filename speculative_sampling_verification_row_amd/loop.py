"""HedgeSpec rounds resident on the device, one captured graph per round.

HedgeSpec note, overall framework and Key designs 1-3: each round the learner
selects a drafter, that drafter's chunk is verified, every drafter is evaluated
on the verified trajectory (gamma, the length estimate and its loss), and the
loss joins the delayed-feedback queue of the learner.  Here a round is two
launches on one stream, with every pointer fixed in advance:

  learner step               queue the previous round's loss, count its
                             verified tokens, apply the losses that have become
                             usable, draw sel[b] for this round
  spec_counterfactual_gamma  fused: gamma / estimate / loss of all N drafters
                             and the verification of drafter sel[b], whose
                             accepted length the next learner step counts

so a round needs nothing from the host, and ``capture()`` records a round as a
graph that ``replay()`` runs again, round after round.  With the censoring
learner the two are one launch by default (``spec_hedgespec_round``: the first
draw unit of each sequence takes the learner step inside the gamma launch), so a
round is one graph node; ``fused=False`` keeps the two launches.  Nothing is allocated
after construction, and nothing in a round clears memory with a memset (the
library's workspace is left zero by every call).

The learner's delay is censoring by default (``CensoredLearner``: a round's loss
is usable once K more tokens are verified), or a schedule given in advance
(``delays``, ``ScheduledLearner``).

Rows.  ``rows`` is one set of round inputs (target, drafts, traj, draft_tokens,
r_accept, u_resample) or a list of such sets; round t reads set t % len(rows),
each with a graph of its own, so that consecutive rounds read different memory.
The launches read the caller's tensors themselves (an input that would have to
be copied to fit the library's layout is refused), so a caller streaming new
rows writes them into those tensors (``inputs[j]``) between rounds.
"""

from __future__ import annotations

import torch

from . import binding
from .hedge import CensoredLearner, ScheduledLearner


# a row set's keys -> the names of the fused launch's arguments
_ROW_KEYS = {"target": "target", "drafts": "drafts", "traj": "traj_tokens", "draft_tokens": "draft_tokens",
             "r_accept": "r_accept", "u_resample": "u_resample"}


class HedgeSpecLoop:
    def __init__(self, rows, v_select, loss_scale: float, temperature: float = 1.0, *, delays=None, eta=None,
                 queue_slots=None, fused: bool = True):
        sets = [rows] if isinstance(rows, dict) else list(rows)
        if not sets:
            raise ValueError("no rows")
        N, B, K, V = sets[0]["drafts"].shape
        T = int(v_select.shape[0])
        self.B, self.K, self.N, self.T = B, K, N, T
        dev = sets[0]["target"].device
        if delays is None:
            self.learner = CensoredLearner(B, N, K, T, loss_scale, v_select, eta=eta, queue_slots=queue_slots,
                                           device=dev)
        else:
            if eta is not None:
                raise ValueError("a delay schedule runs NormalHedge (hedge_queue_update)")
            self.learner = ScheduledLearner(B, N, K, T, loss_scale, v_select, delays, queue_slots=queue_slots,
                                            device=dev)
        self.ws = binding.make_workspace(B, K, N)
        self.fused = bool(fused) and delays is None
        self.calls = []
        out = None
        for rs in sets:
            if self.fused:
                call = binding.prepare_hedgespec_round(
                    rs["target"], rs["drafts"], rs["traj"], temperature, self.learner,
                    draft_tokens=rs["draft_tokens"], r_accept=rs["r_accept"], u_resample=rs["u_resample"],
                    workspace=self.ws, outputs=out, strict=True)
            else:
                call = binding.prepare_counterfactual_gamma(
                    rs["target"], rs["drafts"], rs["traj"], temperature, sel=self.learner.sel,
                    draft_tokens=rs["draft_tokens"], r_accept=rs["r_accept"], u_resample=rs["u_resample"],
                    workspace=self.ws, outputs=out, strict=True)
            out = call.outputs
            self.calls.append(call)
        self.out = out
        self.inputs = [{k: c.inputs[a] for k, a in _ROW_KEYS.items()} for c in self.calls]
        self.graphs = None
        self.t = 0

    @property
    def sel_hist(self):
        return self.learner.sel_hist

    def reset(self) -> None:
        """Learner, queue and round counters back to the start (device fills, no memset)."""
        self.learner.reset()
        self.t = 0

    def _round(self, j: int, stream=None) -> None:
        if not self.fused:
            self.learner.step(self.out["loss"], self.out["accepted_len"], stream)
        self.calls[j].launch(stream)

    def step(self, stream=None) -> None:
        """One round, launched eagerly."""
        self._round(self.t % len(self.calls), stream)
        self.t += 1

    def capture(self) -> None:
        """Record a round per row set as a graph (on a side stream, as torch requires)."""
        self.graphs = []
        for j in range(len(self.calls)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._round(j)
            self.graphs.append(g)

    def replay(self) -> None:
        """One round from its captured graph."""
        self.graphs[self.t % len(self.graphs)].replay()
        self.t += 1

    def check(self) -> None:
        """Synchronise and raise binding.WorkspaceFault if a round timed out in a wait
        between workgroups (its outputs, and the learner steps after it, are then
        unspecified)."""
        binding.check_workspace(self.ws, "HedgeSpecLoop")
