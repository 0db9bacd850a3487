"""HedgeSpec rounds resident on the device, one captured graph per round.

HedgeSpec note, overall framework and Key designs 1-3: each round the learner
selects a drafter, that drafter's chunk is verified, every drafter is evaluated
on the verified trajectory (gamma, the length estimate and its loss), and the
loss joins the delayed-feedback queue of the learner.  Here a round is two
launches on one stream, with every pointer fixed in advance:

  hedge_queue_update         queue round t-1's loss, apply the usable ones
                             (NormalHedge), draw sel[b] for round t
  spec_counterfactual_gamma  fused: gamma / estimate / loss of all N drafters
                             and the verification of drafter sel[b]

so a round needs nothing from the host, and ``capture()`` records one round as a
graph that ``replay()`` runs again, round after round.  Nothing is allocated
after construction, and nothing in a round clears memory with a memset (the
library's workspace is left zero by every call).

The per-round inputs of this loop (logits, drafted tokens, uniforms) are fixed
buffers: a caller that streams new rows writes them into those buffers between
rounds.  Only the schedules (delays [T][B], selection uniforms [T][B]) are
indexed by the round on the device.
"""

from __future__ import annotations

import torch

from . import binding


class HedgeSpecLoop:
    def __init__(self, target, drafts, traj, draft_tokens, r_accept, u_resample, delays, v_select,
                 loss_scale: float, temperature: float = 1.0, queue_slots: int | None = None):
        N, B, K, V = drafts.shape
        T = int(delays.shape[0])
        self.B, self.K, self.N, self.T = B, K, N, T
        dev = target.device
        self.Q = int(queue_slots) if queue_slots is not None else 2 * K + 2
        self.loss_scale = float(loss_scale)
        self.delays = delays.to(torch.int32).contiguous()
        self.v = v_select.to(torch.float32).contiguous()
        self.R = torch.zeros((B, N), dtype=torch.float64, device=dev)
        self.W = torch.full((B, N), 1.0 / N, dtype=torch.float64, device=dev)
        self.qloss = torch.zeros((B, self.Q, N), dtype=torch.float64, device=dev)
        self.qdue = torch.full((B, self.Q), -1, dtype=torch.int32, device=dev)
        self.round = torch.zeros(B, dtype=torch.int32, device=dev)
        self.sel = torch.zeros(B, dtype=torch.int32, device=dev)
        self.sel_hist = torch.zeros((T, B), dtype=torch.int32, device=dev)
        self.ws = binding.make_workspace(B, K, N)
        self.gamma_call = binding.prepare_counterfactual_gamma(
            target, drafts, traj, temperature, sel=self.sel, draft_tokens=draft_tokens, r_accept=r_accept,
            u_resample=u_resample, workspace=self.ws)
        self.out = self.gamma_call.outputs
        self._queue = binding.load().hedge_queue_update
        self._args = (binding._ptr(self.R), binding._ptr(self.W), binding._ptr(self.qloss), binding._ptr(self.qdue),
                      binding._ptr(self.round), binding._ptr(self.out["loss"]), binding._ptr(self.delays),
                      self.loss_scale, binding._ptr(self.v), binding._ptr(self.sel), binding._ptr(self.sel_hist),
                      B, N, self.Q, T)
        self.graph = None

    def reset(self) -> None:
        """Learner, queue and round counters back to the start (device fills, no memset)."""
        self.R.zero_()
        self.W.fill_(1.0 / self.N)
        self.qloss.zero_()
        self.qdue.fill_(-1)
        self.round.zero_()
        self.sel.zero_()
        self.sel_hist.zero_()

    def step(self, stream=None) -> None:
        """One round, launched eagerly."""
        st = self._queue(*self._args, binding._stream(stream))
        if st != binding.SPEC_OK:
            raise binding.SpecError("hedge_queue_update", st)
        self.gamma_call.launch(stream)

    def capture(self) -> None:
        """Record one round as a graph (on a side stream, as torch requires)."""
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.step()

    def replay(self) -> None:
        self.graph.replay()
