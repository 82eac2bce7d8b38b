"""Periodic co-activation placement from moving averages of the statistics.

Each observed step folds that step's pair counts and per-expert counts into
float32 moving averages on the device (``moe_ema_update``); every ``period``
steps the averages come to the host and ``moe_place_experts`` plans a new
expert -> rank placement ("Cobalt: Leveraging Expert Co-activation for
Efficient Distributed MoE Training", Stage 1: periodic re-planning from
moving averages, every 10 steps there; the decay is not given, so it is a
parameter here).
"""

from __future__ import annotations

import torch

from . import ops


class PlacementPlanner:
    def __init__(self, E: int, G: int, *, beta: float = 0.9, eps: float = 0.1, period: int = 10,
                 device="cuda"):
        self.E, self.G, self.beta, self.eps, self.period = E, G, beta, eps, period
        self.coact = torch.zeros(E * E, dtype=torch.float32, device=device)
        self.load = torch.zeros(E, dtype=torch.float32, device=device)
        self.steps = 0

    def observe(self, stats: dict):
        """Fold one step's ``pair_count`` [E,E] and ``expert_count`` [E]."""
        ops.ema_update(self.coact, stats["pair_count"].reshape(-1), self.beta)
        ops.ema_update(self.load, stats["expert_count"], self.beta)
        self.steps += 1

    def due(self) -> bool:
        return self.steps > 0 and self.steps % self.period == 0

    def plan(self):
        """A placement from the current averages (synchronises the stream)."""
        C = self.coact.reshape(self.E, self.E).cpu().numpy()
        w = self.load.cpu().numpy()
        return ops.place_experts(C, w, self.G, self.eps)
