"""Seeded synthetic MoE routing workloads (inputs only).

This package draws the inputs that both the HIP engine and the CPU oracle
consume: router top-k ids, gate weights, an expert->rank placement and the
token hidden rows.  It holds none of the dispatch method's arithmetic (no
statistics, plans, permutes or combines); see ``workloads.gen``.
"""

from .gen import Workload, make, expert_outputs, CONFIGS  # noqa: F401
