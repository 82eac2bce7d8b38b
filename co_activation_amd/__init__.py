"""Co-activation-aware MoE token dispatch engine for MI355X (gfx950).

The compute lives in ``libmoe_coact.so`` (hand-written HIP kernels behind the
C ABI of ``include/moe_coact.h``); ``ops`` marshals torch tensors into it,
``pipeline`` strings the calls into steps (one layer, two layers with the
token shuffle, the expert side, the backward), runs batches through a ring
of steps with each batch's plan beside the previous batch's row traffic, and
captures a step as a HIP graph; ``placement`` keeps the moving averages and
re-plans the expert placement.
"""

from . import ops  # noqa: F401
from ._lib import is_built, lib, LIB_PATH, EXPORTS  # noqa: F401
