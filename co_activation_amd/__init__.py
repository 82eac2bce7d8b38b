"""Co-activation-aware MoE token dispatch engine for MI355X (gfx950).

The compute lives in ``libmoe_coact.so`` (hand-written HIP kernels behind the
C ABI of ``include/moe_coact.h``); ``ops`` marshals torch tensors into it and
``pipeline`` strings the calls together for one two-layer step.
"""

from . import ops  # noqa: F401
from ._lib import is_built, lib, LIB_PATH, EXPORTS  # noqa: F401
