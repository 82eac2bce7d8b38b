"""ctypes loader for libmoe_coact.so.

The library must have been built (``python -m co_activation_amd.build`` or
``__graft_entry__.build()``); there is no fallback: a missing library is an
error.  torch is imported first so that the HIP runtime torch ships is the one
the library binds to (both carry the soname libamdhip64.so.7).
"""

from __future__ import annotations

import ctypes
from ctypes import c_int, c_int64, c_size_t, c_void_p, POINTER
from pathlib import Path

import torch  # noqa: F401  (loads the HIP runtime before the library)

LIB_PATH = Path(__file__).resolve().parent / "libmoe_coact.so"

# Must match include/moe_coact.h.
MOE_OK = 0
STATUS = {
    0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE",
    -4: "MOE_ERR_ALIGN", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_HIP",
}
MOE_F32, MOE_BF16 = 0, 1
DERR_BITS = {
    1: "EXPERT_RANGE", 2: "EXPERT_DUP", 4: "RANK_RANGE", 8: "CAPACITY",
    16: "SRC_OFFSETS", 32: "ROW_RANGE", 64: "SYNC",
}
MAX_K, MAX_E, MAX_G = 8, 256, 64

EXPORTS = (
    "moe_status_string", "moe_coact_stats", "moe_coact_stats_workspace_size",
    "moe_dispatch_plan_workspace_size",
    "moe_dispatch_plan", "moe_permute", "moe_combine",
    "moe_shuffle_predict_workspace_size", "moe_shuffle_predict",
    "moe_expert_plan_workspace_size", "moe_expert_plan",
    "moe_permute_scaled", "moe_row_dot", "moe_ema_update", "moe_place_experts",
    "moe_shuffle_balanced_workspace_size", "moe_shuffle_balanced", "moe_gather",
    "moe_shuffle_dispatch", "moe_dispatch_plan_gathered", "moe_dispatch_plan_noalloc",
)
NOALLOC_SCRATCH_BYTES = 4 << 20  # MOE_NOALLOC_SCRATCH_BYTES

_lib = None


def _declare(lib: ctypes.CDLL) -> None:
    P = c_void_p
    lib.moe_status_string.argtypes = [c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_coact_stats.argtypes = [P, c_int64, c_int, c_int, P, c_int, c_int, P, P, P, P, P, P,
                                    c_size_t, P]
    lib.moe_coact_stats.restype = c_int
    lib.moe_coact_stats_workspace_size.argtypes = [c_int64, c_int, c_int, c_int, POINTER(c_size_t)]
    lib.moe_coact_stats_workspace_size.restype = c_int
    lib.moe_dispatch_plan_workspace_size.argtypes = [c_int64, c_int, POINTER(c_size_t)]
    lib.moe_dispatch_plan_workspace_size.restype = c_int
    lib.moe_dispatch_plan.argtypes = [P, P, c_int64, c_int, c_int, P, c_int, c_int, P, c_int64,
                                      P, P, P, P, P, P, P, P, P, c_size_t, P]
    lib.moe_dispatch_plan.restype = c_int
    lib.moe_dispatch_plan_gathered.argtypes = [P, P, P, c_int64, c_int, c_int, P, c_int, c_int, P,
                                               c_int64, P, P, P, P, P, P, P, P, P, P, P,
                                               c_size_t, P]
    lib.moe_dispatch_plan_gathered.restype = c_int
    lib.moe_dispatch_plan_noalloc.argtypes = [P, P, c_int64, c_int, c_int, P, c_int, c_int, P,
                                              c_int64, P, P, P, P, P, P, P, P, P]
    lib.moe_dispatch_plan_noalloc.restype = c_int
    lib.moe_permute.argtypes = [P, c_int64, c_int64, P, c_int, P, c_int64, P, P, P]
    lib.moe_permute.restype = c_int
    lib.moe_gather.argtypes = [P, c_int64, c_int64, P, c_int64, P, P, P, P]
    lib.moe_gather.restype = c_int
    lib.moe_shuffle_dispatch.argtypes = [P, c_int64, c_int64, P, P, c_int, P, P, c_int64, P, P]
    lib.moe_shuffle_dispatch.restype = c_int
    lib.moe_combine.argtypes = [P, c_int, c_int64, c_int64, P, c_int, P, c_int64, P, c_int, P, P,
                                P]
    lib.moe_combine.restype = c_int
    lib.moe_shuffle_predict_workspace_size.argtypes = [c_int64, c_int, c_int, POINTER(c_size_t)]
    lib.moe_shuffle_predict_workspace_size.restype = c_int
    lib.moe_shuffle_predict.argtypes = [P, c_int64, c_int, c_int, P, c_int, P, c_int, P, P, P, P,
                                        P, P, c_size_t, P]
    lib.moe_shuffle_predict.restype = c_int
    lib.moe_shuffle_balanced_workspace_size.argtypes = [c_int64, c_int, c_int, POINTER(c_size_t)]
    lib.moe_shuffle_balanced_workspace_size.restype = c_int
    lib.moe_shuffle_balanced.argtypes = [P, c_int64, c_int, c_int, P, c_int, P, c_int, P, P, P, P,
                                         P, P, c_size_t, P]
    lib.moe_shuffle_balanced.restype = c_int
    lib.moe_expert_plan_workspace_size.argtypes = [c_int64, c_int, POINTER(c_size_t)]
    lib.moe_expert_plan_workspace_size.restype = c_int
    lib.moe_expert_plan.argtypes = [P, P, c_int64, c_int, c_int, P, c_int, P, c_int64, P, P, P, P,
                                    P, P, P, P, P, P, c_size_t, P]
    lib.moe_expert_plan.restype = c_int
    lib.moe_permute_scaled.argtypes = [P, c_int, c_int64, c_int64, P, c_int, P, P, c_int, c_int64,
                                       P, P, P]
    lib.moe_permute_scaled.restype = c_int
    lib.moe_row_dot.argtypes = [P, c_int, c_int64, c_int64, P, c_int, c_int64, P, c_int, P, P, P,
                                P]
    lib.moe_row_dot.restype = c_int
    lib.moe_ema_update.argtypes = [P, P, c_int64, ctypes.c_float, P]
    lib.moe_ema_update.restype = c_int
    lib.moe_place_experts.argtypes = [P, P, c_int, c_int, ctypes.c_double, P]
    lib.moe_place_experts.restype = c_int


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m co_activation_amd.build` "
                "(the engine has no CPU fallback)")
        handle = ctypes.CDLL(str(LIB_PATH), mode=ctypes.RTLD_GLOBAL)
        _declare(handle)
        _lib = handle
    return _lib


def is_built() -> bool:
    return LIB_PATH.exists()


class MoeError(RuntimeError):
    """A call of the C ABI returned a nonzero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
