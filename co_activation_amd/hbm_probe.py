"""Measured HBM ceilings: the streaming probes of libmoe_hbm_probe.so
(include/moe_hbm_probe.h) timed with HIP events.

``ceilings()`` returns the best sustained rate of each probe over its block
shapes -- read only, write only, copy -- and ``mix_bound_us`` turns the
read-only and write-only rates into the shortest time HBM allows a kernel
that reads R and writes W bytes, R / read + W / write (reads and writes share
the HBM interface, so they do not overlap to a shorter time)."""

from __future__ import annotations

import ctypes
import statistics
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libmoe_hbm_probe.so"
SHAPES = {0: "256 threads, 4 KiB per block", 1: "512 threads, 8 KiB per block",
          2: "1024 threads, 16 KiB per block", 3: "128 threads, 2 KiB per block"}
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m co_activation_amd.build`")
        h = ctypes.CDLL(str(LIB_PATH))
        h.moe_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p]
        h.moe_probe_stream.restype = ctypes.c_int
        _lib = h
    return _lib


def ceilings(bytes_=1 << 30, reps=5, device="cuda") -> dict:
    """GB/s (decimal) per probe: the best shape's median over ``reps``."""
    lib = _load()
    src = torch.ones(bytes_, dtype=torch.uint8, device=device)
    dst = torch.empty(bytes_, dtype=torch.uint8, device=device)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def run(mode, shape, nbytes):
        st = torch.cuda.current_stream().cuda_stream
        rc = lib.moe_probe_stream(mode, shape, src.data_ptr(), dst.data_ptr(), nbytes,
                                  sink.data_ptr(), st)
        if rc != 0:
            raise RuntimeError(f"moe_probe_stream({mode}, {shape}) returned {rc}")

    def timed(mode, shape, nbytes, moved):
        run(mode, shape, nbytes)
        ts = []
        for _ in range(reps):
            e0.record()
            run(mode, shape, nbytes)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return moved / (statistics.median(ts) * 1e-3) / 1e9

    by_shape = {}
    best = {}
    probes = [("read", 0, bytes_, bytes_), ("write", 1, bytes_, bytes_),
              ("copy", 2, bytes_, 2 * bytes_)]
    for name, mode, nbytes, moved in probes:
        rates = {SHAPES[sh]: timed(mode, sh, nbytes, moved) for sh in SHAPES}
        by_shape[name] = {k: round(v, 1) for k, v in rates.items()}
        best[name] = max(rates.values())
    del src, dst, sink
    return {"gbps": {k: round(v, 1) for k, v in best.items()}, "by_shape": by_shape,
            "bytes_per_probe": bytes_, "reps": reps}


def mix_bound_us(read_bytes: float, write_bytes: float, ceil: dict) -> float:
    """Shortest time HBM allows for reading and writing these bytes, at the
    measured read-only and write-only rates (microseconds)."""
    g = ceil["gbps"]
    return (read_bytes / (g["read"] * 1e9) + write_bytes / (g["write"] * 1e9)) * 1e6
