"""Measured HBM ceilings: the streaming probes of libmoe_hbm_probe.so
(include/moe_hbm_probe.h) timed with HIP events.

``ceilings()`` returns the best sustained rate of each probe over its block
shapes -- read only, write only, copy, and for F = 1..8 the fan-out probe
(each vector read once and written to F dense regions) and the fan-in probe
(F regions read and folded into one) -- and ``mix_bound_us``
turns the read-only and write-only rates into the shortest time HBM allows a
kernel that reads R and writes W bytes, R / read + W / write (reads and
writes share the HBM interface, so they do not overlap to a shorter time).
``fanout_bound_us`` gives the time the dense fan-out probe takes for the same
R and W: the ideal of a permute with W / R destinations per row, each written
front to back, interpolated between the two nearest whole fan-outs;
``fanin_bound_us`` the same from the fan-in probe (F regions read and folded
into one written region) for a combine that reads R / W rows per output row.
``same_mix_bound_us`` picks whichever of the two applies to the mix."""

from __future__ import annotations

import ctypes
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
        h.moe_probe_fanout.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
        h.moe_probe_fanout.restype = ctypes.c_int
        h.moe_probe_fanin.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
        h.moe_probe_fanin.restype = ctypes.c_int
        _lib = h
    return _lib


FANOUTS = tuple(range(1, 9))
# Extra bytes between the fan-out probe's regions (293 x 512: not a power of
# two), so that one offset in every region does not map to one HBM channel.
STAGGER = 150016
WAVES = {0: 4, 1: 8, 2: 16, 3: 2}  # waves per block of each shape


def fanout_cap(shape: int, fan: int) -> int:
    """Blocks per CU that leave about 96 write streams (waves x places each
    vector goes) open per CU, the residency the wide-row permute measured
    best at; 0 (no cap) where that is 16 or more blocks, at least 2."""
    blocks = 96 // (WAVES[shape] * fan)
    return 0 if blocks >= 16 else max(2, blocks)


def fanin_cap(shape: int, fan: int) -> int:
    """Blocks per CU that leave about 24 waves resident per CU, the residency
    the many-row combine measured best at; no cap below three regions."""
    if fan < 3:
        return 0
    blocks = 24 // WAVES[shape]
    return 0 if blocks >= 16 else max(2, blocks)


def ceilings(bytes_=1 << 30, reps=5, device="cuda", mixes: bool = True) -> dict:
    """GB/s (decimal) per probe: the best shape's mean over ``reps`` launches
    back to back (read, write and copy; with ``mixes`` also fan-out and
    fan-in).  The
    fan-out probe's rate counts the bytes read and written (1 + F per byte of
    its 1 GiB source); it runs each shape uncapped and with the residency cap
    of ``fanout_cap``, with its regions exactly 1 GiB apart and ``STAGGER``
    bytes further apart, and the best of these is its ceiling.  The fan-in
    probe the same way (F source regions of 1 GiB, caps of ``fanin_cap``)."""
    lib = _load()
    src = torch.ones(bytes_, dtype=torch.uint8, device=device)
    dst = torch.empty(max(FANOUTS) * (bytes_ + STAGGER) if mixes else bytes_, dtype=torch.uint8,
                      device=device)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def run(mode, shape, nbytes):
        st = torch.cuda.current_stream().cuda_stream
        if mode >= 1100:  # fan-in probe: as the fan-out codes below, plus 1000
            fan, kind = mode % 100, (mode - 1000) // 100
            cap = fanin_cap(shape, fan) if kind in (2, 4) else 0
            stride = nbytes + (STAGGER if kind >= 3 else 0)
            rc = lib.moe_probe_fanin(shape, dst.data_ptr(), stride, src.data_ptr(), nbytes, fan,
                                     cap, st)
        elif mode >= 100:  # fan-out probe: F = mode % 100; capped: 2xx, 4xx; staggered: 3xx, 4xx
            fan = mode % 100
            cap = fanout_cap(shape, fan) if mode // 100 in (2, 4) else 0
            stride = nbytes + (STAGGER if mode >= 300 else 0)
            rc = lib.moe_probe_fanout(shape, src.data_ptr(), dst.data_ptr(), nbytes, stride, fan,
                                      cap, st)
        else:
            rc = lib.moe_probe_stream(mode, shape, src.data_ptr(), dst.data_ptr(), nbytes,
                                      sink.data_ptr(), st)
        if rc != 0:
            raise RuntimeError(f"HBM probe ({mode}, {shape}) returned {rc}")

    def timed(mode, shape, nbytes, moved):
        # one untimed launch, then ``reps`` launches back to back between one
        # event pair: an event pair around each launch alone would add the
        # launch latency to every sample (3-13% of these kernels' durations)
        run(mode, shape, nbytes)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run(mode, shape, nbytes)
        e1.record()
        torch.cuda.synchronize()
        return moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    by_shape = {}
    best = {}
    probes = [("read", 0, bytes_, bytes_), ("write", 1, bytes_, bytes_),
              ("copy", 2, bytes_, 2 * bytes_)]
    if mixes:
        probes += [(f"fanout{f}", 100 + f, bytes_, (1 + f) * bytes_) for f in FANOUTS]
        probes += [(f"fanin{f}", 1100 + f, bytes_, (1 + f) * bytes_) for f in FANOUTS]
    for name, mode, nbytes, moved in probes:
        rates = {SHAPES[sh]: timed(mode, sh, nbytes, moved) for sh in SHAPES}
        if mode >= 100:
            f = mode % 100
            capf = fanin_cap if mode >= 1100 else fanout_cap
            rates.update({f"{SHAPES[sh]}, at most {capf(sh, f)} per CU":
                          timed(mode + 100, sh, nbytes, moved)
                          for sh in SHAPES if capf(sh, f)})
            rates.update({f"{SHAPES[sh]}, staggered": timed(mode + 200, sh, nbytes, moved)
                          for sh in SHAPES})
            rates.update({f"{SHAPES[sh]}, at most {capf(sh, f)} per CU, staggered":
                          timed(mode + 300, sh, nbytes, moved)
                          for sh in SHAPES if capf(sh, f)})
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


def _probe_bound_us(small: float, large: float, g: dict, name: str) -> float | None:
    """Time of probe `name` (fanout or fanin) for a kernel that moves `small`
    bytes on its one-region side and `large` on its F-region side: its time
    per one-region byte at F = large / small, linear between the two nearest
    measured whole F; None outside 1 <= F <= 8."""
    if small <= 0:
        return None
    ratio = large / small
    if ratio < FANOUTS[0] or ratio > FANOUTS[-1] or f"{name}{FANOUTS[0]}" not in g:
        return None

    def per_byte(f):  # seconds per one-region byte at whole F
        return (1 + f) / (g[f"{name}{f}"] * 1e9)

    lo = min(int(ratio), FANOUTS[-1] - 1)
    t = per_byte(lo) + (ratio - lo) * (per_byte(lo + 1) - per_byte(lo))
    return small * t * 1e6


def fanout_bound_us(read_bytes: float, write_bytes: float, ceil: dict) -> float | None:
    """Time the dense fan-out probe needs for reading R and writing W bytes
    (microseconds): its time per byte read at F = W / R, linear between the
    two nearest measured whole fan-outs; None outside 1 <= W / R <= 8."""
    return _probe_bound_us(read_bytes, write_bytes, ceil["gbps"], "fanout")


def fanin_bound_us(read_bytes: float, write_bytes: float, ceil: dict) -> float | None:
    """Time the dense fan-in probe needs for reading R and writing W bytes
    (microseconds): its time per byte written at F = R / W, linear between
    the two nearest measured whole fan-ins; None outside 1 <= R / W <= 8."""
    return _probe_bound_us(write_bytes, read_bytes, ceil["gbps"], "fanin")


def same_mix_bound_us(read_bytes: float, write_bytes: float, ceil: dict) -> float | None:
    """The fan-out probe's time for a kernel that writes more than it reads,
    the fan-in probe's for one that reads more than it writes."""
    if write_bytes >= read_bytes:
        return fanout_bound_us(read_bytes, write_bytes, ceil)
    return fanin_bound_us(read_bytes, write_bytes, ceil)


if __name__ == "__main__":
    # python -m co_activation_amd.hbm_probe: this GPU's ceilings as one JSON line
    import json

    print(json.dumps(ceilings()))
