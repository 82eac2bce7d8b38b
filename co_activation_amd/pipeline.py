"""The dispatch path as sequences of C-ABI calls: steps, and a pipeline of
steps.

Single layer (workloads 1-4), ``LayerStep``:
    stats(topk) -> plan(topk, gates, placement) -> permute(x) -> combine(z)
Two layers with token shuffling (workload 5, "Expert Coupling in MoE
Pretraining ..." abstract: shuffle each token toward the rank forecast for
its next-layer experts), ``TwoLayerStep``:
    stats(topk1, topk2) -> shuffle_predict(topk1, transition, placement2)
    -> plan(topk2, gates2, placement2, src_offsets = shard_offsets) over the
       new order, reading the routing through perm and writing it out
       reordered (moe_dispatch_plan_gathered)
    -> x moved into the new order and dispatched into the layer-2 send rows
       in one pass (shuffle_dispatch; or a gather then a permute)
    -> combine(z)

Each step splits into ``plan_phase`` (everything that reads only the
routing), ``dispatch_phase`` and ``combine_phase`` (the row traffic).
``run`` runs one step; latency-bound stages that the bandwidth-bound chain
does not wait for run on a second stream beside it (the statistics of one
layer; the layer-2 plan and the pair statistics beside the token
move of the separate-pass two-layer step).  ``run(..., overlap=False)``
keeps everything on one stream, which is how per-stage times are taken.
``Pipeline`` runs a stream of independent batches over a ring of steps,
each batch's plan phase beside the previous batch's row traffic;
``GraphStep`` captures one step as a HIP graph.

All buffers are allocated once in the constructors; ``run`` only enqueues
kernels (no allocation, no host synchronisation).  ``z`` stands for the
expert side's returned rows (one per send row); ``ExpertSideStep`` and the
backward steps cover the destination side and the gradients.
"""

from __future__ import annotations

import contextlib
import ctypes
from typing import Optional

import torch

from . import ops


class _Hip:
    """The few HIP runtime event calls the timers need (same runtime torch
    loaded; recording through torch's Event wrapper costs far more host time
    than the runtime call itself)."""

    _h = None

    @classmethod
    def get(cls):
        if cls._h is None:
            h = None
            for name in ("libamdhip64.so.7", "libamdhip64.so"):
                try:
                    h = ctypes.CDLL(name)
                    break
                except OSError:
                    continue
            if h is None:
                raise RuntimeError("the HIP runtime library (libamdhip64) could not be loaded")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
            cls._h = h
        return cls._h


# hipEventCreateWithFlags flags.  Fork/join events only order two streams
# of one device, so a device-scope release is enough; timing events skip the
# system-scope fence, which otherwise adds a cache writeback to every record
# (a few microseconds of idle GPU per event after a kernel that wrote much).
_EVENT_DISABLE_TIMING = 0x2
_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_EVENT_RELEASE_TO_DEVICE = 0x40000000
_FORK_EVENT_FLAGS = _EVENT_DISABLE_TIMING | _EVENT_RELEASE_TO_DEVICE
_TIMER_EVENT_FLAGS = _EVENT_DISABLE_SYSTEM_FENCE


class _Fork:
    """A second stream (default priority) with fork and join events: work
    enqueued on it between ``fork`` and ``join`` runs beside the current
    stream's work and is complete before anything the current stream
    enqueues after ``join``."""

    def __init__(self, device):
        self.stream = torch.cuda.Stream(device=device)
        self._side = ctypes.c_void_p(self.stream.cuda_stream)
        h = _Hip.get()
        self._ev = [ctypes.c_void_p(), ctypes.c_void_p()]
        for e in self._ev:
            if h.hipEventCreateWithFlags(ctypes.byref(e), _FORK_EVENT_FLAGS):
                raise RuntimeError("hipEventCreateWithFlags failed")

    def fork(self):
        h = _Hip.get()
        cur = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if h.hipEventRecord(self._ev[0], cur) or h.hipStreamWaitEvent(self._side, self._ev[0], 0):
            raise RuntimeError("fork: hipEventRecord/hipStreamWaitEvent failed")
        return torch.cuda.stream(self.stream)

    def join(self):
        h = _Hip.get()
        cur = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if h.hipEventRecord(self._ev[1], self._side) or h.hipStreamWaitEvent(cur, self._ev[1], 0):
            raise RuntimeError("join: hipEventRecord/hipStreamWaitEvent failed")

    def __del__(self):
        try:
            h = _Hip.get()
            for e in self._ev:
                h.hipEventDestroy(e)
        except Exception:
            pass


class _Inline:
    """Stands in for a _Fork when everything stays on the current stream."""

    def fork(self):
        return _NULL_CTX

    def join(self):
        pass


_INLINE = _Inline()


class StageTimers:
    """HIP event pairs per stage, created up front so that a timed loop only
    records events on the stream the stage's kernels run on."""

    def __init__(self, names, steps, flags=None):
        if flags is None:
            flags = _TIMER_EVENT_FLAGS
        h = _Hip.get()
        self.pairs = {}
        for n in names:
            lst = []
            for _ in range(steps):
                a, b = ctypes.c_void_p(), ctypes.c_void_p()
                if h.hipEventCreateWithFlags(ctypes.byref(a), flags) or \
                        h.hipEventCreateWithFlags(ctypes.byref(b), flags):
                    raise RuntimeError("hipEventCreateWithFlags failed")
                lst.append((a, b))
            self.pairs[n] = lst
        self.used = {n: 0 for n in names}
        self.last_end = {}  # stage -> end event of its latest pair, until taken

    def begin(self, name):
        if name not in self.pairs:
            return None
        pair = self.pairs[name][self.used[name]]
        _Hip.get().hipEventRecord(pair[0], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        return pair

    def end(self, name, pair):
        if pair is None:
            return
        _Hip.get().hipEventRecord(pair[1], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        self.used[name] += 1
        self.last_end[name] = pair[1]

    def take_end(self, name):
        """The end event recorded by the latest ``end(name)`` not yet taken,
        or None: a caller that needs an event at that point of the stream
        can wait on it instead of recording another."""
        return self.last_end.pop(name, None)

    def durations_ms(self, name):
        """Per-launch durations of a stage (call after synchronising)."""
        h = _Hip.get()
        out = []
        for a, b in self.pairs[name][:self.used[name]]:
            f = ctypes.c_float()
            if h.hipEventElapsedTime(ctypes.byref(f), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(f.value)
        return out

    def mean_ms(self):
        return {n: sum(self.durations_ms(n)) / self.used[n] for n in self.pairs if self.used[n]}

    def median_ms(self):
        import statistics

        return {n: statistics.median(self.durations_ms(n)) for n in self.pairs if self.used[n]}

    def __del__(self):
        try:
            h = _Hip.get()
            for lst in self.pairs.values():
                for a, b in lst:
                    h.hipEventDestroy(a)
                    h.hipEventDestroy(b)
        except Exception:
            pass


class _Timed:
    """Records a stage's event pair around a block."""

    __slots__ = ("timers", "name", "pair")

    def __init__(self, timers, name):
        self.timers, self.name, self.pair = timers, name, None

    def __enter__(self):
        self.pair = self.timers.begin(self.name)

    def __exit__(self, *exc):
        self.timers.end(self.name, self.pair)


_NULL_CTX = contextlib.nullcontext()


def _timed(timers, name):
    """The stage's event pair around a block when timers are given (the
    untimed path builds nothing: it runs on every stage of every step)."""
    return _NULL_CTX if timers is None else _Timed(timers, name)


class LayerStep:
    """Stats + plan + permute + combine of one MoE layer."""

    def __init__(self, topk, gates, expert_rank, x, z, G, ranks_per_node, *,
                 out_dtype=None, src_offsets=None):
        dev = topk.device
        self.T, self.k = topk.shape
        self.E = expert_rank.numel()
        self.G, self.Rn = G, ranks_per_node
        self.topk, self.gates, self.expert_rank = topk, gates, expert_rank
        self.x, self.z = x, z
        self.src_offsets = src_offsets
        self.cap = self.T * min(self.k, G)
        self.out_dtype = out_dtype or x.dtype
        self.d_err = ops.new_error_word(dev)
        E = self.E
        self.stats_out = {
            "expert_count": torch.empty(E, dtype=torch.int32, device=dev),
            "pair_count": torch.empty(E, E, dtype=torch.int32, device=dev),
            "ochiai": torch.empty(E, E, dtype=torch.float32, device=dev),
        }
        self.stats_ws = torch.empty(ops.stats_workspace_bytes(self.T, E, True), dtype=torch.uint8,
                                    device=dev)
        self.plan_out = self._plan_buffers(self.T, self.k, G, self.cap, dev)
        self.plan_ws = torch.empty(ops.plan_workspace_bytes(self.T, G), dtype=torch.uint8, device=dev)
        self.send = torch.empty((self.cap,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
        self.y = torch.empty((self.T, x.shape[1]), dtype=self.out_dtype, device=dev)
        self._fork = _Fork(dev)
        # The step's four calls, checked once here and bound to its buffers:
        # each stage then replays its call with no per-call checks, which is
        # what paces small layers, whose kernels take a few microseconds.
        _, self._stats_call = ops.coact_stats(self.topk, E, out=self.stats_out, ws=self.stats_ws,
                                              d_err=self.d_err, bind=True)
        self.plan, self._plan_call = ops.dispatch_plan(
            self.topk, self.gates, self.expert_rank, G, self.Rn, self.src_offsets,
            out=self.plan_out, ws=self.plan_ws, d_err=self.d_err, bind=True)
        _, self._permute_call = ops.permute(self.x, self.plan.token_rows, self.cap, out=self.send,
                                            d_err=self.d_err, bind=True)
        _, self._combine_call = ops.combine(self.z, self.plan.token_rows, self.plan.row_weight,
                                            out_dtype=self.out_dtype, out=self.y,
                                            d_err=self.d_err, bind=True)

    @staticmethod
    def _plan_buffers(T, k, G, cap, dev):
        return {
            "send_counts": torch.empty(G, G, dtype=torch.int32, device=dev),
            "send_offsets": torch.empty(G * G + 1, dtype=torch.int32, device=dev),
            "row_token": torch.empty(cap, dtype=torch.int32, device=dev),
            "row_weight": torch.empty(cap, dtype=torch.float32, device=dev),
            "token_rows": torch.empty(T, k, dtype=torch.int32, device=dev),
            "slot_row": torch.empty(T, k, dtype=torch.int32, device=dev),
            "counters": torch.empty(8, dtype=torch.int64, device=dev),
        }

    STAGES = ("stats", "plan", "permute", "combine")
    DISPATCH_LAST = "permute"  # the last stage of dispatch_phase

    @property
    def plan_beside(self):
        """Where a Pipeline runs this step's plan phase: beside the combine,
        unless the combine reserves LDS to cap its residency (k >= 6 with a
        row per slot, as the expert side returns), which leaves no room on
        the CUs for the statistics histogram and the plan scan; then beside
        the whole move."""
        return "move" if self.k >= 6 and self.z.shape[0] >= 6 * self.T else "combine"

    def _stats(self, timers):
        with _timed(timers, "stats"):
            self._stats_call()

    def _plan(self, timers):
        with _timed(timers, "plan"):
            self._plan_call()

    def plan_phase(self, timers: Optional[StageTimers] = None):
        """Everything that reads only the routing: statistics and plan."""
        self._stats(timers)
        self._plan(timers)
        return self

    def dispatch_phase(self, timers: Optional[StageTimers] = None):
        """The send rows, which need the plan: the permute."""
        with _timed(timers, "permute"):
            self._permute_call()
        return self

    def combine_phase(self, timers: Optional[StageTimers] = None):
        """The returned rows back in token order: the combine."""
        with _timed(timers, "combine"):
            self._combine_call()
        return self

    def move_phase(self, timers: Optional[StageTimers] = None):
        """The row traffic, which needs the plan: permute and combine."""
        self.dispatch_phase(timers)
        return self.combine_phase(timers)

    def run(self, timers: Optional[StageTimers] = None, overlap: bool = True):
        fork = self._fork if overlap else _INLINE
        with fork.fork():
            self._stats(timers)
        self._plan(timers)
        self.move_phase(timers)
        fork.join()
        return self


class TwoLayerStep:
    """Layer-1 statistics with transitions, shuffle prediction, the shuffle,
    and the layer-2 deduplicated dispatch and combine.

    fused=True (the default): the move of the token rows into the shuffled
    order and the layer-2 permute are one pass (moe_shuffle_dispatch), which
    reads each row once; the layer-2 plan, which needs only the shuffled
    routing, runs before it.  fused=False: the move and the permute are
    separate passes, the plan overlapping the move on a second stream."""

    def __init__(self, topk1, topk2, gates2, expert_rank2, x, z, G, ranks_per_node, E1=None,
                 balanced=False, fused=True):
        dev = topk1.device
        self.balanced = balanced
        self.fused = fused
        self.T, self.k1 = topk1.shape
        self.k2 = topk2.shape[1]
        self.E1 = E1 if E1 is not None else expert_rank2.numel()
        self.E2 = expert_rank2.numel()
        self.G, self.Rn = G, ranks_per_node
        self.topk1, self.topk2, self.gates2, self.expert_rank2 = topk1, topk2, gates2, expert_rank2
        self.x, self.z = x, z
        self.d_err = ops.new_error_word(dev)
        E1, E2, T = self.E1, self.E2, self.T
        self.stats_out = {
            "expert_count": torch.empty(E1, dtype=torch.int32, device=dev),
            "pair_count": torch.empty(E1, E1, dtype=torch.int32, device=dev),
            "ochiai": torch.empty(E1, E1, dtype=torch.float32, device=dev),
            "transition": torch.empty(E1, E2, dtype=torch.int32, device=dev),
        }
        self.shuffle_out = {
            "pred_rank": torch.empty(T, dtype=torch.int32, device=dev),
            "dest_pos": torch.empty(T, dtype=torch.int32, device=dev),
            "perm": torch.empty(T, dtype=torch.int32, device=dev),
            "shard_offsets": torch.empty(G + 1, dtype=torch.int32, device=dev),
        }
        self.shuffle_ws = torch.empty(ops.shuffle_workspace_bytes(T, E1, G, balanced),
                                      dtype=torch.uint8, device=dev)
        # the statistics with transitions; without them (the pair counts on
        # the second stream of the separate-pass step) in a workspace of their own
        self.stats_ws = torch.empty(ops.stats_workspace_bytes(T, E1, True, E2), dtype=torch.uint8,
                                    device=dev)
        self.stats_ws2 = torch.empty(ops.stats_workspace_bytes(T, E1, True), dtype=torch.uint8,
                                     device=dev)
        self.x_s = torch.empty_like(x)
        self.topk2_s = torch.empty_like(topk2)
        self.gates2_s = torch.empty_like(gates2)
        self.cap = T * min(self.k2, G)
        self.plan_out = LayerStep._plan_buffers(T, self.k2, G, self.cap, dev)
        self.plan_ws = torch.empty(ops.plan_workspace_bytes(T, G), dtype=torch.uint8, device=dev)
        self.send = torch.empty((self.cap,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
        self.y = torch.empty((T, x.shape[1]), dtype=x.dtype, device=dev)
        self._fork = _Fork(dev)
        self._counts_tmp = torch.empty(E1, dtype=torch.int32, device=dev)
        # The calls of the statistics, the prediction, the plan, the fused
        # dispatch and the combine, checked once and bound (see LayerStep).
        _, self._stats_call = ops.coact_stats(self.topk1, E1, self.topk2, E2, out=self.stats_out,
                                              ws=self.stats_ws, d_err=self.d_err, bind=True)
        self.shuffle, self._shuffle_call = ops.shuffle_predict(
            self.topk1, self.stats_out["transition"], self.expert_rank2, G, balanced=balanced,
            out=self.shuffle_out, ws=self.shuffle_ws, d_err=self.d_err, bind=True)
        perm = self.shuffle["perm"]
        self.plan, self._plan_call = ops.dispatch_plan(
            self.topk2, self.gates2, self.expert_rank2, G, self.Rn, self.shuffle["shard_offsets"],
            out=self.plan_out, ws=self.plan_ws, d_err=self.d_err, perm=perm,
            topk_out=self.topk2_s, gates_out=self.gates2_s, bind=True)
        _, self._dispatch_call = ops.shuffle_dispatch(
            self.x, perm, self.plan.token_rows, self.cap, x_out=self.x_s, send=self.send,
            d_err=self.d_err, bind=True)
        _, self._combine_call = ops.combine(self.z, self.plan.token_rows, self.plan.row_weight,
                                            out=self.y, d_err=self.d_err, bind=True)

    STAGES_FUSED = ("stats", "shuffle_predict", "plan", "shuffle_dispatch", "combine")
    STAGES_SPLIT = ("stats", "shuffle_predict", "shuffle_permute", "plan", "permute", "combine")

    @property
    def STAGES(self):
        return self.STAGES_FUSED if self.fused else self.STAGES_SPLIT

    @property
    def DISPATCH_LAST(self):
        """The last stage of dispatch_phase."""
        return "shuffle_dispatch" if self.fused else "permute"

    @property
    def plan_beside(self):
        """Where a Pipeline runs this step's plan phase (see LayerStep)."""
        return "move" if self.k2 >= 6 and self.z.shape[0] >= 6 * self.T else "combine"

    def run(self, timers: Optional[StageTimers] = None, overlap: bool = True):
        if self.fused:
            return self._run_fused(timers)
        fork = self._fork if overlap else _INLINE
        st = self.stats_out
        with _timed(timers, "stats"):
            if overlap:
                # The prediction needs only the transitions; the pair counts
                # and Ochiai are computed on the second stream below.
                ops.coact_stats(self.topk1, self.E1, self.topk2, self.E2, pairs=False,
                                out={"expert_count": self._counts_tmp,
                                     "transition": st["transition"]}, ws=self.stats_ws,
                                d_err=self.d_err)
            else:
                self._stats_call()
        with _timed(timers, "shuffle_predict"):
            self._shuffle_call()
        perm = self.shuffle["perm"]
        with fork.fork():
            with _timed(timers, "plan"):
                self._plan_call()
            if overlap:
                ops.coact_stats(self.topk1, self.E1, out={k: st[k] for k in
                                                          ("expert_count", "pair_count", "ochiai")},
                                ws=self.stats_ws2, d_err=self.d_err)
        with _timed(timers, "shuffle_permute"):
            ops.gather(self.x, perm, out=self.x_s, d_err=self.d_err)
        fork.join()
        with _timed(timers, "permute"):
            ops.permute(self.x_s, self.plan.token_rows, self.cap, out=self.send, d_err=self.d_err)
        with _timed(timers, "combine"):
            self._combine_call()
        return self

    def plan_phase(self, timers: Optional[StageTimers] = None):
        """Everything that reads only the routing: statistics, prediction,
        and the layer-2 plan over the shuffled order (reading the routing
        through the shuffle's permutation and leaving it in that order in
        topk2_s / gates2_s)."""
        with _timed(timers, "stats"):
            self._stats_call()
        with _timed(timers, "shuffle_predict"):
            self._shuffle_call()
        with _timed(timers, "plan"):
            self._plan_call()
        return self

    def dispatch_phase(self, timers: Optional[StageTimers] = None):
        """The token rows moved to their shuffled places and dispatched into
        the layer-2 send rows: one pass when fused, a gather and a permute
        otherwise."""
        perm = self.shuffle["perm"]
        if self.fused:
            with _timed(timers, "shuffle_dispatch"):
                self._dispatch_call()
        else:
            with _timed(timers, "shuffle_permute"):
                ops.gather(self.x, perm, out=self.x_s, d_err=self.d_err)
            with _timed(timers, "permute"):
                ops.permute(self.x_s, self.plan.token_rows, self.cap, out=self.send,
                            d_err=self.d_err)
        return self

    def combine_phase(self, timers: Optional[StageTimers] = None):
        """The returned rows back in (shuffled) token order: the combine."""
        with _timed(timers, "combine"):
            self._combine_call()
        return self

    def move_phase(self, timers: Optional[StageTimers] = None):
        """The row traffic, which needs the plan: dispatch, then combine."""
        self.dispatch_phase(timers)
        return self.combine_phase(timers)

    def _run_fused(self, timers):
        """One stream: statistics, prediction and the layer-2 plan, then the
        token rows moved and dispatched in one pass, then the combine."""
        self.plan_phase(timers)
        return self.move_phase(timers)


class ExpertSideStep:
    """Destination side of a dispatched layer: the per-expert layout, the
    expansion of received rows into expert rows, and, once the experts have
    produced their rows, the gate-weighted reply rows per (token, rank) and
    the unweighted combine of the replies back to token order.

    ``layer`` is a LayerStep (or TwoLayerStep) that has run; its plan's row
    count stays on the device (``send_offsets[G*G]``), so nothing here waits
    on the host.  The expert computation itself is not part of this path:
    ``run`` takes the expert outputs ``expert_out`` [T*k, H] as an input (a
    stand-in buffer in the benchmark, scaling experts in the tests)."""

    STAGES = ("expert_plan", "expand", "partial_combine", "reply_combine")

    def __init__(self, layer):
        self.layer = layer
        topk = layer.topk if hasattr(layer, "topk") else layer.topk2_s
        self.topk = topk
        self.gates = layer.gates if hasattr(layer, "gates") else layer.gates2_s
        self.expert_rank = layer.expert_rank if hasattr(layer, "expert_rank") else layer.expert_rank2
        dev = topk.device
        self.T, self.k = topk.shape
        self.E = self.expert_rank.numel()
        self.G = layer.G
        self.cap = layer.cap
        H = layer.send.shape[1]
        self.out = {
            "erow": torch.empty(self.T, self.k, dtype=torch.int32, device=dev),
            "expert_first": torch.empty(self.E, dtype=torch.int32, device=dev),
            "expert_count": torch.empty(self.E, dtype=torch.int32, device=dev),
            "rank_offsets": torch.empty(self.G + 1, dtype=torch.int32, device=dev),
            "erow_weight": torch.empty(self.T * self.k, dtype=torch.float32, device=dev),
            "erow_slot": torch.empty(self.T * self.k, dtype=torch.int32, device=dev),
            "erow_src": torch.empty(self.T * self.k, dtype=torch.int32, device=dev),
            "row_dest": torch.empty(self.cap, self.k, dtype=torch.int32, device=dev),
        }
        self.ws = torch.empty(ops.expert_workspace_bytes(self.T, self.E), dtype=torch.uint8,
                              device=dev)
        self.expert_in = torch.empty(self.T * self.k, H, dtype=layer.send.dtype, device=dev)
        self.reply = torch.empty(self.cap, H, dtype=layer.send.dtype, device=dev)
        self.y = torch.empty(self.T, H, dtype=layer.send.dtype, device=dev)
        self.d_err = layer.d_err
        self.plan = None

    def n_rows(self):
        """The dispatch plan's row count, as a device int32 element."""
        so = self.layer.plan.send_offsets
        return so[so.numel() - 1:]

    def dispatch(self, timers: Optional[StageTimers] = None):
        """Expert layout and expansion of the received rows."""
        lp = self.layer.plan
        with _timed(timers, "expert_plan"):
            self.plan = ops.expert_plan(self.topk, self.gates, self.expert_rank, self.G,
                                        lp.slot_row, self.cap, out=self.out, ws=self.ws,
                                        d_err=self.d_err)
        with _timed(timers, "expand"):
            ops.gather(self.layer.send, self.plan["erow_src"], out=self.expert_in,
                       d_err=self.d_err)
        return self

    def reply_and_combine(self, expert_out, timers: Optional[StageTimers] = None):
        """Reply rows from the expert outputs, then the token-order output."""
        with _timed(timers, "partial_combine"):
            ops.combine(expert_out, self.plan["row_dest"], self.plan["erow_weight"],
                        out=self.reply, n_valid=self.n_rows(), d_err=self.d_err)
        with _timed(timers, "reply_combine"):
            ops.combine(self.reply, self.layer.plan.token_rows, None, out=self.y, d_err=self.d_err)
        return self


class LayerBackward:
    """Backward mirror of a LayerStep's weighted combine and permute:
    dz = a(row) * dy scattered to the rows, dw_tj = <dy_t, z[slot_row(t,j)]>,
    and dx = the unweighted combine of the gradient of the send rows."""

    STAGES = ("grad_rows", "grad_gates", "grad_tokens")

    def __init__(self, layer):
        self.layer = layer
        dev = layer.send.device
        H = layer.send.shape[1]
        self.dz = torch.empty(layer.cap, H, dtype=layer.z.dtype, device=dev)
        self.dw = torch.empty(layer.T, layer.k, dtype=torch.float32, device=dev)
        self.dx = torch.empty(layer.T, H, dtype=layer.x.dtype, device=dev)

    def run(self, dy, dsend, timers: Optional[StageTimers] = None):
        p = self.layer.plan
        err = self.layer.d_err
        with _timed(timers, "grad_rows"):
            ops.permute_scaled(dy, p.token_rows, p.row_weight, self.layer.cap, out=self.dz,
                               d_err=err)
        with _timed(timers, "grad_gates"):
            ops.row_dot(dy, self.layer.z, p.slot_row, out=self.dw, d_err=err)
        with _timed(timers, "grad_tokens"):
            ops.combine(dsend, p.token_rows, None, out=self.dx, d_err=err)
        return self


class ExpertSideBackward:
    """Backward mirror of an ExpertSideStep: the reply combine's gradient is
    dy copied to every reply row of its token; each expert output row gets
    its gate times its reply row's gradient; the gate gradients are
    dw_tj = <dy_t, expert_out[erow(t,j)]>; the expert inputs' gradients are
    summed back into send rows and the send rows' back into tokens."""

    STAGES = ("grad_replies", "grad_expert_out", "grad_gates", "grad_send", "grad_tokens")

    def __init__(self, side):
        self.side = side
        dev = side.y.device
        H = side.y.shape[1]
        dt = side.y.dtype
        self.d_reply = torch.empty(side.cap, H, dtype=dt, device=dev)
        self.d_expert_out = torch.empty(side.T * side.k, H, dtype=dt, device=dev)
        self.dw = torch.empty(side.T, side.k, dtype=torch.float32, device=dev)
        self.d_send = torch.empty(side.cap, H, dtype=dt, device=dev)
        self.dx = torch.empty(side.T, H, dtype=dt, device=dev)

    def run(self, dy, expert_out, d_expert_in, timers: Optional[StageTimers] = None):
        s = self.side
        lp = s.layer.plan
        err = s.d_err
        n = s.n_rows()
        with _timed(timers, "grad_replies"):
            ops.permute(dy, lp.token_rows, s.cap, out=self.d_reply, d_err=err)
        with _timed(timers, "grad_expert_out"):
            ops.permute_scaled(self.d_reply, s.plan["row_dest"], s.plan["erow_weight"],
                               s.T * s.k, out=self.d_expert_out, n_valid=n, d_err=err)
        with _timed(timers, "grad_gates"):
            ops.row_dot(dy, expert_out, s.plan["erow"], out=self.dw, d_err=err)
        with _timed(timers, "grad_send"):
            ops.combine(d_expert_in, s.plan["row_dest"], None, out=self.d_send, n_valid=n,
                        d_err=err)
        with _timed(timers, "grad_tokens"):
            ops.combine(self.d_send, lp.token_rows, None, out=self.dx, d_err=err)
        return self


class GraphStep:
    """A step captured once as a HIP graph and replayed: the whole dispatch
    path of a step (both streams, every kernel) is enqueued by one launch,
    so the host does no per-kernel work.  ``step`` is a LayerStep or
    TwoLayerStep whose buffers the graph reads and writes in place; the
    captured kernels keep the launch shapes and pointers of capture time.
    Nothing in the path allocates, synchronises or clears memory with a
    runtime memset, so the capture is complete."""

    def __init__(self, step):
        self.step = step
        # one eager run on a side stream first (settles lazy initialisation)
        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            step.run()
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            step.run()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()
        return self.step


class Pipeline:
    """Independent batches through a ring of steps, the routing-only phase
    of one batch overlapped with the row traffic of the batch before.

    Each step (LayerStep or TwoLayerStep, at least two, on one device) owns
    its buffers; batch i runs on step i mod m.  Its ``plan_phase``
    (statistics, prediction, plan: short latency-bound kernels) runs on a
    second stream; its ``dispatch_phase`` and ``combine_phase`` (the
    bandwidth-bound kernels) run on the current stream once that plan is
    complete.  Where the plan phase runs depends on ``beside``:

    - "combine": it starts once batch i-1 has dispatched, so it runs beside
      batch i-1's combine and the dispatch, the heaviest kernel, never shares
      the GPU with it.  Needs a combine that leaves room on the CUs for the
      plan kernels.
    - "move": it starts once batch i-m, the last user of the step's buffers,
      has combined, so it runs beside batch i-1's dispatch (and combine).

    The default is the steps' ``plan_beside``.  Every batch runs its whole
    path and gets the results it would get alone.

    ``prepare(step, i)``, if given, is called with the second stream current
    just before batch i's plan phase is enqueued, after the step's previous
    batch has left its buffers: the place to write batch i's inputs into the
    step.  ``collect(step, i)`` is called with the current stream current just
    after batch i's combine: the place to read its outputs.  Work that the
    caller enqueued on the current stream before ``run`` is complete before
    any batch starts, and everything ``run`` enqueues is ordered before what
    the caller enqueues on the current stream afterwards."""

    def __init__(self, steps, beside: Optional[str] = None):
        if len(steps) < 2:
            raise ValueError("a pipeline needs at least two steps (one per batch in flight)")
        dev = steps[0].d_err.device
        if any(st.d_err.device != dev for st in steps):
            raise ValueError("all steps of a pipeline must be on one device")
        if len({id(st) for st in steps}) != len(steps):
            raise ValueError("each step may appear once in a pipeline")
        self.beside = beside if beside is not None else steps[0].plan_beside
        if self.beside not in ("combine", "move"):
            raise ValueError("beside must be 'combine' or 'move'")
        self.steps = list(steps)
        self.side = torch.cuda.Stream(device=dev)
        self._side = ctypes.c_void_p(self.side.cuda_stream)
        h = _Hip.get()
        self._start = ctypes.c_void_p()       # current stream at the start of run
        self._planned = ctypes.c_void_p()     # side stream after a plan phase
        self._dispatched = ctypes.c_void_p()  # current stream after a dispatch phase
        self._done = [ctypes.c_void_p() for _ in steps]  # after each step's combine
        for e in self._events():
            if h.hipEventCreateWithFlags(ctypes.byref(e), _FORK_EVENT_FLAGS):
                raise RuntimeError("hipEventCreateWithFlags failed")
        self._next = 0

    def _events(self):
        return [self._start, self._planned, self._dispatched] + self._done

    def run(self, batches: int, timers: Optional[StageTimers] = None, prepare=None,
            collect=None):
        """Runs ``batches`` batches; returns the step that ran the last one."""
        h = _Hip.get()
        main_stream = torch.cuda.current_stream()
        main = ctypes.c_void_p(main_stream.cuda_stream)
        m = len(self.steps)
        # The first batches of a call wait for everything before the call.
        if h.hipEventRecord(self._start, main) or h.hipStreamWaitEvent(self._side, self._start, 0):
            raise RuntimeError("pipeline: hipEventRecord/hipStreamWaitEvent failed")
        by_combine = self.beside == "combine"
        last = None
        dispatched = None  # event after the previous batch's dispatch phase
        for i in range(batches):
            j = self._next % m
            st = self.steps[j]
            # the side stream current for the plan phase (set_stream, not
            # the stream context manager: a few microseconds of host time
            # less per batch, which is what paces small layers)
            torch.cuda.set_stream(self.side)
            try:
                if by_combine:
                    # batch i-1 has dispatched: every earlier batch, the last
                    # user of this step's buffers included, has combined
                    ev = dispatched
                else:
                    # batch i-m, the last user of this step's buffers
                    ev = self._done[j] if i >= m else None
                if ev is not None and h.hipStreamWaitEvent(self._side, ev, 0):
                    raise RuntimeError("pipeline: hipStreamWaitEvent failed")
                if prepare is not None:
                    prepare(st, i)
                st.plan_phase(timers)
            finally:
                torch.cuda.set_stream(main_stream)
            if h.hipEventRecord(self._planned, self._side) or \
                    h.hipStreamWaitEvent(main, self._planned, 0):
                raise RuntimeError("pipeline: hipEventRecord/hipStreamWaitEvent failed")
            st.dispatch_phase(timers)
            if by_combine:
                # a timer's end event at that point serves (one record fewer
                # on the current stream, about 3 us of idle GPU each)
                dispatched = timers.take_end(st.DISPATCH_LAST) if timers is not None else None
                if dispatched is None:
                    if h.hipEventRecord(self._dispatched, main):
                        raise RuntimeError("pipeline: hipEventRecord failed")
                    dispatched = self._dispatched
            st.combine_phase(timers)
            if collect is not None:
                collect(st, i)
            if not by_combine and h.hipEventRecord(self._done[j], main):
                raise RuntimeError("pipeline: hipEventRecord failed")
            self._next += 1
            last = st
        return last

    def __del__(self):
        try:
            h = _Hip.get()
            for e in self._events():
                h.hipEventDestroy(e)
        except Exception:
            pass


class GraphPipeline:
    """``batches`` batches of a ``Pipeline`` captured once as a HIP graph and
    replayed with one launch: the cross-stream order becomes graph edges and
    the host does no per-kernel work.  Inside one replay each batch's plan
    runs beside the previous batch's row traffic as in the eager pipeline;
    replays follow each other on the current stream, so only the first
    batch of a replay waits for the one before.  Worth it where the host
    paces the eager loop (small layers); a large layer, which the GPU paces,
    gains about 1%.  The steps' inputs are read in place at every replay
    (the graph keeps the pointers of capture time)."""

    def __init__(self, pipeline: "Pipeline", batches: int):
        if batches < 1:
            raise ValueError("a graph pipeline runs at least one batch per replay")
        self.pipeline, self.batches = pipeline, batches
        # one eager run on a side stream first (settles lazy initialisation)
        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            pipeline.run(batches)
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            pipeline.run(batches)
        torch.cuda.synchronize()

    def replay(self):
        """Runs the captured batches once more."""
        self.graph.replay()
