"""The pipelined runner's ordering, checked on the CPU: the HIP event calls
and torch's streams are replaced by a recorder, the happens-before relation
of the enqueued work is rebuilt from stream order and event waits, and every
dependency a batch has is checked to be enforced, while the plan of one batch
is left free to run beside the row traffic of the one before."""

import contextlib
import itertools

import pytest
import torch

from co_activation_amd import pipeline as pl


class _Rec:
    """Streams, events and the work enqueued on them."""

    def __init__(self):
        self.ids = itertools.count(1)
        self.current = next(self.ids)  # the caller's stream
        self.frontier = {}             # stream -> ops that precede its next op
        self.last = {}                 # stream -> its last op
        self.events = {}               # event handle -> ops captured by its last record
        self.hb = {}                   # op -> ops that happen before it
        self.ops = []

    # torch.cuda stand-ins
    def new_stream(self, device=None):
        return type("S", (), {"cuda_stream": next(self.ids)})()

    def current_stream(self):
        return type("S", (), {"cuda_stream": self.current})()

    def set_stream(self, s):
        self.current = s.cuda_stream

    @contextlib.contextmanager
    def stream(self, s):
        prev, self.current = self.current, s.cuda_stream
        try:
            yield
        finally:
            self.current = prev

    def enqueue(self, op):
        s = self.current
        before = set(self.frontier.get(s, set()))
        if s in self.last:
            before |= self.hb[self.last[s]] | {self.last[s]}
        self.hb[op] = before
        self.frontier[s] = before | {op}
        self.last[s] = op
        self.ops.append((s, op))

    # HIP stand-ins (handles are ctypes pointers; keyed by address)
    def hipEventCreateWithFlags(self, pe, flags):
        pe._obj.value = next(self.ids)  # pe is ctypes.byref(c_void_p)
        return 0

    def hipEventRecord(self, ev, stream):
        s = stream.value
        ops = set(self.frontier.get(s, set()))
        if s in self.last:
            ops |= {self.last[s]}
        self.events[ev.value] = ops
        return 0

    def hipStreamWaitEvent(self, stream, ev, flags):
        s = stream.value
        self.frontier[s] = self.frontier.get(s, set()) | self.events.get(ev.value, set())
        return 0

    def hipEventDestroy(self, ev):
        return 0


class _FakeStep:
    DISPATCH_LAST = "dispatch"

    def __init__(self, rec, name, beside):
        self.rec, self.name, self.plan_beside = rec, name, beside
        self.d_err = torch.zeros(1, dtype=torch.int32)
        self.batch = None

    def plan_phase(self, timers=None):
        self.rec.enqueue(("plan", self.batch, self.name))

    def dispatch_phase(self, timers=None):
        with pl._timed(timers, "dispatch"):
            self.rec.enqueue(("dispatch", self.batch, self.name))

    def combine_phase(self, timers=None):
        self.rec.enqueue(("combine", self.batch, self.name))


@pytest.fixture
def rec(monkeypatch):
    r = _Rec()
    monkeypatch.setattr(pl._Hip, "get", classmethod(lambda cls: r))
    monkeypatch.setattr(pl.torch.cuda, "Stream", r.new_stream)
    monkeypatch.setattr(pl.torch.cuda, "current_stream", r.current_stream)
    monkeypatch.setattr(pl.torch.cuda, "stream", r.stream)
    monkeypatch.setattr(pl.torch.cuda, "set_stream", r.set_stream)
    return r


def _run(rec, m, beside, calls, timed=False):
    steps = [_FakeStep(rec, f"s{j}", beside) for j in range(m)]
    pipe = pl.Pipeline(steps)
    timers = pl.StageTimers(("dispatch",), sum(calls)) if timed else None
    assert pipe.beside == beside
    rec.enqueue(("inputs", -1, "caller"))
    batch = 0
    for n in calls:
        first = batch

        def prepare(st, i, first=first):
            st.batch = first + i
            rec.enqueue(("prepare", first + i, st.name))

        def collect(st, i, first=first):
            rec.enqueue(("collect", first + i, st.name))

        pipe.run(n, timers, prepare=prepare, collect=collect)
        batch += n
    rec.enqueue(("after", -1, "caller"))
    return steps, batch, pipe


def _op(rec, kind, b):
    return next(op for _, op in rec.ops if op[0] == kind and op[1] == b)


@pytest.mark.parametrize("beside", ["combine", "move"])
@pytest.mark.parametrize("m", [2, 3])
@pytest.mark.parametrize("calls", [(7,), (3, 4), (1, 1, 5)])
@pytest.mark.parametrize("timed", [False, True])
def test_pipeline_orders_every_dependency(rec, beside, m, calls, timed):
    """With the dispatch timed, the side stream waits on the timer's end
    event instead of a record of the pipeline's own: same ordering."""
    steps, n, pipe = _run(rec, m, beside, calls, timed)
    if timed:
        assert pipe._dispatched.value not in rec.events, "the timer's event was not used"
    hb = rec.hb
    inputs, after = _op(rec, "inputs", -1), _op(rec, "after", -1)
    for b in range(n):
        prep, plan = _op(rec, "prepare", b), _op(rec, "plan", b)
        disp, comb, coll = (_op(rec, k, b) for k in ("dispatch", "combine", "collect"))
        name = plan[2]
        assert inputs in hb[prep], "a batch starts before the caller's earlier work"
        assert prep in hb[plan] and plan in hb[disp] and disp in hb[comb] and comb in hb[coll]
        assert comb in hb[after] and plan in hb[after], "work left unordered with the caller's"
        for e in range(b):
            if _op(rec, "plan", e)[2] == name:
                # the step's earlier batch has left its buffers
                assert _op(rec, "collect", e) in hb[prep], (b, e)
    # the plan of a batch is not held behind the previous batch's combine
    # (the first batch of a call waits for everything before the call)
    firsts = {0} | set(itertools.accumulate(calls))
    for b in range(1, n):
        if b in firsts:
            continue
        assert _op(rec, "combine", b - 1) not in hb[_op(rec, "plan", b)], b
        if beside == "combine":
            assert _op(rec, "dispatch", b - 1) in hb[_op(rec, "plan", b)], b
        else:
            assert _op(rec, "dispatch", b - 1) not in hb[_op(rec, "plan", b)], b


def test_pipeline_rejects_bad_arguments(rec):
    a, b = _FakeStep(rec, "a", "combine"), _FakeStep(rec, "b", "combine")
    with pytest.raises(ValueError):
        pl.Pipeline([a])
    with pytest.raises(ValueError):
        pl.Pipeline([a, a])
    with pytest.raises(ValueError):
        pl.Pipeline([a, b], beside="dispatch")
    c = _FakeStep(rec, "c", "combine")
    c.d_err = torch.zeros(1, dtype=torch.int32, device="meta")
    with pytest.raises(ValueError):
        pl.Pipeline([a, c])


def test_pipeline_restores_the_current_stream_on_error(rec):
    """A plan phase that raises leaves the caller's stream current."""
    a, b = _FakeStep(rec, "a", "combine"), _FakeStep(rec, "b", "combine")

    def boom(timers=None):
        raise RuntimeError("plan failed")

    b.plan_phase = boom
    pipe = pl.Pipeline([a, b])
    caller = rec.current
    with pytest.raises(RuntimeError, match="plan failed"):
        pipe.run(3)
    assert rec.current == caller
