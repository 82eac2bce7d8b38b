"""The pipelined runner: batches with their own inputs go through a ring of
steps, each batch's routing-only phase on a second stream beside the row
traffic of the batch before.  Every batch's results must equal, bit for bit,
those of one step run alone (one stream) on that batch."""

import pytest
import torch

from co_activation_amd.pipeline import GraphPipeline, LayerStep, Pipeline, TwoLayerStep
from gpu_util import assert_equal, dev, host, i32, say
from workloads import expert_outputs, make

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def _inputs(two_layer, w, z):
    if two_layer:
        return {"topk1": i32(w.topk), "topk2": i32(w.topk2), "gates2": dev(w.gates2),
                "x": dev(w.x), "z": z}
    return {"topk": i32(w.topk), "gates": dev(w.gates), "x": dev(w.x), "z": z}


def _step(two_layer, inp, w0):
    """A step on its own copies of the inputs (the placement is batch 0's)."""
    c = {k: v.clone() for k, v in inp.items()}
    if two_layer:
        return TwoLayerStep(c["topk1"], c["topk2"], c["gates2"], i32(w0.expert_rank2), c["x"],
                            c["z"], w0.G, w0.ranks_per_node, E1=w0.E)
    return LayerStep(c["topk"], c["gates"], i32(w0.expert_rank), c["x"], c["z"], w0.G,
                     w0.ranks_per_node)


def _bits(t):
    """The tensor's bit patterns, so that equality is bitwise."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _outputs(st, two_layer):
    out = {"y": st.y, "send": st.send}
    out.update({"stats." + k: v for k, v in st.stats_out.items()})
    out.update({"plan." + k: v for k, v in st.plan_out.items()})
    if two_layer:
        out.update({"shuffle." + k: v for k, v in st.shuffle_out.items()})
        out.update({"x_s": st.x_s, "topk2_s": st.topk2_s, "gates2_s": st.gates2_s})
    return out


@pytest.mark.parametrize("two_layer,ring,beside", [(False, 2, None), (False, 3, "combine"),
                                                   (True, 2, None), (True, 3, "move")])
def test_pipelined_batches_match_single_steps(two_layer, ring, beside):
    n = 7
    cfg, T, H = (5, 8192, 1024) if two_layer else (3, 4096, 1024)
    say("pipeline", "two-layer" if two_layer else "one layer", f"ring={ring}", f"beside={beside}",
        f"T={T}", f"H={H}")
    ws = [make(cfg, T=T, H=H, seed=s) for s in range(n)]
    w0 = ws[0]
    k = w0.k
    cap = T * min(k, w0.G)
    batches = [_inputs(two_layer, w, dev(expert_outputs(cap, H, "bf16", seed=10 + s)))
               for s, w in enumerate(ws)]
    steps = [_step(two_layer, batches[0], w0) for _ in range(ring)]
    pipe = Pipeline(steps, beside=beside)
    # workload 3 (k = 6, a row per slot) runs its plan beside the whole move,
    # workload 5 (k = 2) beside the combine
    assert pipe.beside == (beside or ("combine" if two_layer else "move"))
    got = {}

    def run(first, count):
        def prepare(st, i):
            for name, v in batches[first + i].items():
                getattr(st, name).copy_(v)

        def collect(st, i):
            got[first + i] = {key: v.clone() for key, v in _outputs(st, two_layer).items()}

        pipe.run(count, prepare=prepare, collect=collect)

    # two calls, so that the second starts behind the first one's batches
    run(0, 4)
    run(4, n - 4)
    torch.cuda.synchronize()
    for st in steps:
        assert int(st.d_err.item()) == 0
    for b in range(n):
        ref = _step(two_layer, batches[b], w0).run(overlap=False)
        torch.cuda.synchronize()
        assert int(ref.d_err.item()) == 0
        N = int(host(ref.plan.counters)[0])
        for key, want in _outputs(ref, two_layer).items():
            a, e = host(got[b][key]), host(want)
            if key in ("send", "plan.row_token", "plan.row_weight"):
                a, e = a[:N], e[:N]
            assert_equal(a, e, f"batch {b}: {key}")


def test_pipeline_rejects_bad_rings():
    w = make(3, T=512, H=64)
    inp = _inputs(False, w, dev(expert_outputs(512 * min(w.k, w.G), 64, "bf16", seed=1)))
    a = _step(False, inp, w)
    with pytest.raises(ValueError):
        Pipeline([a])
    with pytest.raises(ValueError):
        Pipeline([a, a])
    with pytest.raises(ValueError):
        Pipeline([a, _step(False, inp, w)], beside="dispatch")


@pytest.mark.parametrize("cfg", [5, 3])
def test_pipeline_fullsize_matches_single_steps(cfg):
    """The benchmark's timed configuration at full size: batches through a
    two-step pipeline (the plan beside the combine for workload 5, beside
    the whole move for workload 3), two routings and four row sets
    alternating, each batch equal on the device, bit for bit, to one step
    run alone on it."""
    from workloads.gen import device_normal

    two_layer = cfg == 5
    n = 4
    ws = [make(cfg, seed=s, with_x=False) for s in range(2)]
    w0 = ws[0]
    T, H = w0.T, w0.H
    cap = T * min(w0.k, w0.G)
    say("pipeline fullsize", cfg, f"T={T}", f"H={H}", f"batches={n}")
    batches = []
    for b in range(n):
        w = ws[b % 2]
        x = device_normal(T, H, w0.dtype, seed=20 + b)
        z = device_normal(cap, H, w0.dtype, seed=30 + b)
        if two_layer:
            batches.append({"topk1": i32(w.topk), "topk2": i32(w.topk2), "gates2": dev(w.gates2),
                            "x": x, "z": z})
        else:
            batches.append({"topk": i32(w.topk), "gates": dev(w.gates), "x": x, "z": z})
    steps = [_step(two_layer, batches[0], w0) for _ in range(2)]
    pipe = Pipeline(steps)
    assert pipe.beside == ("combine" if two_layer else "move")
    got = {}

    def prepare(st, i):
        for name, v in batches[i].items():
            getattr(st, name).copy_(v)

    def collect(st, i):
        got[i] = {key: v.clone() for key, v in _outputs(st, two_layer).items()}

    pipe.run(n, prepare=prepare, collect=collect)
    torch.cuda.synchronize()
    for st in steps:
        assert int(st.d_err.item()) == 0
    del steps, pipe
    for b in range(n):
        ref = _step(two_layer, batches[b], w0).run(overlap=False)
        torch.cuda.synchronize()
        assert int(ref.d_err.item()) == 0
        N = int(ref.plan.counters[0].item())
        for key, want in _outputs(ref, two_layer).items():
            a = got[b][key]
            if key in ("send", "plan.row_token", "plan.row_weight"):
                a, want = a[:N], want[:N]
            assert torch.equal(_bits(a), _bits(want)), f"batch {b}: {key}"
        del ref, got[b]
        torch.cuda.empty_cache()


@pytest.mark.parametrize("two_layer", [False, True])
def test_graph_pipeline_replays_match_single_steps(two_layer):
    """Four batches of a two-step pipeline captured as one graph and replayed
    three times, with eager work, synchronisation and cleared outputs in
    between: after every replay each step's outputs equal those of one step
    run alone on its inputs, bit for bit."""
    cfg, T, H = (5, 8192, 1024) if two_layer else (3, 4096, 1024)
    say("graph pipeline", "two-layer" if two_layer else "one layer", f"T={T}", f"H={H}")
    ws = [make(cfg, T=T, H=H, seed=s) for s in range(2)]
    w0 = ws[0]
    cap = T * min(w0.k, w0.G)
    batches = [_inputs(two_layer, w, dev(expert_outputs(cap, H, "bf16", seed=10 + s)))
               for s, w in enumerate(ws)]
    steps = [_step(two_layer, batches[j], w0) for j in range(2)]
    gp = GraphPipeline(Pipeline(steps), 4)
    refs = []
    for j in range(2):
        ref = _step(two_layer, batches[j], w0).run(overlap=False)
        torch.cuda.synchronize()
        refs.append(ref)
    for rep in range(3):
        for st in steps:
            st.y.zero_()
            st.send.zero_()
        torch.cuda.synchronize()
        gp.replay()
        torch.cuda.synchronize()
        for j, (st, ref) in enumerate(zip(steps, refs)):
            assert int(st.d_err.item()) == 0
            N = int(ref.plan.counters[0].item())
            for key, want in _outputs(ref, two_layer).items():
                a = _outputs(st, two_layer)[key]
                if key in ("send", "plan.row_token", "plan.row_weight"):
                    a, want = a[:N], want[:N]
                assert torch.equal(_bits(a), _bits(want)), f"replay {rep}, step {j}: {key}"
