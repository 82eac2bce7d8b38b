"""EMA statistics on the device and the observe / re-plan loop, against the
oracle."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd import ops
from co_activation_amd.placement import PlacementPlanner
from gpu_util import assert_equal, host, i32, say
from workloads import make

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


@pytest.mark.parametrize("beta", [0.9, 0.5, 0.0, 1.0, 0.123])
def test_ema_bit_exact(beta):
    rng = np.random.default_rng(70)
    n = 70000
    state = (rng.standard_normal(n) * 1000).astype(np.float32)
    x = rng.integers(0, 1 << 20, size=n).astype(np.int32)
    say("ema", beta)
    s = torch.from_numpy(state.copy()).cuda()
    ops.ema_update(s, i32(x), beta)
    torch.cuda.synchronize()
    assert_equal(host(s).view(np.uint32), oracle.ema_update(state, x, beta).view(np.uint32), "ema")


def test_observe_and_replan_matches_oracle():
    """Three steps of statistics folded into the averages, then a plan: the
    same placement as the oracle's averages and planner, and fewer rows than
    the contiguous split on the next batch."""
    w = make(2, T=12288, with_x=False)
    say("planner loop")
    planner = PlacementPlanner(w.E, w.G, beta=0.8, eps=0.25, period=3)
    C = np.zeros(w.E * w.E, np.float32)
    L = np.zeros(w.E, np.float32)
    for s in range(3):
        sl = slice(s * 4096, (s + 1) * 4096)
        st = ops.coact_stats(i32(w.topk[sl]), w.E)
        planner.observe(st)
        ref = oracle.coact_stats(w.topk[sl], w.E)
        C = oracle.ema_update(C, ref["pair_count"].reshape(-1), 0.8)
        L = oracle.ema_update(L, ref["expert_count"], 0.8)
    assert planner.due()
    got = planner.plan()
    want = oracle.place_experts(C.reshape(w.E, w.E), L, w.G, 0.25)
    assert (got == want).all()
    assert_equal(host(planner.coact).view(np.uint32), C.view(np.uint32), "averaged pairs")
    n_new = oracle.dispatch_plan(w.topk, None, got, w.G, w.ranks_per_node)["N"]
    n_uni = oracle.dispatch_plan(w.topk, None, np.arange(w.E) // (w.E // w.G), w.G,
                                 w.ranks_per_node)["N"]
    assert n_new < n_uni
