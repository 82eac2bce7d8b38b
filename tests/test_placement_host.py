"""The host placement planner behind the C ABI against the oracle (it runs on
the host, so these run without a GPU)."""

import numpy as np
import pytest

import oracle
from co_activation_amd import ops
from workloads import make


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    return built_lib


@pytest.mark.parametrize("cfg,eps", [(1, 0.1), (2, 0.25), (3, 0.1), (4, 0.05), (5, 0.0)])
def test_planner_matches_oracle_on_workloads(cfg, eps):
    w = make(cfg, T=2048 if cfg != 3 else 1024, with_x=False)
    st = oracle.coact_stats(w.topk, w.E)
    C = st["pair_count"].astype(np.float32)
    load = st["expert_count"].astype(np.float32)
    got = ops.place_experts(C, load, w.G, eps)
    want = oracle.place_experts(C, load, w.G, eps)
    assert (got == want).all()


def test_planner_matches_oracle_random():
    rng = np.random.default_rng(60)
    for trial in range(50):
        G = int(rng.integers(1, 9))
        E = G * int(rng.integers(1, 9))
        C = rng.integers(0, 4, size=(E, E)).astype(np.float32)   # many ties
        C = C + C.T
        load = rng.integers(0, 5, size=E).astype(np.float32)
        eps = float(rng.choice([0.0, 0.1, 1.0]))
        got = ops.place_experts(C, load, G, eps)
        want = oracle.place_experts(C, load, G, eps)
        assert (got == want).all(), (trial, got, want)


def test_planner_rejects():
    C = np.zeros((6, 6), np.float32)
    with pytest.raises(RuntimeError, match="MOE_ERR_SHAPE"):
        ops.place_experts(C, np.ones(6, np.float32), 4, 0.1)     # 6 % 4 != 0
    with pytest.raises(RuntimeError, match="MOE_ERR_SHAPE"):
        ops.place_experts(C, np.ones(6, np.float32), 3, -1.0)
