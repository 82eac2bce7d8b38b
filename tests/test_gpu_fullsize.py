"""Parity at the full workload sizes, through the same step objects the
benchmark times.  Statistics, shuffle and plans are compared in full (bit for
bit); send rows and combined tokens on seeded samples that the oracle computes
one by one."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd.pipeline import LayerStep, TwoLayerStep
from gpu_util import assert_equal, check_combine, dev, host, i32, say, x_tensor
from workloads import make
from workloads.gen import device_normal

pytestmark = pytest.mark.gpu

SAMPLES = 384


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def _check_plan_full(plan, ref):
    N = int(ref["N"])
    assert_equal(host(plan.counters), ref["counters"], "counters")
    assert_equal(host(plan.send_counts), ref["send_counts"], "send_counts")
    assert_equal(host(plan.send_offsets), ref["send_offsets"], "send_offsets")
    assert_equal(host(plan.row_token)[:N], ref["row_token"], "row_token")
    assert_equal(host(plan.row_weight)[:N].view(np.uint32), ref["row_weight"].view(np.uint32),
                 "row_weight")
    assert_equal(host(plan.token_rows), ref["token_rows"], "token_rows")
    assert_equal(host(plan.slot_row), ref["slot_row"], "slot_row")


def _check_samples(step, ref_plan, x_rows_of_token, gates, zdt, rng):
    """Sampled send rows and combined tokens."""
    N = int(ref_plan["N"])
    rows = np.sort(rng.choice(N, size=min(SAMPLES, N), replace=False))
    got = host(step.send[torch.from_numpy(rows).to("cuda")])
    want = x_rows_of_token(ref_plan["row_token"][rows])
    assert_equal(got, want, "sampled send rows")
    T = ref_plan["token_rows"].shape[0]
    toks = np.sort(rng.choice(T, size=min(SAMPLES, T), replace=False))
    slot = ref_plan["slot_row"][toks]
    uniq, inv = np.unique(slot, return_inverse=True)
    Zs = host(step.z[torch.from_numpy(uniq).to("cuda")])
    y_sample = step.y[torch.from_numpy(toks).to("cuda")]
    check_combine(y_sample, Zs, zdt, inv.reshape(slot.shape), gates[toks], zdt, "sampled combine")


@pytest.mark.parametrize("cfg,placement", [(1, "main"), (2, "main"), (2, "alt"), (3, "main"),
                                           (4, "main"), (4, "alt")])
def test_layer_fullsize(cfg, placement):
    w = make(cfg)
    er = w.expert_rank if placement == "main" else w.alt_expert_rank
    say("fullsize layer", cfg, placement, w.T, w.H)
    cap = w.T * min(w.k, w.G)
    z = device_normal(cap, w.H, w.dtype, seed=1)
    step = LayerStep(i32(w.topk), dev(w.gates), i32(er), x_tensor(w), z, w.G, w.ranks_per_node)
    step.run()
    torch.cuda.synchronize()
    assert int(step.d_err.item()) == 0
    st = oracle.coact_stats(w.topk, w.E)
    assert_equal(host(step.stats_out["expert_count"]), st["expert_count"], "expert_count")
    assert_equal(host(step.stats_out["pair_count"]), st["pair_count"], "pair_count")
    assert_equal(host(step.stats_out["ochiai"]), st["ochiai"], "ochiai")
    ref = oracle.dispatch_plan(w.topk, w.gates, er, w.G, w.ranks_per_node)
    _check_plan_full(step.plan, ref)
    _check_samples(step, ref, lambda t: w.x[t], w.gates, w.dtype, np.random.default_rng(cfg))


@pytest.mark.parametrize("balanced", [False, True])
def test_two_layer_fullsize(balanced):
    w = make(5)
    say("fullsize two-layer", w.T, w.H, "balanced" if balanced else "free")
    cap = w.T * min(w.k, w.G)
    z = device_normal(cap, w.H, w.dtype, seed=1)
    step = TwoLayerStep(i32(w.topk), i32(w.topk2), dev(w.gates2), i32(w.expert_rank2),
                        x_tensor(w), z, w.G, w.ranks_per_node, E1=w.E, balanced=balanced)
    step.run()
    torch.cuda.synchronize()
    assert int(step.d_err.item()) == 0
    st = oracle.coact_stats(w.topk, w.E, w.topk2, w.E)
    for key in ("expert_count", "pair_count", "ochiai", "transition"):
        assert_equal(host(step.stats_out[key]), st[key], key)
    sh = (oracle.shuffle_balanced if balanced else oracle.shuffle_predict)(
        w.topk, st["transition"], w.expert_rank2, w.G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(step.shuffle[key]), sh[key], key)
    perm = sh["perm"]
    rng = np.random.default_rng(5)
    q = rng.choice(w.T, size=SAMPLES, replace=False)
    assert_equal(host(step.x_s[torch.from_numpy(q).to("cuda")]), w.x[perm[q]], "x shuffled")
    assert_equal(host(step.topk2_s), w.topk2[perm], "topk2 shuffled")
    assert_equal(host(step.gates2_s), w.gates2[perm], "gates2 shuffled")
    ref = oracle.dispatch_plan(w.topk2[perm], w.gates2[perm], w.expert_rank2, w.G,
                               w.ranks_per_node, src_offsets=sh["shard_offsets"])
    _check_plan_full(step.plan, ref)
    _check_samples(step, ref, lambda t: w.x[perm[t]], w.gates2[perm], w.dtype, rng)
    before = oracle.dispatch_plan(w.topk2, None, w.expert_rank2, w.G, w.ranks_per_node)
    share_before = before["counters"][3] / (w.T * w.k)
    share_after = ref["counters"][3] / (w.T * w.k)
    say("local share before/after shuffle", share_before, share_after)
    assert share_after > share_before
