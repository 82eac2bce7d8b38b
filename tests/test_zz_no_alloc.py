"""The allocation-free plan entry point (moe_dispatch_plan_noalloc) against
the workspace entry point (moe_dispatch_plan) and the CPU oracle, on two
calls in a row, the second with a smaller, ragged input, so that the shared
device scratch holds the first call's per-tile counts when the second runs."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd import ops
from co_activation_amd.pipeline import LayerStep
from gpu_util import assert_equal, host, i32, say
from workloads import make

pytestmark = pytest.mark.gpu

FIELDS = ("send_counts", "send_offsets", "row_token", "row_weight", "token_rows", "slot_row",
          "counters")


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def _outputs(T, k, G, cap):
    return LayerStep._plan_buffers(T, k, G, cap, "cuda")


def _case(cfg, T, uneven):
    w = make(cfg, T=T, with_x=False)
    src = None
    if uneven:
        # ragged source shards: one empty, the rest of unequal length
        rng = np.random.default_rng(T)
        cuts = np.sort(rng.integers(0, T + 1, size=w.G - 2))
        src = np.concatenate([[0, 0], cuts, [T]]).astype(np.int32)
    return w, src


@pytest.mark.parametrize("first,second", [((3, 4992, False), (4, 777, True)),
                                          ((2, 4096, True), (1, 300, False))])
def test_noalloc_matches_workspace_plan(first, second):
    for cfg, T, uneven in (first, second):
        w, src = _case(cfg, T, uneven)
        say("noalloc plan", cfg, T, uneven)
        topk, gates = i32(w.topk), torch.from_numpy(w.gates).cuda()
        er = i32(w.expert_rank)
        src_t = i32(src) if src is not None else None
        cap = T * min(w.k, w.G)
        err_a, err_b = ops.new_error_word(), ops.new_error_word()
        ref = ops.dispatch_plan(topk, gates, er, w.G, w.ranks_per_node, src_t,
                                out=_outputs(T, w.k, w.G, cap), d_err=err_a)
        out = _outputs(T, w.k, w.G, cap)
        for t in out.values():
            t.fill_(-7)  # stale values must all be overwritten where defined
        got = ops.dispatch_plan_noalloc(topk, gates, er, w.G, w.ranks_per_node, src_t, out=out,
                                        d_err=err_b)
        torch.cuda.synchronize()
        assert int(err_a.item()) == 0 and int(err_b.item()) == 0
        N = int(host(ref.counters)[0])
        for f in FIELDS:
            a, b = host(getattr(ref, f)), host(getattr(got, f))
            if f in ("row_token", "row_weight"):
                a, b = a[:N], b[:N]
            if f == "row_weight":
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert_equal(b, a, f)
        want = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node, src)
        assert_equal(host(got.counters), want["counters"], "counters vs oracle")
        assert_equal(host(got.row_token)[:N], want["row_token"], "row_token vs oracle")
        assert_equal(host(got.token_rows), want["token_rows"], "token_rows vs oracle")
