"""Seeded random shapes through every row-level entry point, against the CPU
oracle: routings of 1-8 experts out of 1-256, placements on 1-64 ranks with
any node size, uneven (sometimes empty) source shards, token counts from 0 up
to ten tiles with ragged ends, bf16 and fp32 rows of many widths; the next
layer planned over the shuffled order and dispatched in one pass.  Integer
results and moved rows are compared bit for bit, the combine to the usual
bound."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd import ops
from gpu_util import assert_equal, check_combine, dev, host, i32, say

pytestmark = pytest.mark.gpu

SEEDS = list(range(64))


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def _routing(rng, T, E, k):
    if T == 0:
        return np.zeros((0, k), np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([1, 2, 7, 16, 64, 100, 256]))
    k = int(rng.integers(1, min(8, E) + 1))
    G = int(rng.choice([1, 2, 3, 8, 13, 32, 64]))
    rn = int(rng.choice([d for d in range(1, G + 1) if G % d == 0]))
    T = int(rng.choice([0, 1, 255, 257, 700, 1500, 2561]))
    dt = str(rng.choice(["bf16", "f32"]))
    H = int(rng.choice([8, 64, 136, 512, 1024, 2112]))
    cuts = np.sort(rng.integers(0, T + 1, size=G - 1)) if G > 1 else np.zeros(0, np.int64)
    if rng.random() < 0.3 and G > 2:
        cuts[: G // 3] = 0            # some empty leading shards
    src = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    return rng, E, k, G, rn, T, dt, H, src


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shapes(seed):
    rng, E, k, G, rn, T, dt, H, src = _case(seed)
    say("random", seed, dict(E=E, k=k, G=G, rn=rn, T=T, dt=dt, H=H))
    topk = _routing(rng, T, E, k)
    gates = rng.random((T, k)).astype(np.float32)
    er = rng.integers(0, G, size=E).astype(np.int32)
    E2 = int(rng.choice([1, 9, 64, 256]))
    k2 = int(rng.integers(1, min(8, E2) + 1))
    topk2 = _routing(rng, T, E2, k2)
    er2 = rng.integers(0, G, size=E2).astype(np.int32)
    x32 = rng.standard_normal((T, H)).astype(np.float32)
    x = oracle.bf16_round(x32) if dt == "bf16" else x32
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    err = ops.new_error_word()

    # statistics with transitions
    st = ops.coact_stats(i32(topk), E, i32(topk2), E2, d_err=err)
    ref_st = oracle.coact_stats(topk, E, topk2, E2)
    for key in ("expert_count", "pair_count", "ochiai", "transition"):
        assert_equal(host(st[key]), ref_st[key], key)

    # plan on uneven shards, permute, combine
    cap = max(T * min(k, G), 1)
    plan = ops.dispatch_plan(i32(topk), dev(gates), i32(er), G, rn, src_offsets=i32(src),
                             row_capacity=cap, d_err=err)
    ref = oracle.dispatch_plan(topk, gates, er, G, rn, src_offsets=src)
    N = int(ref["N"])
    assert_equal(host(plan.counters), ref["counters"], "counters")
    assert_equal(host(plan.send_offsets), ref["send_offsets"], "send_offsets")
    assert_equal(host(plan.row_token)[:N], ref["row_token"], "row_token")
    assert_equal(host(plan.row_weight)[:N].view(np.uint32), ref["row_weight"].view(np.uint32),
                 "row_weight")
    assert_equal(host(plan.token_rows), ref["token_rows"], "token_rows")
    assert_equal(host(plan.slot_row), ref["slot_row"], "slot_row")
    xt = dev(x)
    send = ops.permute(xt, plan.token_rows, cap, d_err=err)
    torch.cuda.synchronize()
    assert_equal(host(send)[:N], oracle.permute_rows(x, ref["row_token"]), "send rows")
    z32 = rng.standard_normal((cap, H)).astype(np.float32)
    z = oracle.bf16_round(z32) if dt == "bf16" else z32
    y = ops.combine(dev(z), plan.token_rows, plan.row_weight, out_dtype=tdt, d_err=err)
    check_combine(y, z, dt, ref["slot_row"], gates, dt, "random combine")

    # gather by a random permutation
    perm = rng.permutation(T).astype(np.int32)
    if T:
        g = ops.gather(xt, i32(perm), d_err=err)
        torch.cuda.synchronize()
        assert_equal(host(g), oracle.permute_rows(x, perm), "gather")

    # destination side: layout and expansion
    ep = ops.expert_plan(i32(topk), dev(gates), i32(er), G, plan.slot_row, cap, d_err=err)
    ref_ep = oracle.expert_plan(topk, gates, er, G, ref["slot_row"], N)
    for key in ("erow", "expert_first", "expert_count", "rank_offsets", "erow_slot", "erow_src"):
        assert_equal(host(ep[key]), ref_ep[key], key)
    if T:
        ex = ops.gather(send, ep["erow_src"], d_err=err)
        torch.cuda.synchronize()
        assert_equal(host(ex), x[ref_ep["erow_slot"] // k], "expert rows")

    # shuffles (equal shards for the balanced one)
    sh = ops.shuffle_predict(i32(topk), st["transition"], i32(er2), G, d_err=err)
    ref_sh = oracle.shuffle_predict(topk, ref_st["transition"], er2, G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(sh[key]), ref_sh[key], "free " + key)
    # the next layer planned over the shuffled order (routing read through
    # perm), and the token rows moved and dispatched in one pass
    gates2 = rng.random((T, k2)).astype(np.float32)
    cap2 = max(T * min(k2, G), 1)
    t2_out = torch.empty((T, k2), dtype=torch.int32, device="cuda")
    g2_out = torch.empty((T, k2), dtype=torch.float32, device="cuda")
    plan2 = ops.dispatch_plan(i32(topk2), dev(gates2), i32(er2), G, rn,
                              src_offsets=sh["shard_offsets"], row_capacity=cap2, d_err=err,
                              perm=sh["perm"], topk_out=t2_out, gates_out=g2_out)
    ref2 = oracle.dispatch_plan_gathered(topk2, gates2, ref_sh["perm"], er2, G, rn,
                                         src_offsets=ref_sh["shard_offsets"])
    N2 = int(ref2["N"])
    assert_equal(host(t2_out), ref2["topk_out"], "gathered topk")
    assert_equal(host(g2_out).view(np.uint32), ref2["gates_out"].view(np.uint32), "gathered gates")
    assert_equal(host(plan2.counters), ref2["counters"], "gathered counters")
    assert_equal(host(plan2.row_token)[:N2], ref2["row_token"], "gathered row_token")
    assert_equal(host(plan2.row_weight)[:N2].view(np.uint32), ref2["row_weight"].view(np.uint32),
                 "gathered row_weight")
    assert_equal(host(plan2.token_rows), ref2["token_rows"], "gathered token_rows")
    if T:
        x_s, send2 = ops.shuffle_dispatch(xt, sh["perm"], plan2.token_rows, cap2, d_err=err)
        torch.cuda.synchronize()
        want_x, want_s = oracle.shuffle_dispatch(x, ref_sh["perm"], ref2["token_rows"], cap2)
        assert_equal(host(x_s), want_x, "shuffled rows")
        assert_equal(host(send2)[:N2], want_s[:N2], "shuffle-dispatched send rows")
    if T % G == 0:
        sb = ops.shuffle_predict(i32(topk), st["transition"], i32(er2), G, balanced=True,
                                 d_err=err)
        ref_sb = oracle.shuffle_balanced(topk, ref_st["transition"], er2, G)
        for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
            assert_equal(host(sb[key]), ref_sb[key], "balanced " + key)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))
