"""Parity at the full workload sizes, through the same step objects the
benchmark times.  Statistics, shuffles, plans, every send row (bit for bit)
and every combined token (to the combine's bound) are compared in full, the
rows and tokens in chunks so that host memory stays bounded; the destination
side and the backward on a seeded sample of tokens."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd.pipeline import (ExpertSideBackward, ExpertSideStep, LayerStep,
                                        TwoLayerStep)
import gpu_util
from gpu_util import assert_equal, bf16_ulps, check_combine, dev, host, i32, say, x_tensor
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


ROW_CHUNK = 16384
TOKEN_CHUNK = 2048


def _check_rows_full(step, ref_plan, source_of_token):
    """Every send row: send[i] == x[source_of_token(row_token[i])] bit for bit
    (oracle.permute_rows on chunks of rows)."""
    N = int(ref_plan["N"])
    x = source_of_token(None)
    for a in range(0, N, ROW_CHUNK):
        b = min(N, a + ROW_CHUNK)
        want = oracle.permute_rows(x, source_of_token(ref_plan["row_token"][a:b]))
        assert_equal(host(step.send[a:b]), want, f"send rows {a}..{b}")


def _check_combine_full(step, ref_plan, gates, zdt):
    """Every combined token against oracle.combine, in chunks of tokens (the
    chunks' numpy checks on a few threads; the device reads stay on this
    one); the bf16 elements held to the fp32 bound are counted and
    bounded."""
    from concurrent.futures import ThreadPoolExecutor

    T = ref_plan["token_rows"].shape[0]
    start = len(gpu_util.FALLBACKS)
    with ThreadPoolExecutor(max_workers=8) as pool:
        futures = []
        for a in range(0, T, TOKEN_CHUNK):
            b = min(T, a + TOKEN_CHUNK)
            slot = ref_plan["slot_row"][a:b]
            uniq, inv = np.unique(slot, return_inverse=True)
            Zs = host(step.z[torch.from_numpy(uniq).to("cuda")])
            futures.append(pool.submit(gpu_util.check_combine_host, host(step.y[a:b]), Zs, zdt,
                                       inv.reshape(slot.shape), gates[a:b], zdt,
                                       f"combine tokens {a}..{b}"))
            if len(futures) >= 16:  # bound the chunks held at once
                futures.pop(0).result()
        for f in futures:
            f.result()
    fb = gpu_util.FALLBACKS[start:]
    n = sum(c for _, c, _ in fb)
    total = sum(e for _, _, e in fb)
    say("combine elements held to the fp32 bound (cancellation):", n, "of", total)
    assert n <= max(16, 1e-5 * total), f"{n} of {total} elements needed the fp32 bound"


@pytest.mark.parametrize("cfg,placement", [(1, "main"), (2, "main"), (2, "alt"), (3, "main"),
                                           (3, "alt"), (4, "main"), (4, "alt")])
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
    _check_rows_full(step, ref, lambda t: w.x if t is None else t)
    _check_combine_full(step, ref, w.gates, w.dtype)


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
    for a in range(0, w.T, ROW_CHUNK):  # every shuffled row
        b = min(w.T, a + ROW_CHUNK)
        assert_equal(host(step.x_s[a:b]), oracle.permute_rows(w.x, perm[a:b]), "x shuffled")
    assert_equal(host(step.topk2_s), w.topk2[perm], "topk2 shuffled")
    assert_equal(host(step.gates2_s), w.gates2[perm], "gates2 shuffled")
    ref = oracle.dispatch_plan(w.topk2[perm], w.gates2[perm], w.expert_rank2, w.G,
                               w.ranks_per_node, src_offsets=sh["shard_offsets"])
    _check_plan_full(step.plan, ref)
    _check_rows_full(step, ref, lambda t: w.x if t is None else perm[t])
    _check_combine_full(step, ref, w.gates2[perm], w.dtype)
    before = oracle.dispatch_plan(w.topk2, None, w.expert_rank2, w.G, w.ranks_per_node)
    share_before = before["counters"][3] / (w.T * w.k)
    share_after = ref["counters"][3] / (w.T * w.k)
    say("local share before/after shuffle", share_before, share_after)
    assert share_after > share_before


@pytest.mark.parametrize("cfg", [3, 4])
@pytest.mark.parametrize("balanced", [False, True])
def test_shuffle_at_scale_fullsize(cfg, balanced):
    """Both shuffles at workload 3's and 4's full shapes (G = 32 and 64 ranks,
    T = 65 536 and 32 768 tokens), the next layer routing like this one
    (transitions = this layer's pair counts, computed by the oracle), against
    the oracle in full."""
    from co_activation_amd import ops
    w = make(cfg, with_x=False)
    say("fullsize shuffle", cfg, w.T, w.G, "balanced" if balanced else "free")
    st = oracle.coact_stats(w.topk, w.E, w.topk, w.E)
    err = ops.new_error_word()
    got = ops.shuffle_predict(i32(w.topk), i32(st["transition"]), i32(w.expert_rank), w.G,
                              balanced=balanced, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))
    ref = (oracle.shuffle_balanced if balanced else oracle.shuffle_predict)(
        w.topk, st["transition"], w.expert_rank, w.G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(got[key]), ref[key], key)


@pytest.mark.parametrize("balanced", [False, True])
def test_shuffle_past_exchange_limit(balanced):
    """More tokens than the one-launch exchange form takes (over 2^20): the
    shuffles fall back to one launch per round and the plan's sort; checked
    in full against the oracle."""
    from co_activation_amd import ops
    T, E, k, G = 1_100_000, 16, 2, 8
    rng = np.random.default_rng(11)
    topk = np.stack([rng.choice(E, size=k, replace=False) for _ in range(512)])[
        rng.integers(0, 512, size=T)].astype(np.int32)
    X = rng.integers(0, 50, size=(E, E)).astype(np.int32)
    er = (np.arange(E) // (E // G)).astype(np.int32)
    say("shuffle past the exchange limit", T, G, balanced)
    err = ops.new_error_word()
    got = ops.shuffle_predict(i32(topk), i32(X), i32(er), G, balanced=balanced, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))
    ref = (oracle.shuffle_balanced if balanced else oracle.shuffle_predict)(topk, X, er, G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(got[key]), ref[key], key)


@pytest.mark.parametrize("T,G,E,k", [(200_000, 8, 16, 2), (300_000, 32, 64, 2),
                                     (409_600, 64, 256, 4)])
def test_balanced_exchange_several_tokens_per_thread(T, G, E, k):
    """The one-launch balanced shuffle with two to four tokens per thread
    (more than 2^17 tokens, up to its limit of 2^19): checked in full
    against the oracle."""
    from co_activation_amd import ops
    rng = np.random.default_rng(T + G)
    topk = np.stack([rng.choice(E, size=k, replace=False) for _ in range(1024)])[
        rng.integers(0, 1024, size=T)].astype(np.int32)
    X = rng.integers(0, 50, size=(E, E)).astype(np.int32)
    er = rng.permutation(np.arange(E) // (E // G)).astype(np.int32)
    say("balanced exchange, several tokens per thread", T, G)
    err = ops.new_error_word()
    got = ops.shuffle_predict(i32(topk), i32(X), i32(er), G, balanced=True, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))
    ref = oracle.shuffle_balanced(topk, X, er, G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(got[key]), ref[key], key)


def _check_sum(got, ref32, scale, dt, what):
    """A sum of several terms: fp32 within 1e-5 of the terms' magnitude; bf16
    within 1 ulp of the oracle's fp32 value rounded once, or within the fp32
    bound where the terms cancel."""
    if dt == "bf16":
        d = bf16_ulps(got, oracle.bf16_round(ref32))
        near = np.abs(oracle.bf16_to_f32(got).astype(np.float64) - ref32) <= 1e-5 * scale
        ok = (d <= 1) | near
    else:
        ok = np.abs(got.astype(np.float64) - ref32) <= 1e-5 * scale + 1e-30
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} elements out of tolerance"


def _f64(a, dt):
    return oracle.bf16_to_f32(a).astype(np.float64) if dt == "bf16" else a.astype(np.float64)


@pytest.mark.parametrize("cfg", [5, 4])
def test_expert_side_fullsize(cfg):
    """Destination side and its backward at full size, after the step the
    benchmark times (the two-layer step of workload 5, the layer of workload
    4): the expert layout in full, and expansion, reply rows, reply combine
    and every backward output on a seeded sample of tokens, each computed by
    the oracle on that sample."""
    w = make(cfg)
    dt = w.dtype
    say("fullsize expert side", cfg, w.T, w.H)
    cap = w.T * min(w.k, w.G)
    z = device_normal(cap, w.H, dt, seed=1)
    if cfg == 5:
        step = TwoLayerStep(i32(w.topk), i32(w.topk2), dev(w.gates2), i32(w.expert_rank2),
                            x_tensor(w), z, w.G, w.ranks_per_node, E1=w.E)
    else:
        step = LayerStep(i32(w.topk), dev(w.gates), i32(w.expert_rank), x_tensor(w), z, w.G,
                         w.ranks_per_node)
    step.run()
    side = ExpertSideStep(step)
    side.dispatch()
    y_expert = device_normal(w.T * w.k, w.H, dt, seed=2)
    dy = device_normal(w.T, w.H, dt, seed=3)
    d_in = device_normal(w.T * w.k, w.H, dt, seed=4)
    side.reply_and_combine(y_expert)
    bw = ExpertSideBackward(side).run(dy, y_expert, d_in)
    torch.cuda.synchronize()
    assert int(step.d_err.item()) == 0

    if cfg == 5:
        st = oracle.coact_stats(w.topk, w.E, w.topk2, w.E)
        sh = oracle.shuffle_predict(w.topk, st["transition"], w.expert_rank2, w.G)
        perm, er, src = sh["perm"], w.expert_rank2, sh["shard_offsets"]
        topk_s, gates_s = w.topk2[perm], w.gates2[perm]
    else:
        perm, er, src = np.arange(w.T), w.expert_rank, None
        topk_s, gates_s = w.topk, w.gates
    rp = oracle.dispatch_plan(topk_s, gates_s, er, w.G, w.ranks_per_node, src_offsets=src)
    ref = oracle.expert_plan(topk_s, gates_s, er, w.G, rp["slot_row"], rp["N"])
    for key in ("erow", "expert_first", "expert_count", "rank_offsets", "erow_slot", "erow_src"):
        assert_equal(host(side.plan[key]), ref[key], key)
    assert_equal(host(side.plan["erow_weight"]).view(np.uint32),
                 ref["erow_weight"].view(np.uint32), "erow_weight")
    rd = host(side.plan["row_dest"])
    N = int(rp["N"])
    assert_equal(rd[:N], ref["row_dest"], "row_dest")
    assert (rd[N:] == -1).all()

    # a sample of tokens; every row they touch, in compact numbering
    rng = np.random.default_rng(55)
    toks = np.sort(rng.choice(w.T, size=SAMPLES, replace=False))
    S, k = toks.size, w.k
    erows = ref["erow"][toks]                               # [S, k] expert rows
    erow_c = np.arange(S * k).reshape(S, k)                 # compact expert rows
    srows = rp["slot_row"][toks]                            # [S, k] send rows
    uniq, inv = np.unique(srows, return_inverse=True)
    slot_c = inv.reshape(S, k)                              # compact send rows
    trows = rp["token_rows"][toks]
    trows_c = np.where(trows >= 0, np.searchsorted(uniq, np.maximum(trows, 0)), -1)
    rd_c = np.full((uniq.size, k), -1, np.int64)            # compact row_dest
    pos = {int(e): i for i, e in enumerate(erows.reshape(-1))}
    for i, r in enumerate(uniq):
        for q in range(k):
            if ref["row_dest"][r, q] >= 0:
                rd_c[i, q] = pos[int(ref["row_dest"][r, q])]
    sel_e = torch.from_numpy(erows.reshape(-1)).cuda()
    sel_s = torch.from_numpy(uniq).cuda()
    sel_t = torch.from_numpy(toks).cuda()

    # expansion: each expert row is its token's (shuffled) row
    assert_equal(host(side.expert_in[sel_e]), np.repeat(w.x[perm[toks]], k, axis=0), "expanded")
    # reply rows
    Y = host(y_expert[sel_e])
    Yf = _f64(Y, dt)
    Zref = oracle.partial_combine(Y, dt, erow_c, gates_s[toks], slot_c, uniq.size, "f32")
    scale = np.zeros((uniq.size, w.H))
    for s_ in range(S):
        for j in range(k):
            scale[slot_c[s_, j]] += abs(float(gates_s[toks[s_], j])) * np.abs(Yf[erow_c[s_, j]])
    Z = host(side.reply[sel_s])
    _check_sum(Z, Zref.astype(np.float64), scale, dt, "reply rows")
    # reply combine
    Zf = _f64(Z, dt)
    yref = oracle.combine_unweighted(Z, dt, trows_c, "f32").astype(np.float64)
    sc = np.zeros((S, w.H))
    for q in range(k):
        m = trows_c[:, q] >= 0
        sc[m] += np.abs(Zf[trows_c[m, q]])
    _check_sum(host(side.y[sel_t]), yref, sc, dt, "reply combine")

    # backward: reply-row gradients are copies of dy
    DY = host(dy[sel_t])
    tok_of_row = np.empty(uniq.size, np.int64)
    for s_ in range(S):
        tok_of_row[slot_c[s_]] = s_
    dR = host(bw.d_reply[sel_s])
    assert_equal(dR, DY[tok_of_row], "reply-row gradients")
    # expert-output gradients: gate times the reply-row gradient, rounded once
    want = oracle.permute_scaled(dR, dt, rd_c, ref["erow_weight"][erows.reshape(-1)], S * k, dt)
    assert_equal(host(bw.d_expert_out[sel_e]), want, "expert-output gradients")
    # gate gradients
    dw = host(bw.dw[sel_t]).astype(np.float64)
    dref = oracle.row_dot(DY, dt, Y, dt, erow_c).astype(np.float64)
    DYf = _f64(DY, dt)
    dsc = np.array([[float(np.sum(np.abs(DYf[s_] * Yf[erow_c[s_, j]]))) for j in range(k)]
                    for s_ in range(S)])
    assert (np.abs(dw - dref) <= 1e-5 * dsc + 1e-30).all(), "gate gradients"
    # send-row gradients: sum of the expert-input gradients of the row
    DI = host(d_in[sel_e])
    DIf = _f64(DI, dt)
    sref = oracle.combine_unweighted(DI, dt, rd_c, "f32").astype(np.float64)
    ssc = np.zeros((uniq.size, w.H))
    for q in range(k):
        m = rd_c[:, q] >= 0
        ssc[m] += np.abs(DIf[rd_c[m, q]])
    dS = host(bw.d_send[sel_s])
    _check_sum(dS, sref, ssc, dt, "send-row gradients")
    # token gradients
    dSf = _f64(dS, dt)
    xref = oracle.combine_unweighted(dS, dt, trows_c, "f32").astype(np.float64)
    xsc = np.zeros((S, w.H))
    for q in range(k):
        m = trows_c[:, q] >= 0
        xsc[m] += np.abs(dSf[trows_c[m, q]])
    _check_sum(host(bw.dx[sel_t]), xref, xsc, dt, "token gradients")
