"""Parity of the destination-side path (expert layout, expansion, reply rows,
reply combine) with the CPU oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd import ops
from co_activation_amd.pipeline import ExpertSideStep, LayerStep
from gpu_util import assert_equal, bf16_ulps, combine_scale, dev, host, i32, say, x_tensor
from workloads import make, expert_outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def _no_errors(err):
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))


def _check_expert_plan(ep, ref, cap):
    for key in ("erow", "expert_first", "expert_count", "rank_offsets", "erow_slot", "erow_src"):
        assert_equal(host(ep[key]), ref[key], key)
    assert_equal(host(ep["erow_weight"]).view(np.uint32), ref["erow_weight"].view(np.uint32),
                 "erow_weight")
    want = np.full((cap, ref["row_dest"].shape[1]), -1, np.int64)
    want[:ref["row_dest"].shape[0]] = ref["row_dest"]
    assert_equal(host(ep["row_dest"]), want, "row_dest")


CASES = [(1, 2048, "main"), (2, 3000, "main"), (2, 3000, "alt"), (3, 3104, "main"),
         (4, 1472, "main"), (4, 1472, "alt"), (5, 4104, "main"), (3, 32, "main")]


@pytest.mark.parametrize("cfg,T,placement", CASES)
def test_expert_plan_parity(cfg, T, placement):
    w = make(cfg, T=T, with_x=False)
    er = w.expert_rank if placement == "main" else w.alt_expert_rank
    say("expert plan", cfg, w.T, placement)
    err = ops.new_error_word()
    plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(er), w.G, w.ranks_per_node, d_err=err)
    cap = w.T * min(w.k, w.G)
    ep = ops.expert_plan(i32(w.topk), dev(w.gates), i32(er), w.G, plan.slot_row, cap, d_err=err)
    _no_errors(err)
    rp = oracle.dispatch_plan(w.topk, w.gates, er, w.G, w.ranks_per_node)
    ref = oracle.expert_plan(w.topk, w.gates, er, w.G, rp["slot_row"], rp["N"])
    _check_expert_plan(ep, ref, cap)


@pytest.mark.parametrize("T,E,k,G,seed", [(0, 8, 2, 4, 0), (257, 256, 8, 64, 1), (1000, 16, 3, 1, 2),
                                          (600, 64, 1, 8, 3)])
def test_expert_plan_edges(T, E, k, G, seed):
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    er = rng.integers(0, G, size=E).astype(np.int32)
    say("expert plan edge", T, E, k, G)
    err = ops.new_error_word()
    plan = ops.dispatch_plan(i32(topk), dev(gates), i32(er), G, G, src_offsets=i32([0] * G + [T]),
                             row_capacity=max(T * min(k, G), 1), d_err=err)
    cap = max(T * min(k, G), 1)
    ep = ops.expert_plan(i32(topk), dev(gates), i32(er), G, plan.slot_row, cap, d_err=err)
    _no_errors(err)
    rp = oracle.dispatch_plan(topk, gates, er, G, G, src_offsets=[0] * G + [T])
    ref = oracle.expert_plan(topk, gates, er, G, rp["slot_row"], rp["N"])
    _check_expert_plan(ep, ref, cap)


@pytest.mark.parametrize("cfg,T,H", [(3, 1056, 1024), (5, 2048, 4096), (4, 448, 7168), (1, 2048, 128)])
def test_expert_side_parity(cfg, T, H):
    """Expansion bit-exact; reply rows within the combine tolerance and rows
    past N untouched; reply combine against the oracle's reply combine, and
    the whole path against the plain MoE output for scaling experts."""
    w = make(cfg, T=T, H=H)
    say("expert side", cfg, T, H)
    cap = w.T * min(w.k, w.G)
    z = dev(expert_outputs(cap, w.H, w.dtype, seed=1))
    layer = LayerStep(i32(w.topk), dev(w.gates), i32(w.expert_rank), x_tensor(w), z, w.G,
                      w.ranks_per_node)
    layer.run()
    side = ExpertSideStep(layer)
    side.reply.fill_(7)
    side.dispatch()
    _no_errors(layer.d_err)
    rp = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    N = int(rp["N"])
    ref = oracle.expert_plan(w.topk, w.gates, w.expert_rank, w.G, rp["slot_row"], N)
    _check_expert_plan(side.plan, ref, cap)
    tok = ref["erow_slot"] // w.k
    assert_equal(host(side.expert_in), w.x[tok], "expanded rows")
    # scaling experts, computed here with torch as the stand-in expert GEMM
    rng = np.random.default_rng(cfg)
    c = rng.uniform(0.5, 2.0, size=w.E).astype(np.float32)
    e_of_row = torch.from_numpy(w.topk.reshape(-1)[ref["erow_slot"]].astype(np.int64)).cuda()
    Y = (side.expert_in.float() * torch.from_numpy(c).cuda()[e_of_row][:, None]).to(side.expert_in.dtype)
    side.reply_and_combine(Y)
    _no_errors(layer.d_err)
    Yh = host(Y)
    Zref32 = oracle.partial_combine(Yh, w.dtype, ref["erow"], w.gates, rp["slot_row"], N, "f32")
    Z = host(side.reply)
    Zf = oracle.bf16_to_f32(Z) if w.dtype == "bf16" else Z
    # reply-row scale: sum over the token's slots on the row's rank of |w| |Y|
    Yf = oracle.bf16_to_f32(Yh) if w.dtype == "bf16" else Yh
    scale = np.zeros((N, w.H), np.float64)
    for t in range(w.T):
        for j in range(w.k):
            scale[rp["slot_row"][t, j]] += abs(float(w.gates[t, j])) * np.abs(Yf[ref["erow"][t, j]])
    if w.dtype == "bf16":
        d = bf16_ulps(Z[:N], oracle.bf16_round(Zref32))
        near = np.abs(Zf[:N].astype(np.float64) - Zref32) <= 1e-5 * scale
        assert ((d <= 1) | near).all()
        assert (Z[N:] == host(torch.full((1,), 7, dtype=side.reply.dtype))[0]).all()
    else:
        assert (np.abs(Zf[:N] - Zref32) <= 1e-5 * scale + 1e-30).all()
        assert (Z[N:] == 7).all()
    # reply combine (unweighted) against the oracle on the GPU's reply rows
    yref = oracle.combine_unweighted(Z[:N], w.dtype, rp["token_rows"], "f32")
    y = host(side.y)
    yf = oracle.bf16_to_f32(y) if w.dtype == "bf16" else y
    sc2 = np.zeros_like(yref, dtype=np.float64)
    for q in range(w.k):
        m = rp["token_rows"][:, q] >= 0
        sc2[m] += np.abs(Zf[rp["token_rows"][m, q]])
    if w.dtype == "bf16":
        d = bf16_ulps(y, oracle.bf16_round(yref))
        assert ((d <= 1) | (np.abs(yf - yref) <= 1e-5 * sc2)).all()
    else:
        assert (np.abs(yf - yref) <= 1e-5 * sc2 + 1e-30).all()
    # the whole path reproduces the plain MoE layer output
    moe = oracle.moe_output(w.x, w.dtype, w.topk, w.gates, c)
    xf = oracle.bf16_to_f32(w.x) if w.dtype == "bf16" else w.x
    sc3 = np.zeros_like(moe)
    for j in range(w.k):
        sc3 += np.abs(w.gates[:, j:j + 1]) * c[w.topk[:, j]][:, None] * np.abs(xf)
    assert (np.abs(yf - moe) <= 2.0 ** -6 * sc3 + 1e-30).all()


def test_n_valid_limits_work():
    """permute and combine stop at the device-side count."""
    rng = np.random.default_rng(30)
    x = torch.from_numpy(rng.standard_normal((64, 16)).astype(np.float32)).cuda()
    dest = i32(np.arange(64).reshape(64, 1))
    out = torch.full((64, 16), -1.0, device="cuda")
    ops.permute(x, dest, 64, out=out, n_valid=i32([40]))
    torch.cuda.synchronize()
    assert torch.equal(out[:40], x[:40]) and (out[40:] == -1).all()
    y = torch.full((64, 16), -2.0, device="cuda")
    ops.combine(x, dest, None, out=y, n_valid=i32([10]))
    torch.cuda.synchronize()
    assert torch.equal(y[:10], x[:10]) and (y[10:] == -2).all()


def test_expert_plan_row_range_error():
    topk = np.array([[0, 1], [1, 2]], np.int32)
    er = np.array([0, 1, 1], np.int32)
    slot = np.array([[0, 1], [5, 2]], np.int32)   # 5 is past the 4 send rows
    err = ops.new_error_word()
    ops.expert_plan(i32(topk), None, i32(er), 2, i32(slot), 4, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 32
