"""Parity of the backward mirror with the CPU oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd import ops
from co_activation_amd.pipeline import ExpertSideBackward, ExpertSideStep, LayerBackward, LayerStep
from gpu_util import assert_equal, bf16_ulps, dev, host, i32, say, x_tensor
from workloads import make, expert_outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def _no_errors(err):
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))


def _f(x, dt):
    return oracle.bf16_to_f32(x).astype(np.float64) if dt == "bf16" else x.astype(np.float64)


def _check_dot(got, a, adt, b, bdt, rows, what):
    ref = oracle.row_dot(a, adt, b, bdt, rows).astype(np.float64)
    af, bf = _f(a, adt), _f(b, bdt)
    scale = np.zeros(rows.shape)
    for t in range(rows.shape[0]):
        for q in range(rows.shape[1]):
            if rows[t, q] >= 0:
                scale[t, q] = float(np.sum(np.abs(af[t] * bf[rows[t, q]])))
    assert (np.abs(got.astype(np.float64) - ref) <= 1e-5 * scale + 1e-30).all(), what


@pytest.mark.parametrize("xd,od,H", [("bf16", "bf16", 4096), ("f32", "f32", 128), ("bf16", "f32", 512),
                                     ("f32", "bf16", 256), ("bf16", "bf16", 7168)])
def test_permute_scaled_bit_exact(xd, od, H):
    """The fp32 product of an fp32 scale and a bf16/fp32 value, rounded once,
    equals the oracle's exact product rounded once: bit for bit."""
    rng = np.random.default_rng(H)
    T, width = 300, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    xin = oracle.bf16_round(x) if xd == "bf16" else x
    out_rows = T * width + 11
    dest = rng.permutation(out_rows)[:T * width].reshape(T, width).astype(np.int32)
    dest[rng.random((T, width)) < 0.25] = -1
    scale = rng.standard_normal(out_rows).astype(np.float32)
    say("permute_scaled", xd, od, H)
    err = ops.new_error_word()
    tdt = torch.bfloat16 if od == "bf16" else torch.float32
    out = torch.zeros((out_rows, H), dtype=tdt, device="cuda")
    ops.permute_scaled(dev(xin), i32(dest), dev(scale), out_rows, out_dtype=tdt, out=out, d_err=err)
    _no_errors(err)
    ref = oracle.permute_scaled(xin, xd, dest, scale, out_rows, od)
    got = host(out)
    if od == "f32":
        assert_equal(got.view(np.uint32), ref.view(np.uint32), "scaled rows")
    else:
        assert_equal(got, ref, "scaled rows")


@pytest.mark.parametrize("ad,bd,H,width", [("bf16", "bf16", 4096, 2), ("f32", "f32", 128, 3),
                                            ("bf16", "f32", 1024, 8), ("bf16", "bf16", 7168, 6)])
def test_row_dot_parity(ad, bd, H, width):
    rng = np.random.default_rng(H + width)
    T, b_rows = 200, 500
    a = rng.standard_normal((T, H)).astype(np.float32)
    b = rng.standard_normal((b_rows, H)).astype(np.float32)
    a_in = oracle.bf16_round(a) if ad == "bf16" else a
    b_in = oracle.bf16_round(b) if bd == "bf16" else b
    rows = rng.integers(-1, b_rows, size=(T, width)).astype(np.int32)
    say("row_dot", ad, bd, H, width)
    err = ops.new_error_word()
    got = ops.row_dot(dev(a_in), dev(b_in), i32(rows), d_err=err)
    _no_errors(err)
    _check_dot(host(got), a_in, ad, b_in, bd, rows, "row dot")


@pytest.mark.parametrize("cfg,T,H", [(2, 1000, 2048), (3, 1056, 1024), (1, 2048, 128)])
def test_layer_backward_parity(cfg, T, H):
    w = make(cfg, T=T, H=H)
    say("layer backward", cfg, T, H)
    cap = w.T * min(w.k, w.G)
    Zh = expert_outputs(cap, w.H, w.dtype, seed=1)
    layer = LayerStep(i32(w.topk), dev(w.gates), i32(w.expert_rank), x_tensor(w), dev(Zh), w.G,
                      w.ranks_per_node)
    layer.run()
    dyh = expert_outputs(w.T, w.H, w.dtype, seed=3)
    dsh = expert_outputs(cap, w.H, w.dtype, seed=4)
    bw = LayerBackward(layer).run(dev(dyh), dev(dsh))
    _no_errors(layer.d_err)
    rp = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    N = rp["N"]
    dz = oracle.permute_scaled(dyh, w.dtype, rp["token_rows"], rp["row_weight"], N, w.dtype)
    got = host(bw.dz)[:N]
    assert_equal(got.view(np.uint16 if w.dtype == "bf16" else np.uint32),
                 dz.view(np.uint16 if w.dtype == "bf16" else np.uint32), "dz")
    _check_dot(host(bw.dw), dyh, w.dtype, Zh, w.dtype, rp["slot_row"], "dw")
    dx = oracle.combine_unweighted(dsh[:N], w.dtype, rp["token_rows"], "f32")
    dxf = _f(host(bw.dx), w.dtype)
    sc = np.zeros_like(dx, dtype=np.float64)
    for q in range(w.k):
        m = rp["token_rows"][:, q] >= 0
        sc[m] += np.abs(_f(dsh, w.dtype)[rp["token_rows"][m, q]])
    if w.dtype == "bf16":
        d = bf16_ulps(host(bw.dx), oracle.bf16_round(dx))
        assert ((d <= 1) | (np.abs(dxf - dx) <= 1e-5 * sc)).all()
    else:
        assert (np.abs(dxf - dx) <= 1e-5 * sc + 1e-30).all()


def test_expert_side_backward_adjoint():
    """With identity experts the backward chain is the transpose of the
    forward chain: <dy, y(x)> = <dx, x> (dy = x, so both sides are of the
    size of |x|^2 and a missing gate factor shows), and dw_tj = <dy_t, x_t>."""
    w = make(5, T=2048, H=1024)
    say("expert side backward")
    cap = w.T * min(w.k, w.G)
    z = dev(expert_outputs(cap, w.H, w.dtype, seed=1))
    layer = LayerStep(i32(w.topk), dev(w.gates), i32(w.expert_rank), x_tensor(w), z, w.G,
                      w.ranks_per_node)
    layer.run()
    side = ExpertSideStep(layer).dispatch()
    expert_out = side.expert_in                   # identity experts
    side.reply_and_combine(expert_out)
    dyh = w.x
    dy = dev(dyh)
    bw = ExpertSideBackward(side)
    bw.run(dy, expert_out, bw.d_expert_out)       # identity experts: d(in) = d(out)
    _no_errors(layer.d_err)
    xf = _f(w.x, "bf16")
    dyf = _f(dyh, "bf16")
    y = _f(host(side.y), "bf16")
    dx = _f(host(bw.dx), "bf16")
    lhs = float(np.sum(dyf * y))
    rhs = float(np.sum(dx * xf))
    mag = float(np.sum(np.abs(dyf) * np.abs(xf)))
    assert lhs > 0.9 * mag and abs(lhs - rhs) <= 1e-2 * mag
    dw = host(bw.dw)
    ref = np.einsum("th,th->t", dyf, xf)
    for j in range(w.k):
        assert (np.abs(dw[:, j] - ref) <= 1e-2 * np.einsum("th,th->t", np.abs(dyf), np.abs(xf))).all()
