"""Parity of the HIP engine with the CPU oracle, through the C ABI.

Sizes here let the oracle finish in seconds while spanning several 256-token
tiles and a ragged last tile; the full-size workloads run in
``test_gpu_fullsize.py``.  Integers, plans and permuted rows are compared bit
for bit; the combine within 1e-5 relative (fp32 output) or 1 bf16 ulp of the
oracle's fp32 value rounded once (bf16 output)."""

import numpy as np
import pytest
import torch

import oracle
from co_activation_amd import ops
from co_activation_amd.pipeline import GraphStep, LayerStep, TwoLayerStep
import gpu_util
from gpu_util import (assert_equal, check_combine, dev, f32_ulps, host, i32, say, x_tensor)
from workloads import make, expert_outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def _err():
    return ops.new_error_word()


def _no_errors(err):
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))


# ------------------------------------------------------------------ stats

STATS_CASES = [(1, 2048), (2, 3000), (3, 2900), (4, 1500), (5, 4001), (4, 257), (3, 1)]


@pytest.mark.parametrize("cfg,T", STATS_CASES)
def test_stats_parity(cfg, T):
    w = make(cfg, T=T, with_x=False)
    nxt = w.topk2 if cfg == 5 else None
    say("stats", cfg, T)
    err = _err()
    res = ops.coact_stats(i32(w.topk), w.E, i32(nxt) if nxt is not None else None,
                          w.E if nxt is not None else None, d_err=err)
    _no_errors(err)
    ref = oracle.coact_stats(w.topk, w.E, nxt, w.E if nxt is not None else None)
    assert_equal(host(res["expert_count"]), ref["expert_count"], "expert_count")
    assert_equal(host(res["pair_count"]), ref["pair_count"], "pair_count")
    assert f32_ulps(host(res["ochiai"]), ref["ochiai"]).max() <= 1
    assert_equal(host(res["ochiai"]), ref["ochiai"], "ochiai (expected bit-exact)")
    if nxt is not None:
        assert_equal(host(res["transition"]), ref["transition"], "transition")


def test_stats_counts_only_and_large_E():
    rng = np.random.default_rng(11)
    T, E, k = 5000, 256, 8
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    nxt = np.stack([rng.permutation(200)[:3] for _ in range(T)]).astype(np.int32)
    say("stats counts-only / E=256 transitions")
    err = _err()
    res = ops.coact_stats(i32(topk), E, pairs=False, d_err=err)
    _no_errors(err)
    ref = oracle.coact_stats(topk, E, nxt, 200)
    assert_equal(host(res["expert_count"]), ref["expert_count"], "expert_count")
    res = ops.coact_stats(i32(topk), E, i32(nxt), 200, d_err=err)
    _no_errors(err)
    assert_equal(host(res["pair_count"]), ref["pair_count"], "pair_count")
    assert_equal(host(res["transition"]), ref["transition"], "transition")
    assert_equal(host(res["ochiai"]), ref["ochiai"], "ochiai")


# ------------------------------------------------------------------ plan

def _check_plan(plan, ref, T, k):
    N = int(ref["N"])
    assert_equal(host(plan.counters), ref["counters"], "counters")
    assert_equal(host(plan.send_counts), ref["send_counts"], "send_counts")
    assert_equal(host(plan.send_offsets), ref["send_offsets"], "send_offsets")
    assert_equal(host(plan.row_token)[:N], ref["row_token"], "row_token")
    if plan.row_weight is not None:
        assert_equal(host(plan.row_weight)[:N].view(np.uint32),
                     ref["row_weight"].view(np.uint32), "row_weight bits")
    assert_equal(host(plan.token_rows), ref["token_rows"], "token_rows")
    if plan.slot_row is not None:
        assert_equal(host(plan.slot_row), ref["slot_row"], "slot_row")


PLAN_CASES = [(1, 2048, "main"), (2, 3000, "main"), (2, 3000, "alt"), (3, 3104, "main"),
              (3, 3104, "alt"), (4, 1472, "main"), (4, 1472, "alt"), (5, 4104, "main")]


@pytest.mark.parametrize("cfg,T,placement", PLAN_CASES)
def test_plan_parity(cfg, T, placement):
    w = make(cfg, T=T, with_x=False)
    er = w.expert_rank if placement == "main" else w.alt_expert_rank
    say("plan", cfg, T, placement)
    err = _err()
    plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(er), w.G, w.ranks_per_node, d_err=err)
    _no_errors(err)
    ref = oracle.dispatch_plan(w.topk, w.gates, er, w.G, w.ranks_per_node)
    _check_plan(plan, ref, w.T, w.k)


@pytest.mark.parametrize("G,rn", [(64, 8), (32, 4)])
def test_plan_large_tile_count(G, rn):
    """Many tiles on many ranks: 65 536 tokens on 64 ranks and 147 456 on
    32, over uneven shards (the scan walks several chunks of 64 tiles per
    rank), compared in full."""
    T = 65536 if G == 64 else 147456
    rng = np.random.default_rng(G)
    E, k = 128, 4
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    er = rng.integers(0, G, size=E).astype(np.int32)
    cuts = np.sort(rng.integers(0, T + 1, size=G - 1))
    src = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    say("plan, large tile count", T, G)
    err = _err()
    plan = ops.dispatch_plan(i32(topk), dev(gates), i32(er), G, rn, src_offsets=i32(src),
                             d_err=err)
    _no_errors(err)
    ref = oracle.dispatch_plan(topk, gates, er, G, rn, src_offsets=src)
    _check_plan(plan, ref, T, k)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plan_uneven_shards(seed):
    """Explicit source offsets: uneven, empty shards, a shard of one token."""
    rng = np.random.default_rng(100 + seed)
    w = make(3, T=3000, with_x=False)
    cuts = np.sort(rng.integers(0, w.T + 1, size=w.G - 1))
    cuts[:3] = cuts[3]           # empty shards
    cuts[-1] = w.T               # empty last shard
    off = np.concatenate([[0], cuts, [w.T]]).astype(np.int32)
    say("plan uneven", seed)
    err = _err()
    plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(w.expert_rank), w.G,
                             w.ranks_per_node, i32(off), d_err=err)
    _no_errors(err)
    ref = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node, off)
    _check_plan(plan, ref, w.T, w.k)


EDGE = [
    # T, E, k, G, Rn, seed
    (0, 8, 2, 4, 2, 0),
    (1, 8, 2, 1, 1, 1),
    (5, 4, 1, 1, 1, 2),
    (256, 16, 4, 16, 4, 3),
    (257, 16, 4, 1, 1, 4),
    (4096, 256, 8, 64, 8, 5),
    (640, 64, 8, 64, 1, 6),
    (512, 8, 8, 8, 2, 7),        # E = G = k: every token goes to every rank
]


@pytest.mark.parametrize("T,E,k,G,Rn,seed", EDGE)
def test_plan_edges(T, E, k, G, Rn, seed):
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    er = rng.integers(0, G, size=E).astype(np.int32)
    say("plan edge", T, E, k, G, Rn)
    err = _err()
    plan = ops.dispatch_plan(i32(topk), dev(gates), i32(er), G, Rn,
                             row_capacity=max(T * min(k, G), 1), d_err=err)
    _no_errors(err)
    ref = oracle.dispatch_plan(topk, gates, er, G, Rn)
    _check_plan(plan, ref, T, k)


# ------------------------------------------------------------------ permute

@pytest.mark.parametrize("cfg,T,H", [(1, 2048, 128), (2, 3000, 512), (4, 1472, 7168),
                                     (3, 1056, 4096), (5, 1032, 4096), (2, 1000, 2048)])
def test_permute_parity(cfg, T, H):
    w = make(cfg, T=T, H=H)
    say("permute", cfg, T, H)
    err = _err()
    plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(w.expert_rank), w.G,
                             w.ranks_per_node, d_err=err)
    ref = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    N = int(ref["N"])
    cap = w.T * min(w.k, w.G)
    x = x_tensor(w)
    out = torch.empty((cap, H), dtype=x.dtype, device=x.device)
    ops.permute(x, plan.token_rows, cap, out=out, d_err=err)
    _no_errors(err)
    _check_plan(plan, ref, w.T, w.k)
    want = oracle.permute_rows(w.x, ref["row_token"])
    assert_equal(host(out)[:N], want, "send rows")


def test_permute_narrow_rows_and_untouched():
    """4-byte path (8-byte rows), width 1, and rows nobody targets stay as
    they were."""
    rng = np.random.default_rng(12)
    T = 1000
    rows = rng.integers(-2**31, 2**31 - 1, size=(T, 2), dtype=np.int64).astype(np.int32)
    dest = rng.permutation(T + 37)[:T].astype(np.int32)
    say("permute narrow")
    err = _err()
    out = torch.full((T + 37, 2), -7, dtype=torch.int32, device="cuda")
    ops.permute(i32(rows), i32(dest), T + 37, out=out, d_err=err)
    _no_errors(err)
    got = host(out)
    exp = oracle.scatter_rows(rows, dest, T + 37)
    targeted = np.isin(np.arange(T + 37), dest)
    assert_equal(got[targeted], exp[targeted], "scattered rows")
    assert (got[~targeted] == -7).all()


@pytest.mark.parametrize("row_bytes,width", [(8192, 6), (14336, 8), (6400, 3), (16384, 4),
                                             (8464, 5)])
def test_permute_fanout_paths(row_bytes, width):
    """Wide rows with more than two destinations, through the fan-out launch
    (6-8 KiB rows) and the split one (rows over 8 KiB, one wave per 2 KiB
    part; 8464 bytes leave a ragged last part): scattered -1 entries, a
    device row count, and a destination past the output (reported, skipped,
    nothing else written wrong)."""
    rng = np.random.default_rng(row_bytes + width)
    T = 700
    words = row_bytes // 4
    x = rng.integers(-2**31, 2**31 - 1, size=(T, words), dtype=np.int64).astype(np.int32)
    out_rows = T * width + 5
    dest = rng.permutation(out_rows)[:T * width].reshape(T, width).astype(np.int32)
    dest[rng.random((T, width)) < 0.3] = -1
    say("permute fan-out", row_bytes, width)
    err = _err()
    out = torch.full((out_rows, words), -7, dtype=torch.int32, device="cuda")
    ops.permute(i32(x), i32(dest), out_rows, out=out, d_err=err)
    _no_errors(err)
    got = host(out)
    want = np.full((out_rows, words), -7, np.int32)
    for t in range(T):
        for q in range(width):
            if dest[t, q] >= 0:
                want[dest[t, q]] = x[t]
    assert_equal(got, want, "fan-out rows")
    # device row count: tokens past it move nothing
    out2 = torch.full((out_rows, words), -7, dtype=torch.int32, device="cuda")
    ops.permute(i32(x), i32(dest), out_rows, out=out2, n_valid=i32([123]), d_err=err)
    _no_errors(err)
    want2 = np.full((out_rows, words), -7, np.int32)
    for t in range(123):
        for q in range(width):
            if dest[t, q] >= 0:
                want2[dest[t, q]] = x[t]
    assert_equal(host(out2), want2, "fan-out rows, device count")
    # one destination past the output: reported and skipped
    bad = dest.copy()
    bad[5, width - 1] = out_rows
    out3 = torch.full((out_rows, words), -7, dtype=torch.int32, device="cuda")
    ops.permute(i32(x), i32(bad), out_rows, out=out3, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 32
    want3 = want.copy()
    if dest[5, width - 1] >= 0:
        want3[dest[5, width - 1]] = -7
    assert_equal(host(out3), want3, "fan-out rows with a bad destination")


@pytest.mark.parametrize("row_bytes,k", [(8192, 2), (14336, 8), (1024, 3), (48, 1), (8, 2), (12, 4)])
def test_shuffle_dispatch_parity(row_bytes, k):
    """The shuffle's move fused with the next layer's permute, bit for bit
    against the oracle over every launch shape (16-byte and 4-byte rows);
    rows no position targets stay as they were."""
    rng = np.random.default_rng(row_bytes + k)
    T = 777
    words = row_bytes // 4
    x = rng.integers(-2**31, 2**31 - 1, size=(T, words), dtype=np.int64).astype(np.int32)
    perm = rng.permutation(T).astype(np.int32)
    send_rows = T * k + 9
    token_rows = rng.permutation(send_rows)[:T * k].reshape(T, k).astype(np.int32)
    token_rows[rng.random((T, k)) < 0.3] = -1
    say("shuffle dispatch", row_bytes, k)
    err = _err()
    xo = torch.full((T, words), -5, dtype=torch.int32, device="cuda")
    sd = torch.full((send_rows, words), -7, dtype=torch.int32, device="cuda")
    ops.shuffle_dispatch(i32(x), i32(perm), i32(token_rows), send_rows, x_out=xo, send=sd,
                         d_err=err)
    _no_errors(err)
    want_x, want_s = oracle.shuffle_dispatch(x, perm, token_rows, send_rows)
    assert_equal(host(xo), want_x, "shuffled rows")
    got = host(sd)
    hit = np.isin(np.arange(send_rows), token_rows[token_rows >= 0])
    assert_equal(got[hit], want_s[hit], "send rows")
    assert (got[~hit] == -7).all()


def test_shuffle_dispatch_errors():
    """A token index outside [0, T) or a send row past the buffer is
    reported and that copy skipped; nothing else changes."""
    T, k, words = 64, 2, 4
    rng = np.random.default_rng(77)
    x = rng.integers(0, 1000, size=(T, words)).astype(np.int32)
    perm = np.arange(T, dtype=np.int32)
    token_rows = np.arange(T * k, dtype=np.int32).reshape(T, k)
    bad_pos = perm.copy()
    bad_pos[3] = T
    say("shuffle dispatch errors")
    for dp, tr in ((bad_pos, token_rows), (perm, np.where(token_rows == 10, T * k, token_rows))):
        err = _err()
        xo = torch.full((T, words), -5, dtype=torch.int32, device="cuda")
        sd = torch.full((T * k, words), -7, dtype=torch.int32, device="cuda")
        ops.shuffle_dispatch(i32(x), i32(dp), i32(tr.astype(np.int32)), T * k, x_out=xo, send=sd,
                             d_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 32
        gx, gs = host(xo), host(sd)
        if dp is bad_pos:
            keep = np.arange(T) != 3
            assert_equal(gx[keep], x[keep], "moved rows")
            assert (gx[3] == -5).all() and (gs[6:8] == -7).all()
        else:
            assert_equal(gx, x, "moved rows")
            assert (gs[10] == -7).all()
            assert_equal(np.delete(gs, 10, axis=0), np.delete(np.repeat(x, k, axis=0), 10, axis=0),
                         "send rows")


GATHER_CASES = [(3000, 2500, 8192, 0.1), (1001, 1001, 14336, 0.0), (777, 900, 512, 0.2),
                (1500, 64, 1024, 0.0), (613, 400, 2064, 0.05), (5000, 4000, 8, 0.1),
                (300, 300, 4, 0.0), (200, 150, 48, 0.3), (1, 1, 16384, 0.0)]


@pytest.mark.parametrize("n,x_rows,row_bytes,neg", GATHER_CASES)
def test_gather_parity(n, x_rows, row_bytes, neg):
    """out[i] = x[src[i]] bit for bit over every launch shape (word rows,
    flat, wave per row, 512 threads per row with a ragged second pass);
    rows with a negative source stay as they were."""
    rng = np.random.default_rng(n + row_bytes)
    words = row_bytes // 4
    x = rng.integers(-2**31, 2**31 - 1, size=(x_rows, words), dtype=np.int64).astype(np.int32)
    src = rng.integers(0, x_rows, size=n).astype(np.int32)
    src[rng.random(n) < neg] = -1
    say("gather", n, x_rows, row_bytes)
    err = _err()
    out = torch.full((n, words), -7, dtype=torch.int32, device="cuda")
    ops.gather(i32(x), i32(src), out=out, d_err=err)
    _no_errors(err)
    got = host(out)
    ok = src >= 0
    assert_equal(got[ok], oracle.permute_rows(x, src[ok]), "gathered rows")
    assert (got[~ok] == -7).all()


def test_gather_is_the_inverse_scatter():
    """Gathering by a permutation equals scattering by its inverse: the
    shuffle's move in either form (bf16 rows of 4096 elements)."""
    w = make(5, T=2056, H=4096)
    rng = np.random.default_rng(14)
    perm = rng.permutation(w.T).astype(np.int32)
    dest = np.argsort(perm).astype(np.int32)
    say("gather vs scatter")
    err = _err()
    x = x_tensor(w)
    a = ops.gather(x, i32(perm), d_err=err)
    b = ops.permute(x, i32(dest), w.T, d_err=err)
    _no_errors(err)
    assert_equal(host(a), oracle.permute_rows(w.x, perm), "gather")
    assert_equal(host(a), host(b), "gather vs scatter")


def test_gather_n_valid_and_row_range():
    rng = np.random.default_rng(15)
    x = torch.from_numpy(rng.standard_normal((64, 32)).astype(np.float32)).cuda()
    src = i32(rng.integers(0, 64, size=50))
    out = torch.full((50, 32), -1.0, device="cuda")
    ops.gather(x, src, out=out, n_valid=i32([20]))
    torch.cuda.synchronize()
    assert torch.equal(out[:20], x[src[:20].long()]) and (out[20:] == -1).all()
    say("gather row range")
    err = _err()
    bad = i32([0, 1, 64, 3])        # 64 is past the 64 source rows
    out2 = torch.full((4, 32), -1.0, device="cuda")
    ops.gather(x, bad, out=out2, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 32
    assert torch.equal(out2[[0, 1, 3]], x[[0, 1, 3]]) and (out2[2] == -1).all()


# ------------------------------------------------------------------ combine

COMBINE_CASES = [(1, 2048, 128, "f32", "f32"), (1, 2048, 128, "f32", "bf16"),
                 (5, 1032, 4096, "bf16", "bf16"), (2, 1000, 2048, "bf16", "f32"),
                 (2, 3000, 512, "bf16", "bf16"), (2, 3000, 512, "bf16", "f32"),
                 (3, 1056, 4096, "bf16", "bf16"), (4, 1472, 7168, "bf16", "bf16")]


@pytest.mark.parametrize("cfg,T,H,zd,yd", COMBINE_CASES)
def test_combine_parity(cfg, T, H, zd, yd):
    w = make(cfg, T=T, H=H, with_x=False)
    say("combine", cfg, T, H, zd, yd)
    err = _err()
    plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(w.expert_rank), w.G,
                             w.ranks_per_node, d_err=err)
    ref = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    N = int(ref["N"])
    Z = expert_outputs(N, H, zd, seed=1)
    tdt = torch.bfloat16 if yd == "bf16" else torch.float32
    y = ops.combine(dev(Z), plan.token_rows, plan.row_weight, out_dtype=tdt, d_err=err)
    _no_errors(err)
    check_combine(y, Z, zd, ref["slot_row"], w.gates, yd, what=f"combine cfg{cfg}")
    # unweighted mode: the plain sum of the token's rows
    yu = ops.combine(dev(Z), plan.token_rows, None, out_dtype=torch.float32, d_err=err)
    _no_errors(err)
    refu = oracle.combine_unweighted(Z, zd, ref["token_rows"], "f32")
    Zf = oracle.bf16_to_f32(Z) if zd == "bf16" else Z
    scale = np.zeros_like(refu, dtype=np.float64)
    for q in range(w.k):
        m = ref["token_rows"][:, q] >= 0
        scale[m] += np.abs(Zf[ref["token_rows"][m, q]])
    assert (np.abs(host(yu) - refu) <= 1e-5 * scale + 1e-30).all()


@pytest.mark.parametrize("yd", ["bf16", "f32"])
def test_combine_special_values(yd):
    """Rows holding signed zeros, a subnormal, the bf16 maximum, infinities
    and NaN, weighted by 1/4, 1/2 or 1: NaN and infinities (with their sign)
    appear exactly where the oracle has them, sums past the fp32 range
    overflow on both sides, and every finite element meets the usual bound.
    With this pool every sum is either exactly representable or at least 3%
    away from an overflow threshold, far beyond any rounding-order effect.
    (No zero gates: when two slots share a row the kernel scales the row by
    their summed gate, while the definition sums the slots; with an infinite
    row and a zero gate the two differ by 0 * inf.)"""
    rng = np.random.default_rng(41)
    T, E, k, G, H = 512, 4, 2, 2, 64
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    er = np.array([0, 0, 1, 1], np.int32)
    gates = rng.choice(np.array([0.25, 0.5, 1.0], np.float32), size=(T, k))
    say("combine special values", yd)
    err = _err()
    plan = ops.dispatch_plan(i32(topk), dev(gates), i32(er), G, G, d_err=err)
    ref_plan = oracle.dispatch_plan(topk, gates, er, G, G)
    N = int(ref_plan["N"])
    pool = np.array([0x0000, 0x8000, 0x0001, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
                     0x7FC0, 0x7E00, 0x4049], np.uint16)
    Z = rng.choice(pool, size=(T * min(k, G), H)).astype(np.uint16)
    tdt = torch.bfloat16 if yd == "bf16" else torch.float32
    y = ops.combine(dev(Z), plan.token_rows, plan.row_weight, out_dtype=tdt, d_err=err)
    _no_errors(err)
    got = oracle.bf16_to_f32(host(y)) if yd == "bf16" else host(y)
    with np.errstate(all="ignore"):  # the reference overflows and makes NaN on purpose
        ref32 = oracle.combine(Z, "bf16", ref_plan["slot_row"], gates, "f32")
        ref = oracle.bf16_to_f32(oracle.bf16_round(ref32)) if yd == "bf16" else ref32
        scale_all = gpu_util.combine_scale(Z, "bf16", ref_plan["slot_row"], gates)
    assert N > T
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN positions"
    for sign in (1, -1):
        assert np.array_equal(got == sign * np.inf, ref == sign * np.inf), f"{sign:+d} infinity"
    assert np.isnan(ref).any() and np.isinf(ref).any() and np.isfinite(ref).any()
    fin = np.isfinite(ref)
    dev_err = np.abs(got[fin].astype(np.float64) - ref32[fin].astype(np.float64))
    scale = scale_all[fin]
    if yd == "f32":
        assert (dev_err <= 1e-5 * scale + 1e-30).all()
    else:
        d = gpu_util.bf16_ulps(host(y)[fin], oracle.bf16_round(ref32)[fin])
        assert ((d <= 1) | (dev_err <= 1e-5 * scale)).all()


@pytest.mark.parametrize("cfg,T", [(5, 4096), (3, 2560), (4, 1313)])
def test_gathered_plan_parity(cfg, T):
    """moe_dispatch_plan_gathered against the oracle: random orders, shards
    of uneven length (as a shuffle leaves them, some empty), ragged tiles;
    every plan output and the gathered routing bit for bit.  Then a position
    whose perm entry is out of range: ROW_RANGE, no rows for it, and every
    other position planned as before."""
    w = make(cfg, T=T, H=64)
    rng = np.random.default_rng(cfg * 1000 + T)
    G = w.G
    cuts = np.sort(rng.integers(0, T + 1, size=G - 1))
    cuts[: G // 4] = 0
    src = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    perm = rng.permutation(T).astype(np.int32)
    say("gathered plan", cfg, T)
    err = _err()
    topk_out = torch.empty(T, w.k, dtype=torch.int32, device="cuda")
    gates_out = torch.empty(T, w.k, dtype=torch.float32, device="cuda")
    plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(w.expert_rank), G, w.ranks_per_node,
                             i32(src), d_err=err, perm=i32(perm), topk_out=topk_out,
                             gates_out=gates_out)
    _no_errors(err)
    ref = oracle.dispatch_plan_gathered(w.topk, w.gates, perm, w.expert_rank, G,
                                        w.ranks_per_node, src_offsets=src)
    N = int(ref["N"])
    assert_equal(host(topk_out), ref["topk_out"], "topk_out")
    assert_equal(host(gates_out).view(np.uint32), ref["gates_out"].view(np.uint32), "gates_out")
    assert_equal(host(plan.counters), ref["counters"], "counters")
    assert_equal(host(plan.send_offsets), ref["send_offsets"], "send_offsets")
    assert_equal(host(plan.row_token)[:N], ref["row_token"], "row_token")
    assert_equal(host(plan.row_weight)[:N].view(np.uint32), ref["row_weight"].view(np.uint32),
                 "row_weight")
    assert_equal(host(plan.token_rows), ref["token_rows"], "token_rows")
    assert_equal(host(plan.slot_row), ref["slot_row"], "slot_row")
    # one out-of-range entry
    bad = perm.copy()
    bad[T // 2] = T + 5
    err2 = _err()
    ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(w.expert_rank), G, w.ranks_per_node,
                      i32(src), d_err=err2, perm=i32(bad), topk_out=topk_out, gates_out=gates_out)
    torch.cuda.synchronize()
    assert int(err2.item()) == 32
    got_tr = host(topk_out)
    assert (got_tr[T // 2] == -1).all()
    keep = np.arange(T) != T // 2
    assert_equal(got_tr[keep], w.topk[bad[keep]], "topk_out around the bad entry")


def test_gathered_plan_without_gates():
    """A gathered plan with no gates (an unweighted dispatch): the routing
    alone is gathered, row weights are 0, and everything else matches the
    oracle bit for bit; equal shards (src_offsets NULL), a ragged last tile."""
    w = make(3, T=32 * 37, H=64)
    T, G = w.T, w.G
    perm = np.random.default_rng(5).permutation(T).astype(np.int32)
    say("gathered plan without gates", T, G)
    err = _err()
    topk_out = torch.empty(T, w.k, dtype=torch.int32, device="cuda")
    plan = ops.dispatch_plan(i32(w.topk), None, i32(w.expert_rank), G, w.ranks_per_node,
                             d_err=err, perm=i32(perm), topk_out=topk_out)
    _no_errors(err)
    ref = oracle.dispatch_plan_gathered(w.topk, None, perm, w.expert_rank, G, w.ranks_per_node)
    N = int(ref["N"])
    assert_equal(host(topk_out), ref["topk_out"], "topk_out")
    assert_equal(host(plan.counters), ref["counters"], "counters")
    assert_equal(host(plan.row_token)[:N], ref["row_token"], "row_token")
    assert (host(plan.row_weight)[:N] == 0).all()
    assert_equal(host(plan.token_rows), ref["token_rows"], "token_rows")
    assert_equal(host(plan.slot_row), ref["slot_row"], "slot_row")


def test_combine_of_permute_is_identity():
    """permute then weighted combine returns x bit-exact in bf16 (gates sum
    to 1 within 2^-10), and the unweighted combine gives |R_t| * x exactly."""
    w = make(3, T=1056, H=1024)
    say("combine(permute(x))")
    err = _err()
    plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(w.expert_rank), w.G,
                             w.ranks_per_node, d_err=err)
    x = x_tensor(w)
    send = ops.permute(x, plan.token_rows, w.T * min(w.k, w.G), d_err=err)
    y = ops.combine(send, plan.token_rows, plan.row_weight, d_err=err)
    yu = ops.combine(send, plan.token_rows, None, out_dtype=torch.float32, d_err=err)
    _no_errors(err)
    assert_equal(host(y), w.x, "combine(permute(x)) == x")
    nr = (host(plan.token_rows) >= 0).sum(axis=1).astype(np.float32)
    assert_equal(host(yu), oracle.bf16_to_f32(w.x) * nr[:, None], "unweighted == |R_t| x")


# ------------------------------------------------------------------ shuffle

@pytest.mark.parametrize("T", [4104, 1, 300])
def test_shuffle_parity(T):
    w = make(5, T=T, with_x=False)
    say("shuffle", T)
    err = _err()
    st = ops.coact_stats(i32(w.topk), w.E, i32(w.topk2), w.E, d_err=err)
    sh = ops.shuffle_predict(i32(w.topk), st["transition"], i32(w.expert_rank2), w.G, d_err=err)
    _no_errors(err)
    ref_st = oracle.coact_stats(w.topk, w.E, w.topk2, w.E)
    ref = oracle.shuffle_predict(w.topk, ref_st["transition"], w.expert_rank2, w.G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(sh[key]), ref[key], key)


@pytest.mark.parametrize("E,E2,k,G,seed", [(256, 256, 8, 64, 0), (16, 40, 3, 5, 1), (8, 8, 1, 3, 2)])
def test_shuffle_ties_and_shapes(E, E2, k, G, seed):
    """Small integer transitions (many ties), odd G, E up to 256."""
    rng = np.random.default_rng(seed)
    T = 2000
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    X = rng.integers(0, 3, size=(E, E2)).astype(np.int32)
    er2 = rng.integers(0, G, size=E2).astype(np.int32)
    say("shuffle shapes", E, E2, k, G)
    err = _err()
    sh = ops.shuffle_predict(i32(topk), i32(X), i32(er2), G, d_err=err)
    _no_errors(err)
    ref = oracle.shuffle_predict(topk, X, er2, G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(sh[key]), ref[key], key)


# ------------------------------------------------------------------ pipelines

def test_layer_step_parity():
    w = make(2, T=3000, H=256)
    say("layer step cfg2")
    ref = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    cap = w.T * min(w.k, w.G)
    Z = expert_outputs(cap, w.H, "bf16", seed=1)
    step = LayerStep(i32(w.topk), dev(w.gates), i32(w.expert_rank), x_tensor(w), dev(Z), w.G,
                     w.ranks_per_node)
    step.run()
    _no_errors(step.d_err)
    _check_plan(step.plan, ref, w.T, w.k)
    N = int(ref["N"])
    assert_equal(host(step.send)[:N], oracle.permute_rows(w.x, ref["row_token"]), "send")
    check_combine(step.y, Z, "bf16", ref["slot_row"], w.gates, "bf16", "layer step")
    st = oracle.coact_stats(w.topk, w.E)
    assert_equal(host(step.stats_out["pair_count"]), st["pair_count"], "pairs")


@pytest.mark.parametrize("fused", [True, False])
def test_two_layer_step_parity(fused):
    w = make(5, T=4104, H=256)
    say("two-layer step cfg5", "fused" if fused else "split")
    cap = w.T * min(w.k, w.G)
    Z = expert_outputs(cap, w.H, "bf16", seed=1)
    step = TwoLayerStep(i32(w.topk), i32(w.topk2), dev(w.gates2), i32(w.expert_rank2),
                        x_tensor(w), dev(Z), w.G, w.ranks_per_node, E1=w.E, fused=fused)
    step.run()
    _no_errors(step.d_err)
    ref = oracle.two_layer_pipeline(w.topk, w.topk2, w.gates2, w.x, w.expert_rank2, w.E, w.E,
                                    w.G, w.ranks_per_node)
    assert_equal(host(step.stats_out["transition"]), ref["stats"]["transition"], "transition")
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(step.shuffle[key]), ref["shuffle"][key], key)
    assert_equal(host(step.x_s), ref["x_shuffled"], "x shuffled")
    assert_equal(host(step.topk2_s), ref["topk2_shuffled"], "topk2 shuffled")
    assert_equal(host(step.gates2_s), ref["gates2_shuffled"], "gates2 shuffled")
    _check_plan(step.plan, ref["plan"], w.T, w.k)
    N = int(ref["plan"]["N"])
    assert_equal(host(step.send)[:N], ref["send"], "layer-2 send")
    check_combine(step.y, Z, "bf16", ref["plan"]["slot_row"], ref["gates2_shuffled"], "bf16",
                  "two-layer combine")
    c = host(step.plan.counters)
    assert c[3] / (w.T * w.k) > ref["local_share_before"]


@pytest.mark.parametrize("two_layer", [False, True])
def test_graph_replays_match_eager(two_layer):
    """A step captured as a HIP graph: every replay, with eager work and
    synchronisations between replays and the outputs cleared before each,
    gives exactly what an eager single-stream step gives."""
    if two_layer:
        w = make(5, T=8192, H=1024)
        mk = lambda: TwoLayerStep(i32(w.topk), i32(w.topk2), dev(w.gates2), i32(w.expert_rank2),
                                  x_tensor(w), dev(Z), w.G, w.ranks_per_node, E1=w.E)
    else:
        w = make(3, T=4096, H=1024)
        mk = lambda: LayerStep(i32(w.topk), dev(w.gates), i32(w.expert_rank), x_tensor(w), dev(Z),
                               w.G, w.ranks_per_node)
    say("graph replay", "two-layer" if two_layer else "one layer")
    cap = w.T * min(w.k, w.G)
    Z = expert_outputs(cap, w.H, "bf16", seed=1)
    ref = mk().run(overlap=False)
    torch.cuda.synchronize()
    N = int(host(ref.plan.counters)[0])
    want = {k: host(v) for k, v in ref.stats_out.items()}
    want.update(token_rows=host(ref.plan.token_rows), counters=host(ref.plan.counters),
                send=host(ref.send)[:N], y=host(ref.y))
    g = GraphStep(mk())
    st = g.step
    for rep in range(4):
        ref.run()                      # eager work between replays
        torch.cuda.synchronize()
        for t in (st.y, st.send, st.plan.token_rows, st.plan.counters, *st.stats_out.values()):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _no_errors(st.d_err)
        got = {k: host(v) for k, v in st.stats_out.items()}
        got.update(token_rows=host(st.plan.token_rows), counters=host(st.plan.counters),
                   send=host(st.send)[:N], y=host(st.y))
        for k in want:
            assert_equal(got[k], want[k], f"replay {rep}: {k}")


@pytest.mark.parametrize("two_layer", [False, True])
def test_overlapped_steps_match_serial(two_layer):
    """Steps that run latency-bound stages on a second stream give, after
    several back-to-back steps, exactly what one single-stream step gives
    (the two-layer step in its separate-pass form, whose layer-2 plan
    overlaps the token move)."""
    if two_layer:
        w = make(5, T=8192, H=1024)
        mk = lambda: TwoLayerStep(i32(w.topk), i32(w.topk2), dev(w.gates2), i32(w.expert_rank2),
                                  x_tensor(w), dev(Z), w.G, w.ranks_per_node, E1=w.E,
                                  fused=False)
    else:
        w = make(4, T=2048, H=1024)
        mk = lambda: LayerStep(i32(w.topk), dev(w.gates), i32(w.expert_rank), x_tensor(w), dev(Z),
                               w.G, w.ranks_per_node)
    say("overlapped vs serial steps", "two-layer" if two_layer else "one layer")
    cap = w.T * min(w.k, w.G)
    Z = expert_outputs(cap, w.H, "bf16", seed=1)
    ser = mk().run(overlap=False)
    ovl = mk()
    for _ in range(6):
        ovl.run()
    torch.cuda.synchronize()
    _no_errors(ovl.d_err)
    N = int(host(ser.plan.counters)[0])
    for key, a in ser.stats_out.items():
        assert_equal(host(ovl.stats_out[key]), host(a), key)
    for a, b, name in ((ovl.plan.token_rows, ser.plan.token_rows, "token_rows"),
                       (ovl.plan.send_offsets, ser.plan.send_offsets, "send_offsets"),
                       (ovl.plan.counters, ser.plan.counters, "counters"),
                       (ovl.y, ser.y, "y")):
        assert_equal(host(a), host(b), name)
    assert_equal(host(ovl.send)[:N], host(ser.send)[:N], "send")


# ------------------------------------------------------------------ determinism

def test_determinism():
    w = make(3, T=3104, H=512)
    say("determinism")
    outs = []
    for _ in range(2):
        err = _err()
        st = ops.coact_stats(i32(w.topk), w.E, d_err=err)
        plan = ops.dispatch_plan(i32(w.topk), dev(w.gates), i32(w.expert_rank), w.G,
                                 w.ranks_per_node, d_err=err)
        Z = dev(expert_outputs(w.T * min(w.k, w.G), w.H, "bf16", seed=1))
        y = ops.combine(Z, plan.token_rows, plan.row_weight, d_err=err)
        _no_errors(err)
        N = int(host(plan.counters)[0])
        outs.append([host(st["pair_count"]), host(st["ochiai"]), host(plan.row_token)[:N],
                     host(plan.row_weight)[:N], host(plan.token_rows), host(plan.slot_row),
                     host(plan.send_offsets), host(y)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


# ------------------------------------------------------------------ device error bits

def test_device_error_bits():
    """Bad data is reported in d_err, never read or written out of bounds."""
    rng = np.random.default_rng(13)
    T, E, k, G = 512, 16, 2, 4
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    er = (np.arange(E) // (E // G)).astype(np.int32)

    def plan_bits(tk=topk, ers=er, cap=None, off=None):
        err = _err()
        ops.dispatch_plan(i32(tk), dev(gates), i32(ers), G, G, None if off is None else i32(off),
                          row_capacity=cap, d_err=err)
        torch.cuda.synchronize()
        return int(err.item())

    say("device error bits")
    bad = topk.copy(); bad[7, 1] = E
    assert plan_bits(bad) & 1
    bad = topk.copy(); bad[9, 1] = -3
    assert plan_bits(bad) & 1
    bad = topk.copy(); bad[11, 1] = bad[11, 0]
    assert plan_bits(bad) & 2
    ers = er.copy(); ers[5] = G
    assert plan_bits(ers=ers) & 4
    ref = oracle.dispatch_plan(topk, gates, er, G, G)
    assert plan_bits(cap=int(ref["N"]) - 1) == 8
    assert plan_bits(cap=int(ref["N"])) == 0
    assert plan_bits(off=np.array([0, 100, 50, 300, T], np.int32)) & 16
    assert plan_bits(off=np.array([0, 100, 200, 300, T - 1], np.int32)) & 16
    # counters stay valid under a capacity overflow
    err = _err()
    p = ops.dispatch_plan(i32(topk), dev(gates), i32(er), G, G, row_capacity=10, d_err=err)
    torch.cuda.synchronize()
    assert_equal(host(p.counters), ref["counters"], "counters under overflow")
    # stats
    err = _err()
    bad = topk.copy(); bad[3, 0] = 99
    ops.coact_stats(i32(bad), E, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    # permute / combine row range
    err = _err()
    x = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    ops.permute(x, i32([[0], [1], [9], [2]]), 4, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 32
    err = _err()
    ops.combine(x, i32([[0, 1], [5, -1]]), None, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 32


def test_stats_repeated_ids_count_once():
    """A token that lists an expert twice is flagged and still counted as the
    set D_t: counts equal the products of the token-by-expert 0/1 matrices."""
    rng = np.random.default_rng(17)
    T, E, k, E2 = 3000, 256, 8, 64
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    nxt = np.stack([rng.permutation(E2)[:k] for _ in range(T)]).astype(np.int32)
    rows = rng.choice(T, 500, replace=False)
    topk[rows, 3] = topk[rows, 0]
    topk[rows[:100], 7] = topk[rows[:100], 0]
    A = np.zeros((T, E), np.int64)
    np.put_along_axis(A, topk.astype(np.int64), 1, axis=1)
    B = np.zeros((T, E2), np.int64)
    np.put_along_axis(B, nxt.astype(np.int64), 1, axis=1)
    say("stats with repeated ids")
    err = _err()
    res = ops.coact_stats(i32(topk), E, i32(nxt), E2, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    assert_equal(host(res["expert_count"]), A.sum(0), "expert_count")
    assert_equal(host(res["pair_count"]), A.T @ A, "pair_count")
    assert_equal(host(res["transition"]), A.T @ B, "transition")


@pytest.mark.parametrize("H,width", [(4096, 1), (7168, 1), (4096, 2), (2048, 1)])
def test_permute_token_moves(H, width):
    """One destination per token (the shuffle's move) and two, on the
    launch shapes of the wide rows."""
    rng = np.random.default_rng(H + width)
    T = 700
    x = rng.integers(0, 2**16, size=(T, H), dtype=np.int64).astype(np.uint16)
    out_rows = T * width
    dest = rng.permutation(out_rows).reshape(T, width).astype(np.int32)
    say("permute token moves", H, width)
    err = _err()
    out = ops.permute(dev(x), i32(dest), out_rows, d_err=err)
    _no_errors(err)
    want = np.empty((out_rows, H), np.uint16)
    for q in range(width):
        want[dest[:, q]] = x
    assert_equal(host(out), want, "moved rows")


@pytest.mark.parametrize("words,width", [(65, 3), (16, 2), (1, 1), (300, 8)])
def test_permute_word_rows(words, width):
    """Rows whose size is a multiple of 4 but not of 16 bytes (4-byte path,
    flat and wave-per-token variants), several destinations per token."""
    rng = np.random.default_rng(words)
    T = 777
    rows = rng.integers(-2**31, 2**31 - 1, size=(T, words), dtype=np.int64).astype(np.int32)
    out_rows = T * width + 5
    dest = rng.permutation(out_rows)[:T * width].reshape(T, width).astype(np.int32)
    dest[rng.random((T, width)) < 0.2] = -1
    say("permute words", words, width)
    err = _err()
    out = torch.full((out_rows, words), 3, dtype=torch.int32, device="cuda")
    ops.permute(i32(rows), i32(dest), out_rows, out=out, d_err=err)
    _no_errors(err)
    want = np.full((out_rows, words), 3, np.int32)
    for t in range(T):
        for q in range(width):
            if dest[t, q] >= 0:
                want[dest[t, q]] = rows[t]
    assert_equal(host(out), want, "word rows")


# ------------------------------------------------------------------ balanced shuffle

@pytest.mark.parametrize("E,E2,k,G,T,seed", [(64, 64, 2, 8, 4096, 0), (256, 256, 8, 64, 2048, 1),
                                             (16, 40, 3, 5, 1000, 2), (8, 8, 1, 3, 300, 3),
                                             (8, 8, 2, 1, 64, 4), (32, 32, 2, 4, 4, 5)])
def test_balanced_shuffle_parity(E, E2, k, G, T, seed):
    """Random small-integer transitions (many ties), every shape path."""
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    X = rng.integers(0, 3, size=(E, E2)).astype(np.int32)
    er2 = rng.integers(0, G, size=E2).astype(np.int32)
    say("balanced shuffle", E, E2, k, G, T)
    err = _err()
    sh = ops.shuffle_predict(i32(topk), i32(X), i32(er2), G, balanced=True, d_err=err)
    _no_errors(err)
    ref = oracle.shuffle_balanced(topk, X, er2, G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(sh[key]), ref[key], key)


def test_balanced_two_layer_step():
    w = make(5, T=4104, H=256)
    say("balanced two-layer step")
    cap = w.T * min(w.k, w.G)
    Z = expert_outputs(cap, w.H, "bf16", seed=1)
    step = TwoLayerStep(i32(w.topk), i32(w.topk2), dev(w.gates2), i32(w.expert_rank2),
                        x_tensor(w), dev(Z), w.G, w.ranks_per_node, E1=w.E, balanced=True)
    step.run()
    _no_errors(step.d_err)
    st = oracle.coact_stats(w.topk, w.E, w.topk2, w.E)
    sh = oracle.shuffle_balanced(w.topk, st["transition"], w.expert_rank2, w.G)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert_equal(host(step.shuffle[key]), sh[key], key)
    perm = sh["perm"]
    ref = oracle.dispatch_plan(w.topk2[perm], w.gates2[perm], w.expert_rank2, w.G,
                               w.ranks_per_node, src_offsets=sh["shard_offsets"])
    _check_plan(step.plan, ref, w.T, w.k)
