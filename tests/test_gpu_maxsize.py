"""Sizes far beyond the benchmark's, too large for the oracle's loops, so
checked against properties that fix the results at any size.

The plan at 2^25 tokens with k = 8 on 64 ranks (2^28 slots, up to 2^28 rows):
the counters and the per-(source, destination) counts from the tokens'
destination masks; every token's rows in the segments of its source rank and
its destination ranks, ascending; the tokens of each segment ascending; every
slot's row; the row weights against the definition on a sample of tokens.

Permute and combine with row indices past 2^31 16-byte vectors (a 40 GiB
send buffer): combine(permute(x)) = x exactly when each token's gates sum to
one, and sampled send rows equal their tokens' rows; then the one-pass
shuffle dispatch into the same buffer under a random order."""

import numpy as np
import pytest
import torch

from co_activation_amd import ops
from gpu_util import host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def test_plan_at_2_pow_28_slots():
    T, k, E, G, rn = 1 << 25, 8, 256, 64, 8
    rng = np.random.default_rng(7)
    # k distinct experts per token: base + j * step (mod E) with an odd step
    base = rng.integers(0, E, size=T, dtype=np.int32)
    step = (2 * rng.integers(0, E // 2, size=T, dtype=np.int32) + 1).astype(np.int32)
    j = np.arange(k, dtype=np.int32)
    topk = (base[:, None] + step[:, None] * j[None, :]) % E
    del base, step
    er = (rng.permutation(E) % G).astype(np.int32)
    gates = rng.random((T, k), dtype=np.float32)
    say("plan at 2^28 slots", T, k, G)

    err = ops.new_error_word()
    plan = ops.dispatch_plan(torch.from_numpy(topk).cuda(), torch.from_numpy(gates).cuda(),
                             torch.from_numpy(er).cuda(), G, rn, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))

    # destination masks, sources, counts
    ranks = er[topk]
    del topk
    mask = np.zeros(T, np.uint64)
    for jj in range(k):
        mask |= np.left_shift(np.uint64(1), ranks[:, jj].astype(np.uint64))
    cnt = np.bitwise_count(mask).astype(np.int64)
    N = int(cnt.sum())
    src = np.arange(T, dtype=np.int64) // (T // G)
    bits = np.unpackbits(mask.view(np.uint8).reshape(T, 8), axis=1, bitorder="little")
    S = bits.reshape(G, T // G, 64).sum(axis=1, dtype=np.int64)
    recv_max = int(bits.sum(axis=0, dtype=np.int64).max())
    local_rows = int(bits[np.arange(T), src].sum(dtype=np.int64))
    del bits
    nodes = np.zeros(T, np.uint64)
    for jj in range(k):
        nodes |= np.left_shift(np.uint64(1), (ranks[:, jj] // rn).astype(np.uint64))
    node_rows = int(np.bitwise_count(nodes).sum(dtype=np.int64))
    own = np.left_shift(np.uint64(1), (src // rn).astype(np.uint64))
    V = int(np.bitwise_count(nodes & ~own).sum(dtype=np.int64))
    del nodes, own
    local_assign = int((ranks == src[:, None]).sum(dtype=np.int64))
    want_counters = np.array([N, T * k, local_rows, local_assign, node_rows, V, recv_max, 0],
                             np.int64)
    np.testing.assert_array_equal(host(plan.counters), want_counters, "counters")
    np.testing.assert_array_equal(host(plan.send_counts), S, "send_counts")
    offsets = np.concatenate([[0], np.cumsum(S.ravel())])
    np.testing.assert_array_equal(host(plan.send_offsets), offsets, "send_offsets")

    # every token's rows: a prefix of its k slots, in the segments (s_t, r)
    # of its destination ranks r in ascending order, each row naming it
    tr = host(plan.token_rows)
    valid = tr >= 0
    assert (valid[:, :-1] >= valid[:, 1:]).all(), "rows not a prefix of the slots"
    np.testing.assert_array_equal(valid.sum(axis=1), cnt, "rows per token")
    rows = tr[valid].astype(np.int64)
    del tr, valid
    rt = host(plan.row_token)[:N]
    np.testing.assert_array_equal(rt[rows], np.repeat(np.arange(T, dtype=np.int32), cnt),
                                  "row_token of each token's rows")
    sr = np.sort(ranks, axis=1)
    first = np.ones_like(sr, dtype=bool)
    first[:, 1:] = sr[:, 1:] != sr[:, :-1]
    want_seg = np.repeat(src, cnt) * G + sr[first]
    got_seg = np.searchsorted(offsets, rows, side="right") - 1
    np.testing.assert_array_equal(got_seg, want_seg, "segment of each row")
    del sr, first, want_seg, got_seg, rows
    # tokens ascending inside each segment
    seg_of_row = np.repeat(np.arange(G * G), S.ravel())
    same = seg_of_row[1:] == seg_of_row[:-1]
    assert (np.diff(rt.astype(np.int64))[same] > 0).all(), "tokens out of order in a segment"
    del seg_of_row, same

    # every slot's row: in segment (s_t, rank of the slot), naming the token
    sl = host(plan.slot_row).astype(np.int64)
    np.testing.assert_array_equal(rt[sl], np.broadcast_to(np.arange(T, dtype=np.int32)[:, None],
                                                          (T, k)), "row_token of slot rows")
    got = np.searchsorted(offsets, sl.ravel(), side="right") - 1
    np.testing.assert_array_equal(got, (src[:, None] * G + ranks).ravel(), "segment of slot rows")
    del got

    # row weights on a sample of tokens: the gates of the token's slots on
    # that rank, summed in fp32 in slot order
    rw = host(plan.row_weight)[:N]
    for t in rng.choice(T, size=2048, replace=False):
        for jj in range(k):
            acc = np.float32(0)
            for i in range(k):
                if ranks[t, i] == ranks[t, jj]:
                    acc = np.float32(acc + gates[t, i])
            assert rw[sl[t, jj]].view(np.uint32) == acc.view(np.uint32), (t, jj)


def test_rows_beyond_2_pow_31_vectors():
    """Permute then combine with row indices past 2^31 16-byte vectors
    (2.6 M tokens of 8 KiB bf16 rows, a 40 GiB send buffer): every address
    is formed in 64 bits.  With each token's gates summing to 1 the combine
    of the permuted rows returns x exactly (fp32 error far below half a bf16
    ulp), checked on every token; send rows are checked against their tokens'
    rows on the last 4096 rows and 4096 random ones."""
    from workloads.gen import device_normal

    T, H, E, k, G, rn = (1 << 21) + (1 << 19), 4096, 64, 2, 8, 8
    rng = np.random.default_rng(11)
    base = rng.integers(0, E, size=T, dtype=np.int32)
    step = 2 * rng.integers(0, E // 2, size=T, dtype=np.int32) + 1
    topk = np.stack([base, (base + step) % E], axis=1).astype(np.int32)
    er = (np.arange(E) // (E // G)).astype(np.int32)
    g = rng.random((T, k), dtype=np.float32) + np.float32(0.1)
    gates = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    cap = T * min(k, G)
    say("rows beyond 2^31 vectors", T, H, cap)
    x = device_normal(T, H, "bf16", seed=3)
    err = ops.new_error_word()
    plan = ops.dispatch_plan(torch.from_numpy(topk).cuda(), torch.from_numpy(gates).cuda(),
                             torch.from_numpy(er).cuda(), G, rn, d_err=err)
    N = int(plan.counters[0].item())
    assert N * (H // 8) > (1 << 31) + (1 << 28), "the largest rows must lie past 2^31 vectors"
    send = ops.permute(x, plan.token_rows, cap, d_err=err)
    y = ops.combine(send, plan.token_rows, plan.row_weight, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))
    assert torch.equal(y.view(torch.int16), x.view(torch.int16)), "combine(permute(x)) != x"
    del y
    idx = torch.cat([torch.arange(N - 4096, N, device="cuda"),
                     torch.randint(0, N, (4096,), device="cuda")])
    tok = plan.row_token[:N].long()[idx]
    assert torch.equal(send[idx].view(torch.int16), x[tok].view(torch.int16)), "send rows"
    # the one-pass shuffle dispatch at the same size, into the same buffer:
    # x_s[p] = x[perm[p]] everywhere, send[token_rows[p, q]] = x[perm[p]] sampled
    perm = torch.randperm(T, device="cuda", dtype=torch.int64)
    x_s, send = ops.shuffle_dispatch(x, perm.int(), plan.token_rows, cap, send=send, d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, ops.decode_errors(int(err.item()))
    assert torch.equal(x_s.view(torch.int16), x[perm].view(torch.int16)), "shuffled rows"
    del x_s
    pos = torch.cat([torch.arange(T - 2048, T, device="cuda"),
                     torch.randint(0, T, (2048,), device="cuda")])
    tr = plan.token_rows.long()[pos]
    for q in range(k):
        ok = tr[:, q] >= 0
        assert torch.equal(send[tr[ok, q]].view(torch.int16),
                           x[perm[pos[ok]]].view(torch.int16)), f"shuffle-dispatched rows, slot {q}"
