"""Pins for the CPU oracle: values and identities fixed by the pages and by
the mathematics, computed here without calling back into the oracle's own
formulas.  Each test names what it pins and what mistake it would catch."""

import itertools
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from workloads import make
from workloads.gen import uniform_contiguous

GOLDEN = Path(__file__).parent / "golden"


def _golden_placement():
    er = np.full(64, -1, dtype=np.int64)
    for line in (GOLDEN / "uniform_placement_64x8.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        d, a, b = (int(v) for v in line.split())
        er[a:b + 1] = d
    assert (er >= 0).all()
    return er


def _random_routing(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def _random_gates(rng, T, k):
    w = rng.random((T, k)) + 0.05
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


# ------------------------------------------------------------ placement

def test_golden_uniform_placement_matches_generator():
    """Printed 64-on-8 mapping (Expert Placement Strategies) equals the
    contiguous split the workloads use."""
    assert (uniform_contiguous(64, 8) == _golden_placement()).all()


def test_plan_rows_follow_printed_devices():
    """With the printed mapping, a token's rows are one per distinct device
    range in the printed table (looked up in the table, not computed)."""
    er = _golden_placement()
    rng = np.random.default_rng(3)
    topk = _random_routing(rng, 256, 64, 4)
    plan = oracle.dispatch_plan(topk, None, er, 8, 8)
    ranges = []
    for line in (GOLDEN / "uniform_placement_64x8.txt").read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            ranges.append(tuple(int(v) for v in line.split()))
    expect = 0
    for t in range(256):
        devs = {d for e in topk[t] for (d, a, b) in ranges if a <= e <= b}
        expect += len(devs)
    assert plan["N"] == expect


# ------------------------------------------------------------ statistics

def test_stats_bruteforce_token_sets():
    """n, C, Ochiai and transitions from explicit token sets (set algebra)."""
    rng = np.random.default_rng(0)
    for trial in range(20):
        T = int(rng.integers(1, 12))
        E = int(rng.integers(2, 7))
        k = int(rng.integers(1, E + 1))
        E2 = int(rng.integers(2, 7))
        k2 = int(rng.integers(1, E2 + 1))
        topk = _random_routing(rng, T, E, k)
        topk2 = _random_routing(rng, T, E2, k2)
        st = oracle.coact_stats(topk, E, topk2, E2)
        A = [{t for t in range(T) if e in set(topk[t].tolist())} for e in range(E)]
        B = [{t for t in range(T) if e in set(topk2[t].tolist())} for e in range(E2)]
        for i in range(E):
            assert st["expert_count"][i] == len(A[i])
            for j in range(E):
                inter = len(A[i] & A[j])
                assert st["pair_count"][i, j] == inter
                if A[i] and A[j]:
                    want = np.float32(inter / math.sqrt(len(A[i]) * len(A[j])))
                    assert st["ochiai"][i, j] == want
                else:
                    assert st["ochiai"][i, j] == 0.0
            for j in range(E2):
                assert st["transition"][i, j] == len(A[i] & B[j])


def test_stats_hand_example():
    """Four tokens {0,1},{0,1},{0,2},{1,2}: n = 3,3,2; both 0 and 1 are picked
    by tokens 0 and 1, so Ochiai(0,1) = 2/3; Ochiai(0,2) = 1/sqrt(6)."""
    topk = np.array([[0, 1], [1, 0], [0, 2], [2, 1]], dtype=np.int32)
    st = oracle.coact_stats(topk, 3)
    assert st["expert_count"].tolist() == [3, 3, 2]
    assert st["pair_count"].tolist() == [[3, 2, 1], [2, 3, 1], [1, 1, 2]]
    assert st["ochiai"][0, 1] == np.float32(2.0 / 3.0)
    assert st["ochiai"][0, 2] == np.float32(1.0 / math.sqrt(6.0))
    assert st["ochiai"][2, 2] == 1.0


def test_stats_transition_direction():
    """Rows index this layer, columns the next: a token going 0 -> 2 counts
    at [0][2] only (catches a transposed operand)."""
    st = oracle.coact_stats(np.array([[0]], np.int32), 3, np.array([[2]], np.int32), 3)
    X = st["transition"]
    assert X[0, 2] == 1 and X[2, 0] == 0 and X.sum() == 1


def test_stats_invariants_workload3():
    w = make(3, T=1500, with_x=False)
    st = oracle.coact_stats(w.topk, w.E)
    n, C = st["expert_count"], st["pair_count"]
    T, k = w.topk.shape
    assert n.sum() == T * k
    assert (C == C.T).all()
    assert (np.diag(C) == n).all()
    assert (C.sum(axis=1) == k * n).all()
    assert C.sum() == T * k * k


def test_stats_same_layer_transition_equals_pairs():
    """If the next layer routes exactly like this one, X = C; row sums of X
    are k' * n_i."""
    w = make(5, T=800, with_x=False)
    st = oracle.coact_stats(w.topk, w.E, w.topk, w.E)
    assert (st["transition"] == st["pair_count"]).all()
    st2 = oracle.coact_stats(w.topk, w.E, w.topk2, w.E)
    assert (st2["transition"].sum(axis=1) == w.topk2.shape[1] * st2["expert_count"]).all()


def test_ochiai_identical_and_disjoint_sets():
    """Experts always picked together -> 1; never together -> 0; never
    picked -> 0 (the 0/0 reading)."""
    topk = np.array([[0, 1], [0, 1], [2, 3], [2, 3], [0, 1]], dtype=np.int32)
    O = oracle.coact_stats(topk, 5)["ochiai"]
    assert O[0, 1] == 1.0 and O[2, 3] == 1.0
    assert O[0, 2] == 0.0 and O[1, 3] == 0.0
    assert (O[4] == 0).all() and (O[:, 4] == 0).all()


# ------------------------------------------------------------ dispatch plan

def _bruteforce_plan(topk, gates, er, G, Rn, off):
    """Row index of (t, r) = number of (s', r', t') strictly before
    (s_t, r, t) in lexicographic order among all dispatched pairs."""
    T, k = topk.shape
    src = [next(s for s in range(G) if off[s] <= t < off[s + 1]) for t in range(T)]
    pairs = [(src[t], int(er[e]), t) for t in range(T) for e in topk[t]]
    pairs = sorted(set(pairs))
    row_of = {}
    for (s, r, t) in pairs:
        row_of[(t, r)] = sum(1 for q in pairs if q < (s, r, t))
    N = len(pairs)
    S = np.zeros((G, G), np.int64)
    for (s, r, t) in pairs:
        S[s, r] += 1
    row_token = [None] * N
    for (s, r, t) in pairs:
        row_token[row_of[(t, r)]] = t
    V = 0
    for t in range(T):
        nodes = {int(er[e]) // Rn for e in topk[t]}
        nodes.discard(src[t] // Rn)
        V += len(nodes)
    local_rows = sum(1 for (s, r, t) in pairs if s == r)
    local_assign = sum(1 for t in range(T) for e in topk[t] if int(er[e]) == src[t])
    node_rows = sum(len({int(er[e]) // Rn for e in topk[t]}) for t in range(T))
    wsum = {}
    for t in range(T):
        for j in range(k):
            key = (t, int(er[topk[t, j]]))
            wsum[key] = np.float32(wsum.get(key, np.float32(0)) + gates[t, j])
    return dict(N=N, S=S, row_token=row_token, row_of=row_of, V=V, local_rows=local_rows,
                local_assign=local_assign, node_rows=node_rows, wsum=wsum,
                max_recv=int(S.sum(axis=0).max()))


def _check_plan(plan, bf, topk, er, T, k):
    assert plan["N"] == bf["N"]
    assert (plan["send_counts"] == bf["S"]).all()
    assert plan["send_offsets"][-1] == bf["N"]
    assert plan["row_token"].tolist() == bf["row_token"]
    c = plan["counters"]
    assert c[0] == bf["N"] and c[1] == T * k
    assert c[2] == bf["local_rows"] and c[3] == bf["local_assign"]
    assert c[4] == bf["node_rows"] and c[5] == bf["V"] and c[6] == bf["max_recv"] and c[7] == 0
    for t in range(T):
        ranks = sorted({int(er[e]) for e in topk[t]})
        want = [bf["row_of"][(t, r)] for r in ranks] + [-1] * (k - len(ranks))
        assert plan["token_rows"][t].tolist() == want
        for j in range(k):
            assert plan["slot_row"][t, j] == bf["row_of"][(t, int(er[topk[t, j]]))]
    for (t, r), i in bf["row_of"].items():
        assert plan["row_weight"][i] == bf["wsum"][(t, r)]


def test_plan_exhaustive_tiny():
    """Every routing of 2 tokens over 3 experts (k=2) under every placement
    on G = 1..3 ranks, ranks_per_node in {1, G}."""
    rng = np.random.default_rng(1)
    E, k, T = 3, 2, 2
    rows = [list(p) for p in itertools.permutations(range(E), k)]
    for G in (1, 2, 3):
        for er in itertools.product(range(G), repeat=E):
            er = np.array(er, np.int32)
            for r0, r1 in itertools.product(rows, rows):
                topk = np.array([r0, r1], np.int32)
                gates = _random_gates(rng, T, k)
                for Rn in sorted({1, G}):
                    off = [s * T // G if G <= T else min(s, T) for s in range(G + 1)]
                    off[-1] = T
                    plan = oracle.dispatch_plan(topk, gates, er, G, Rn, src_offsets=off)
                    bf = _bruteforce_plan(topk, gates, er, G, Rn, off)
                    _check_plan(plan, bf, topk, er, T, k)


def test_plan_random_small_vs_bruteforce():
    rng = np.random.default_rng(2)
    for trial in range(150):
        T = int(rng.integers(1, 9))
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, min(E, 4) + 1))
        G = int(rng.integers(1, 6))
        Rn = int(rng.choice([d for d in range(1, G + 1) if G % d == 0]))
        topk = _random_routing(rng, T, E, k)
        gates = _random_gates(rng, T, k)
        er = rng.integers(0, G, size=E).astype(np.int32)
        cuts = np.sort(rng.integers(0, T + 1, size=G - 1))
        off = [0] + cuts.tolist() + [T]
        plan = oracle.dispatch_plan(topk, gates, er, G, Rn, src_offsets=off)
        bf = _bruteforce_plan(topk, gates, er, G, Rn, off)
        _check_plan(plan, bf, topk, er, T, k)


def test_plan_dedup_identity_and_bounds():
    """N = sum_t |R_t| = sum S (each token to each rank once); T <= N <=
    T*min(k, G); every (t, r in R_t) appears once; rows ascend in t inside
    each (s, r) block."""
    w = make(3, T=2048, with_x=False)
    plan = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    R = [set(w.expert_rank[row].tolist()) for row in w.topk]
    N = sum(len(r) for r in R)
    assert plan["N"] == N == plan["send_counts"].sum() == plan["send_offsets"][-1]
    assert w.T <= N <= w.T * min(w.k, w.G)
    seen = set()
    off = plan["send_offsets"]
    for q in range(w.G * w.G):
        blk = plan["row_token"][off[q]:off[q + 1]]
        assert (np.diff(blk) > 0).all()
        s, r = divmod(q, w.G)
        for t in blk:
            assert (int(t), r) not in seen and r in R[int(t)]
            assert s == int(t) // (w.T // w.G)
            seen.add((int(t), r))
    assert len(seen) == N


def test_plan_special_cases():
    rng = np.random.default_rng(4)
    T, k = 96, 3
    # one expert per rank: nothing to dedup -> N = T*k
    topk = _random_routing(rng, T, 8, k)
    p = oracle.dispatch_plan(topk, None, np.arange(8), 8, 4)
    assert p["N"] == T * k
    # a single rank: one row per token
    p = oracle.dispatch_plan(topk, None, np.zeros(8, np.int32), 1, 1)
    assert p["N"] == T and p["counters"][2] == T and p["counters"][5] == 0
    # one rank per node: every non-local row crosses nodes
    er = rng.integers(0, 4, size=8).astype(np.int32)
    p = oracle.dispatch_plan(topk, None, er, 4, 1)
    assert p["counters"][5] == p["N"] - p["counters"][2]
    # a single node: nothing crosses nodes
    p = oracle.dispatch_plan(topk, None, er, 4, 4)
    assert p["counters"][5] == 0 and p["counters"][4] == T


def test_plan_uniform_local_share_one_over_G():
    """Position-independent routing over equal contiguous shards keeps 1/G of
    the assignments on the token's own rank (12.5% at G = 8)."""
    rng = np.random.default_rng(5)
    T, E, k, G = 16384, 64, 2, 8
    topk = _random_routing(rng, T, E, k)
    p = oracle.dispatch_plan(topk, None, uniform_contiguous(E, G), G, G)
    share = p["counters"][3] / (T * k)
    assert abs(share - 1.0 / G) < 0.006


def test_plan_rejects_bad_inputs():
    with pytest.raises(oracle.OracleInputError):
        oracle.dispatch_plan(np.array([[0, 0]], np.int32), None, np.zeros(2, np.int32), 1, 1)
    with pytest.raises(oracle.OracleInputError):
        oracle.dispatch_plan(np.array([[0, 5]], np.int32), None, np.zeros(2, np.int32), 1, 1)
    with pytest.raises(oracle.OracleInputError):
        oracle.dispatch_plan(np.array([[0, 1]], np.int32), None, np.array([0, 3], np.int32), 2, 2,
                             src_offsets=[0, 1, 1])
    with pytest.raises(oracle.OracleInputError):
        oracle.dispatch_plan(np.array([[0, 1]], np.int32), None, np.array([0, 1], np.int32), 2, 2,
                             src_offsets=[0, 2, 1])


# ------------------------------------------------------------ permute

def test_permute_matches_per_block_construction():
    """Send buffer built block by block: for s, for r, the x rows of shard s
    that have an expert on r, ascending t."""
    w = make(2, T=512, H=64)
    plan = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    send = oracle.permute_rows(w.x, plan["row_token"])
    sh = w.T // w.G
    want = []
    for s in range(w.G):
        for r in range(w.G):
            for t in range(s * sh, (s + 1) * sh):
                if r in set(w.expert_rank[w.topk[t]].tolist()):
                    want.append(w.x[t])
    assert np.array_equal(send, np.stack(want))


def test_scatter_roundtrip():
    rng = np.random.default_rng(6)
    x = rng.integers(0, 2**16, size=(50, 8), dtype=np.uint16)
    dest = rng.permutation(50)
    out = oracle.scatter_rows(x, dest, 50)
    assert np.array_equal(out[dest], x)
    inv = np.argsort(dest)
    assert np.array_equal(out, x[inv])


# ------------------------------------------------------------ combine

def test_bf16_round_against_torch_and_edges():
    rng = np.random.default_rng(7)
    with np.errstate(over="ignore"):  # the near-overflow draws may round to infinity
        vals = np.concatenate([
            rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
            (rng.standard_normal(2000) * 1.5e38).astype(np.float32),    # near overflow
            np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                      1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, 2**-133, 2**-134,
                      3 * 2**-134], np.float32),
        ])
    got = oracle.bf16_round(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # ties go to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert oracle.bf16_round(np.array([1.0 + 2**-8], np.float32))[0] == 0x3F80
    assert oracle.bf16_round(np.array([1.0 + 3 * 2**-8], np.float32))[0] == 0x3F82
    nan = oracle.bf16_round(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_combine_hand_example():
    Z = np.array([[1.0, 2.0], [3.0, 4.0]], np.float32)
    y = oracle.combine(Z, "f32", np.array([[0, 1]]), np.array([[0.25, 0.75]], np.float32), "f32")
    assert y.tolist() == [[2.5, 3.5]]


def test_combine_of_permute_identities():
    """Unweighted combine of permute(x) is |R_t| * x exactly; weighted combine
    with gates summing to 1 returns x bit-exact in bf16 (routing and values
    are unchanged by the dispatch)."""
    w = make(3, T=640, H=32)
    plan = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    send = oracle.permute_rows(w.x, plan["row_token"])
    nr = (plan["token_rows"] >= 0).sum(axis=1)
    y = oracle.combine_unweighted(send, "bf16", plan["token_rows"], "f32")
    assert np.array_equal(y, oracle.bf16_to_f32(w.x) * nr[:, None].astype(np.float32))
    yb = oracle.combine(send, "bf16", plan["slot_row"], w.gates, "bf16")
    assert np.array_equal(yb, w.x)


def test_combine_dedup_equals_expanded_path():
    """Combine over the deduplicated rows with per-rank gate mass equals the
    expanded path with one row per (token, slot)."""
    w = make(4, T=320, H=16)
    plan = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    rng = np.random.default_rng(8)
    Z = rng.standard_normal((plan["N"], 16)).astype(np.float32)
    y = oracle.combine(Z, "f32", plan["slot_row"], w.gates, "f32")
    # dedup form, accumulated here in float64 from token_rows and row_weight
    yd = np.zeros_like(y, dtype=np.float64)
    for t in range(w.T):
        for q in range(w.k):
            i = plan["token_rows"][t, q]
            if i >= 0:
                yd[t] += float(plan["row_weight"][i]) * Z[i].astype(np.float64)
    scale = np.zeros_like(yd)
    for t in range(w.T):
        for j in range(w.k):
            scale[t] += abs(float(w.gates[t, j])) * np.abs(Z[plan["slot_row"][t, j]])
    assert (np.abs(y - yd) <= 1e-6 * scale + 1e-30).all()


# ------------------------------------------------------------ shuffle

def test_shuffle_bruteforce_small():
    rng = np.random.default_rng(9)
    for trial in range(60):
        T = int(rng.integers(1, 30))
        E = int(rng.integers(2, 7))
        E2 = int(rng.integers(2, 7))
        k = int(rng.integers(1, E + 1))
        G = int(rng.integers(1, 5))
        topk = _random_routing(rng, T, E, k)
        X = rng.integers(0, 4, size=(E, E2))
        er2 = rng.integers(0, G, size=E2).astype(np.int32)
        sh = oracle.shuffle_predict(topk, X, er2, G)
        for t in range(T):
            scores = [sum(int(X[i, j]) for i in topk[t] for j in range(E2) if er2[j] == r)
                      for r in range(G)]
            best = max(scores)
            assert sh["pred_rank"][t] == scores.index(best)
        order = sorted(range(T), key=lambda t: (int(sh["pred_rank"][t]), t))
        assert sh["perm"].tolist() == order
        for q, t in enumerate(order):
            assert sh["dest_pos"][t] == q
        cnt = np.bincount(sh["pred_rank"], minlength=G)
        assert sh["shard_offsets"].tolist() == [0] + np.cumsum(cnt).tolist()


def test_shuffle_ties_and_zero_scores_go_low():
    X = np.zeros((2, 4), np.int64)
    sh = oracle.shuffle_predict(np.array([[0], [1]], np.int32), X, np.array([0, 1, 2, 3]), 4)
    assert sh["pred_rank"].tolist() == [0, 0]
    X = np.array([[0, 5, 5, 0], [1, 0, 0, 0]])
    sh = oracle.shuffle_predict(np.array([[0], [1]], np.int32), X, np.array([3, 2, 1, 0]), 4)
    assert sh["pred_rank"].tolist() == [1, 3]


def test_two_layer_shuffle_raises_local_share():
    """Token shuffling raises the share of next-layer assignments on the
    token's own rank above the 1/G baseline; routing is only moved, never
    changed."""
    w = make(5, T=4096, H=16)
    res = oracle.two_layer_pipeline(w.topk, w.topk2, w.gates2, w.x, w.expert_rank2, w.E, w.E,
                                    w.G, w.ranks_per_node)
    assert abs(res["local_share_before"] - 0.125) < 0.02
    assert res["local_share_after"] > res["local_share_before"] + 0.05
    perm = res["shuffle"]["perm"]
    assert np.array_equal(res["topk2_shuffled"], w.topk2[perm])
    assert np.array_equal(res["x_shuffled"], w.x[perm])
    assert sorted(perm.tolist()) == list(range(w.T))


def test_shuffle_dispatch_is_move_then_permute():
    """One pass (each shuffled position takes its token's row and writes it
    to the next layer's send rows) equals the two steps it replaces: the
    shuffle's move, then the permute of the shuffled rows by the plan."""
    w = make(5, T=1032, H=16)
    res = oracle.two_layer_pipeline(w.topk, w.topk2, w.gates2, w.x, w.expert_rank2, w.E, w.E,
                                    w.G, w.ranks_per_node)
    plan = res["plan"]
    N = int(plan["N"])
    x_s, send = oracle.shuffle_dispatch(w.x, res["shuffle"]["perm"], plan["token_rows"], N)
    assert np.array_equal(x_s, res["x_shuffled"])
    assert np.array_equal(send, res["send"])
    # a hand case: 3 tokens, shuffled order (2, 0, 1), rows by shuffled position
    x = np.array([[1], [2], [3]], np.int32)
    perm = np.array([2, 0, 1])
    token_rows = np.array([[0, 3], [1, -1], [2, 4]])
    xs, sd = oracle.shuffle_dispatch(x, perm, token_rows, 5)
    assert xs[:, 0].tolist() == [3, 1, 2]
    assert sd[:, 0].tolist() == [3, 1, 2, 3, 2]


# ------------------------------------------------------------ expert side

def test_expert_plan_hand_example():
    """p = [0, 0, 1, 1]; token 0 picks experts 1, 2 and token 1 picks 0, 1.
    Rows in (rank, expert, token) order: (e0,t1) (e1,t0) (e1,t1) (e2,t0)."""
    topk = np.array([[1, 2], [0, 1]], np.int32)
    gates = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    er = np.array([0, 0, 1, 1], np.int32)
    plan = oracle.dispatch_plan(topk, gates, er, 2, 2)
    ep = oracle.expert_plan(topk, gates, er, 2, plan["slot_row"], plan["N"])
    assert ep["erow"].tolist() == [[1, 3], [0, 2]]
    assert ep["expert_count"].tolist() == [1, 2, 1, 0]
    assert ep["expert_first"].tolist() == [0, 1, 3, 4]
    assert ep["rank_offsets"].tolist() == [0, 3, 4]
    assert ep["erow_slot"].tolist() == [2, 0, 3, 1]
    assert ep["erow_weight"].tolist() == [0.5, 0.75, 0.5, 0.25]
    # send rows (s, r, t): (0,0,0) (0,1,0) (1,0,1); token 1 has both experts on rank 0
    assert plan["row_token"].tolist() == [0, 0, 1]
    assert ep["erow_src"].tolist() == [2, 0, 2, 1]


def test_expert_plan_bruteforce_and_counts():
    """erow(t, j) = number of slots whose (rank, expert, token) key is
    smaller, counted directly; per-expert counts match the statistics."""
    rng = np.random.default_rng(20)
    for trial in range(40):
        T = int(rng.integers(1, 30))
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        G = int(rng.integers(1, 5))
        topk = _random_routing(rng, T, E, k)
        gates = _random_gates(rng, T, k)
        er = rng.integers(0, G, size=E).astype(np.int32)
        plan = oracle.dispatch_plan(topk, gates, er, G, 1, src_offsets=[0] * G + [T])
        ep = oracle.expert_plan(topk, gates, er, G, plan["slot_row"], plan["N"])
        keys = [(int(er[topk[t, j]]), int(topk[t, j]), t) for t in range(T) for j in range(k)]
        for t in range(T):
            for j in range(k):
                me = (int(er[topk[t, j]]), int(topk[t, j]), t)
                assert ep["erow"][t, j] == sum(1 for q in keys if q < me)
        st = oracle.coact_stats(topk, E)
        assert (ep["expert_count"] == st["expert_count"]).all()
        for r in range(G):
            assert ep["rank_offsets"][r + 1] - ep["rank_offsets"][r] == \
                sum(int(st["expert_count"][e]) for e in range(E) if er[e] == r)
        # each send row lists exactly the expert rows of its token's slots on its rank,
        # and each expert row names that send row as its source
        for t in range(T):
            for j in range(k):
                i = plan["slot_row"][t, j]
                on_r = [ep["erow"][t, jj] for jj in range(k) if plan["slot_row"][t, jj] == i]
                assert ep["row_dest"][i].tolist() == on_r + [-1] * (k - len(on_r))
                assert ep["erow_src"][ep["erow"][t, j]] == i
                assert plan["row_token"][i] == t


def test_expert_side_reproduces_moe_output():
    """Dispatch, expansion, experts that scale their rows, partial combine
    (rounded to bf16 as a reply row) and the unweighted combine give the
    plain MoE output sum_j w_tj c_e x_t within the two bf16 roundings."""
    w = make(3, T=640, H=32)
    rng = np.random.default_rng(21)
    c = rng.uniform(0.5, 2.0, size=w.E)
    plan = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    N = plan["N"]
    ep = oracle.expert_plan(w.topk, w.gates, w.expert_rank, w.G, plan["slot_row"], N)
    send = oracle.permute_rows(w.x, plan["row_token"])
    # expansion: expert row i is a copy of the send row its slot points to
    erows = np.zeros((w.T * w.k, w.H), np.uint16)
    for i in range(N):
        for q in range(w.k):
            if ep["row_dest"][i, q] >= 0:
                erows[ep["row_dest"][i, q]] = send[i]
    tok = ep["erow_slot"] // w.k
    assert np.array_equal(erows, w.x[tok])
    # the same expansion as a gather by source row
    assert np.array_equal(oracle.permute_rows(send, ep["erow_src"]), erows)
    # experts: scale each row by its expert's constant (float32, rounded to bf16)
    e_of_row = w.topk.reshape(-1)[ep["erow_slot"]]
    Y = oracle.bf16_round((oracle.bf16_to_f32(erows) * c[e_of_row][:, None]).astype(np.float32))
    Z = oracle.partial_combine(Y, "bf16", ep["erow"], w.gates, plan["slot_row"], N, "bf16")
    y = oracle.combine_unweighted(Z, "bf16", plan["token_rows"], "f32")
    ref = oracle.moe_output(w.x, "bf16", w.topk, w.gates, c)
    scale = np.zeros_like(ref)
    xf = oracle.bf16_to_f32(w.x).astype(np.float64)
    for j in range(w.k):
        scale += np.abs(w.gates[:, j:j + 1]) * c[w.topk[:, j]][:, None] * np.abs(xf)
    assert (np.abs(y - ref) <= 2.0 ** -7 * scale + 1e-30).all()


def test_moe_output_special_cases():
    """Unit experts with gates summing to 1 return x; one slot returns w*c*x."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((50, 8)).astype(np.float32)
    topk = _random_routing(rng, 50, 6, 3)
    gates = _random_gates(rng, 50, 3)
    y = oracle.moe_output(x, "f32", topk, gates, np.ones(6))
    assert np.allclose(y, x, rtol=1e-6, atol=1e-7)
    y1 = oracle.moe_output(x, "f32", topk[:, :1], gates[:, :1], np.full(6, 3.0))
    assert np.allclose(y1, 3.0 * gates[:, :1].astype(np.float64) * x, rtol=1e-12)


# ------------------------------------------------------------ backward

def _f64(x, dt):
    return oracle.bf16_to_f32(x).astype(np.float64) if dt == "bf16" else x.astype(np.float64)


def test_backward_adjoint_identities():
    """<dY, combine(Z)> = <permute_scaled(dY), Z> (the scaled scatter is the
    adjoint of the weighted combine in its rows) and
    <dS, permute(x)> = <combine_unweighted(dS), x> (the plain combine is the
    adjoint of the permute), both in float64 on fp32 data."""
    w = make(4, T=320, H=24)
    rng = np.random.default_rng(40)
    plan = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    N = plan["N"]
    Z = rng.standard_normal((N, w.H)).astype(np.float32)
    dY = rng.standard_normal((w.T, w.H)).astype(np.float32)
    # forward combine in float64 from the rows' gate mass
    y = np.zeros((w.T, w.H))
    for t in range(w.T):
        for q in range(w.k):
            i = plan["token_rows"][t, q]
            if i >= 0:
                y[t] += float(plan["row_weight"][i]) * Z[i].astype(np.float64)
    dZ = oracle.permute_scaled(dY, "f32", plan["token_rows"], plan["row_weight"], N, "f32")
    lhs = float(np.sum(dY.astype(np.float64) * y))
    rhs = float(np.sum(dZ.astype(np.float64) * Z.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-6 * float(np.sum(np.abs(dY.astype(np.float64) * y))) + 1e-9
    x = rng.standard_normal((w.T, w.H)).astype(np.float32)
    dS = rng.standard_normal((N, w.H)).astype(np.float32)
    send = oracle.permute_rows(x, plan["row_token"])
    dx = oracle.combine_unweighted(dS, "f32", plan["token_rows"], "f32")
    lhs = float(np.sum(dS.astype(np.float64) * send.astype(np.float64)))
    rhs = float(np.sum(dx.astype(np.float64) * x.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-6 * float(np.sum(np.abs(dS.astype(np.float64) * send))) + 1e-9


def test_gate_gradient_matches_finite_differences():
    """dL/dw_tj for L = <dY, y(w)>, y_t = sum_j w_tj Z[slot_row(t, j)], equals
    row_dot(dY, Z, slot_row); y is linear in w, so a central difference in
    float64 is exact up to rounding."""
    w = make(3, T=96, H=16)
    rng = np.random.default_rng(41)
    plan = oracle.dispatch_plan(w.topk, w.gates, w.expert_rank, w.G, w.ranks_per_node)
    Z = rng.standard_normal((plan["N"], w.H)).astype(np.float32)
    dY = rng.standard_normal((w.T, w.H)).astype(np.float32)
    dw = oracle.row_dot(dY, "f32", Z, "f32", plan["slot_row"])

    def loss(g):
        y = np.zeros((w.T, w.H))
        for t in range(w.T):
            for j in range(w.k):
                y[t] += g[t, j] * Z[plan["slot_row"][t, j]].astype(np.float64)
        return float(np.sum(dY.astype(np.float64) * y))

    g0 = w.gates.astype(np.float64)
    for (t, j) in [(0, 0), (5, 3), (95, 5), (40, 1)]:
        gp, gm = g0.copy(), g0.copy()
        gp[t, j] += 0.5
        gm[t, j] -= 0.5
        fd = loss(gp) - loss(gm)
        assert abs(fd - float(dw[t, j])) <= 1e-5 * (abs(fd) + 1.0)


def test_permute_scaled_and_row_dot_small():
    x = np.array([[1.0, -2.0], [3.0, 0.5]], np.float32)
    dest = np.array([[1, -1], [0, 2]])
    scale = np.array([0.5, 2.0, -1.0], np.float32)
    out = oracle.permute_scaled(x, "f32", dest, scale, 4, "f32")
    assert out.tolist() == [[1.5, 0.25], [2.0, -4.0], [-3.0, -0.5], [0.0, 0.0]]
    d = oracle.row_dot(x, "f32", out, "f32", np.array([[1, 3], [2, -1]]))
    assert d.tolist() == [[10.0, 0.0], [-9.25, 0.0]]
    # a scaled scatter with bf16 output rounds the exact product once
    xb = oracle.bf16_round(np.array([[1.0 + 2 ** -7]], np.float32))
    ob = oracle.permute_scaled(xb, "bf16", np.array([[0]]), np.array([1.0 + 2 ** -8], np.float32),
                               1, "bf16")
    exact = (1.0 + 2 ** -7) * (1.0 + 2 ** -8)
    assert ob[0, 0] == oracle.bf16_round(np.array([exact], np.float32))[0]


# ------------------------------------------------------------ EMA, placement

def test_ema_closed_form():
    """A constant input x from a zero state gives x * (1 - beta^n)."""
    s = np.zeros(5, np.float32)
    x = np.array([0, 1, 7, 100, 12345], np.int32)
    for n in range(1, 40):
        s = oracle.ema_update(s, x, 0.9)
        want = x.astype(np.float64) * (1.0 - 0.9 ** n)
        assert np.allclose(s, want, rtol=1e-5, atol=1e-6)
    s1 = oracle.ema_update(np.full(3, 5.0, np.float32), np.array([5, 5, 5]), 0.37)
    assert np.allclose(s1, 5.0, rtol=1e-6)


def test_placement_recovers_planted_clusters():
    """Clusters of E/G experts that are co-selected only among themselves
    land one cluster per rank."""
    rng = np.random.default_rng(50)
    for E, G in [(8, 2), (64, 8), (128, 32), (256, 64)]:
        cap = E // G
        perm = rng.permutation(E)
        C = np.zeros((E, E), np.float32)
        for c in range(G):
            mem = perm[c * cap:(c + 1) * cap]
            for i in mem:
                for j in mem:
                    if i != j:
                        C[i, j] = rng.uniform(1, 10)
        C = np.maximum(C, C.T)
        load = rng.uniform(0.5, 1.5, size=E).astype(np.float32)
        er = oracle.place_experts(C, load, G, 0.5)
        assert (np.bincount(er, minlength=G) == cap).all()
        for c in range(G):
            mem = perm[c * cap:(c + 1) * cap]
            assert len(set(er[mem].tolist())) == 1


def test_placement_capacity_load_and_pairs():
    """Every rank gets E/G experts; with a feasible workload limit no rank
    exceeds it; on workload 2's planted pairs the placement keeps at least
    as much co-activation inside ranks as the contiguous split and removes
    dispatched rows."""
    w = make(2, T=8192, with_x=False)
    st = oracle.coact_stats(w.topk, w.E)
    C = st["pair_count"].astype(np.float32)
    np.fill_diagonal(C, 0)
    load = st["expert_count"].astype(np.float32)
    er = oracle.place_experts(C, load, w.G, 0.25)
    assert (np.bincount(er, minlength=w.G) == w.E // w.G).all()
    loads = np.bincount(er, weights=load, minlength=w.G)
    assert loads.max() <= 1.25 * load.sum() / w.G + 1e-3
    kept = oracle.colocated_coactivation(C, er)
    assert kept >= oracle.colocated_coactivation(C, uniform_contiguous(w.E, w.G))
    n_planned = oracle.dispatch_plan(w.topk, None, er, w.G, w.ranks_per_node)["N"]
    n_uniform = oracle.dispatch_plan(w.topk, None, uniform_contiguous(w.E, w.G), w.G,
                                     w.ranks_per_node)["N"]
    assert n_planned < n_uniform


def test_placement_tiny_exhaustive_optimum():
    """On 4 experts / 2 ranks with one heavy pair per rank, the greedy reaches
    the exhaustive optimum of co-located co-activation."""
    C = np.array([[0, 9, 1, 0], [9, 0, 0, 2], [1, 0, 0, 8], [0, 2, 8, 0]], np.float32)
    er = oracle.place_experts(C, np.ones(4, np.float32), 2, 0.0)
    best = max(oracle.colocated_coactivation(C, np.array(p)) for p in
               itertools.product(range(2), repeat=4) if sorted(p).count(0) == 2)
    assert oracle.colocated_coactivation(C, er) == best == 17.0


# ------------------------------------------------------------ balanced shuffle

def _deferred_acceptance(score, G, cap):
    """Tokens propose down their preference lists; each rank keeps its cap
    lowest-index proposers and rejects the rest, until nobody is rejected.
    With the same token priority at every rank this gives the same matching
    as taking tokens in order (written here independently of the oracle)."""
    T = score.shape[0]
    prefs = [sorted(range(G), key=lambda r: (-int(score[t, r]), r)) for t in range(T)]
    nxt = [0] * T
    held = {r: [] for r in range(G)}
    free = list(range(T))
    while free:
        for t in free:
            held[prefs[t][nxt[t]]].append(t)
            nxt[t] += 1
        free = []
        for r in range(G):
            held[r].sort()
            free += held[r][cap:]
            held[r] = held[r][:cap]
    out = np.empty(T, np.int64)
    for r in range(G):
        for t in held[r]:
            out[t] = r
    return out


def test_balanced_shuffle_matches_deferred_acceptance():
    rng = np.random.default_rng(80)
    for trial in range(40):
        G = int(rng.integers(1, 6))
        T = G * int(rng.integers(1, 12))
        E = int(rng.integers(2, 7))
        k = int(rng.integers(1, E + 1))
        topk = _random_routing(rng, T, E, k)
        X = rng.integers(0, 3, size=(E, E))
        er2 = rng.integers(0, G, size=E).astype(np.int32)
        sh = oracle.shuffle_balanced(topk, X, er2, G)
        M = oracle.shuffle_predict(topk, X, er2, G)["rank_score"]
        score = np.stack([M[topk[t]].sum(axis=0) for t in range(T)]) if T else np.zeros((0, G))
        assert sh["pred_rank"].tolist() == _deferred_acceptance(score, G, T // G).tolist()
        assert (np.bincount(sh["pred_rank"], minlength=G) == T // G).all()
        order = sorted(range(T), key=lambda t: (int(sh["pred_rank"][t]), t))
        assert sh["perm"].tolist() == order


def test_balanced_shuffle_equals_free_shuffle_when_balanced():
    """If every rank is predicted by exactly T/G tokens, the capacity never
    binds and the balanced shuffle is the unconstrained one."""
    topk = np.array([[0], [1], [2], [3], [0], [1], [2], [3]], np.int32)
    X = np.eye(4, dtype=np.int64) * 5
    er2 = np.array([0, 1, 2, 3], np.int32)
    a = oracle.shuffle_predict(topk, X, er2, 4)
    b = oracle.shuffle_balanced(topk, X, er2, 4)
    for key in ("pred_rank", "dest_pos", "perm", "shard_offsets"):
        assert a[key].tolist() == b[key].tolist()


def test_balanced_shuffle_local_share():
    """Equal shards still keep more next-layer assignments local than the
    1/G baseline, though fewer than the unconstrained shuffle can."""
    w = make(5, T=4096, with_x=False)
    st = oracle.coact_stats(w.topk, w.E, w.topk2, w.E)
    sh = oracle.shuffle_balanced(w.topk, st["transition"], w.expert_rank2, w.G)
    perm = sh["perm"]
    p = oracle.dispatch_plan(w.topk2[perm], None, w.expert_rank2, w.G, w.ranks_per_node,
                             src_offsets=sh["shard_offsets"])
    share = p["counters"][3] / (w.T * w.k)
    assert share > 0.125 + 0.05


def test_gathered_plan_pins():
    """The plan of a shuffled batch: the identity order gives the plain plan;
    reversing two tokens on two ranks gives the hand-worked reversed rows;
    and the gathered routing is exactly the rows of topk in perm's order."""
    rng = np.random.default_rng(77)
    T, E, k, G = 96, 8, 2, 4
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    er = (np.arange(E) // 2).astype(np.int32)
    ident = oracle.dispatch_plan_gathered(topk, gates, np.arange(T), er, G, G)
    plain = oracle.dispatch_plan(topk, gates, er, G, G)
    for key in ("row_token", "token_rows", "slot_row", "send_offsets", "counters"):
        assert np.array_equal(ident[key], plain[key]), key
    assert np.array_equal(ident["row_weight"].view(np.uint32), plain["row_weight"].view(np.uint32))
    # hand case: token 0 -> experts {0} (rank 0), token 1 -> experts {2} (rank 1); one source
    # rank; perm = [1, 0] puts token 1 first, so rank 0's single row carries position 1
    t2 = np.array([[0], [2]], np.int32)
    g2 = np.array([[0.25], [0.75]], np.float32)
    er2 = np.array([0, 0, 1, 1], np.int32)
    hp = oracle.dispatch_plan_gathered(t2, g2, np.array([1, 0]), er2, 2, 2,
                                       src_offsets=np.array([0, 2, 2]))
    assert hp["topk_out"].tolist() == [[2], [0]]
    assert hp["row_token"].tolist() == [1, 0]          # rank 0: position 1; rank 1: position 0
    assert hp["token_rows"].tolist() == [[1], [0]]
    assert np.allclose(hp["row_weight"], [0.25, 0.75])
    perm = rng.permutation(T)
    gp = oracle.dispatch_plan_gathered(topk, gates, perm, er, G, G)
    assert np.array_equal(gp["topk_out"], topk[perm]) and np.array_equal(gp["gates_out"], gates[perm])
