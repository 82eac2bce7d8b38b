"""Plain CPU oracle for co-activation statistics, deduplicated dispatch,
permute, combine and token-shuffle prediction.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the engine.  It shares no code with the
HIP engine.  Everything is written for clarity, not speed: Python loops over
tokens, exact integers, float64 for real arithmetic unless a step fixes a
narrower type.

Sources (cited by page title and section):
  [EC]  "Expert Coupling in MoE Pretraining: Reducing All-to-All Overhead with
        Correlated Placement and Token Shuffling" -- abstract: co-selection of
        experts within a layer, cross-layer predictability, deduplicated
        dispatch (a token reaches a given GPU at most one time), token
        shuffling (tokens reordered by the rank forecast for their
        next-layer experts).
  [CB]  "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
        Training" -- Key Observation (Ochiai similarity over the token sets of
        two experts; node-level deduplication) and Problem Formulation (the
        cross-node volume V with D_t, s_t, N(r), r_t^e).
  [EP]  "Expert Parallelism > Expert Placement Strategies" -- uniform
        contiguous placement, device = expert // experts_per_device.
  [CE]  "Training Communication-Efficient Mixture-of-Experts Language Models
        with Layer Re-Configuration" -- footnote 3: routed probabilities are
        dispatched alongside hidden states and the hidden states are combined.

Readings where the pages leave a step open are listed beside each function.
Every function here is pinned by tests in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np


class OracleInputError(ValueError):
    """A precondition of the method is violated by the inputs."""


# --------------------------------------------------------------- validation

def validate_routing(topk: np.ndarray, E: int) -> None:
    """Each token selects k distinct experts out of E ([CB] Problem
    Formulation: D_t is a *set* of selected experts)."""
    topk = np.asarray(topk)
    if topk.ndim != 2:
        raise OracleInputError("topk must be [T, k]")
    for t in range(topk.shape[0]):
        row = [int(e) for e in topk[t]]
        for e in row:
            if e < 0 or e >= E:
                raise OracleInputError(f"token {t}: expert id {e} not in [0, {E})")
        if len(set(row)) != len(row):
            raise OracleInputError(f"token {t}: expert listed twice")


def validate_placement(expert_rank: np.ndarray, E: int, G: int) -> None:
    """One replica per expert: expert e lives on rank p(e) in [0, G)."""
    expert_rank = np.asarray(expert_rank)
    if expert_rank.shape != (E,):
        raise OracleInputError("expert_rank must have E entries")
    for e in range(E):
        if not 0 <= int(expert_rank[e]) < G:
            raise OracleInputError(f"expert {e}: rank {int(expert_rank[e])} not in [0, {G})")


def source_offsets(T: int, G: int, src_offsets=None) -> list:
    """Token ranges per source rank.

    Reading: sequence parallelism shards the tokens across the EP group
    ([EC] abstract), taken as contiguous shards in token order.  With no
    explicit offsets the shards are equal, s_t = t div (T/G).
    """
    if src_offsets is None:
        if T % G != 0:
            raise OracleInputError("equal shards need T divisible by G")
        return [s * (T // G) for s in range(G + 1)]
    off = [int(v) for v in src_offsets]
    if len(off) != G + 1 or off[0] != 0 or off[-1] != T:
        raise OracleInputError("src_offsets must run from 0 to T over G+1 entries")
    for s in range(G):
        if off[s + 1] < off[s]:
            raise OracleInputError("src_offsets must be nondecreasing")
    return off


def source_rank_of_tokens(T: int, G: int, src_offsets=None) -> np.ndarray:
    """s_t of [CB] Problem Formulation: the rank that holds token t."""
    off = source_offsets(T, G, src_offsets)
    s_of = np.empty(T, dtype=np.int64)
    for s in range(G):
        for t in range(off[s], off[s + 1]):
            s_of[t] = s
    return s_of


# ------------------------------------------------------- co-activation stats

def ochiai(pair_count: np.ndarray, expert_count: np.ndarray) -> np.ndarray:
    """Ochiai(A, B) = |A n B| / sqrt(|A| |B|) over the token sets of two
    experts ([CB] Key Observation).

    Computed in float64 (the product |A||B| as a double, a correctly rounded
    square root and quotient) and rounded once to float32.  Reading: 0 where
    either set is empty (the formula is 0/0 there); the diagonal follows the
    formula, so it is 1 for every expert that some token selected.
    """
    E = len(expert_count)
    out = np.zeros((E, E), dtype=np.float32)
    for i in range(E):
        for j in range(E):
            d = float(expert_count[i]) * float(expert_count[j])
            if d > 0.0:
                out[i, j] = np.float32(float(pair_count[i, j]) / math.sqrt(d))
    return out


def coact_stats(topk: np.ndarray, E: int, topk_next: Optional[np.ndarray] = None,
                E_next: Optional[int] = None) -> dict:
    """Per-expert counts, E x E co-selection counts, Ochiai similarity and
    layer-to-layer transition counts.

    * expert_count[e] = |A_e| with A_e = {t : e in D_t}  ([CB] Key Observation:
      the set of active tokens of each expert).
    * pair_count[i][j] = |A_i n A_j|: the number of tokens that select both i
      and j ([EC] abstract: expert pairs selected together).  Full symmetric
      matrix, diagonal = expert_count.
    * ochiai as above.
    * transition[i][j] = #{t : i in D_t at this layer, j in D'_t at the next}
      ([EC] abstract: the experts a token selects at one layer predict those it
      selects at the next).  Rows index this layer, columns the next.
    """
    topk = np.asarray(topk)
    validate_routing(topk, E)
    T = topk.shape[0]
    n = np.zeros(E, dtype=np.int64)
    C = np.zeros((E, E), dtype=np.int64)
    for t in range(T):
        D = [int(e) for e in topk[t]]
        for i in D:
            n[i] += 1
            for j in D:
                C[i, j] += 1
    out = {"expert_count": n, "pair_count": C, "ochiai": ochiai(C, n)}
    if topk_next is not None:
        topk_next = np.asarray(topk_next)
        validate_routing(topk_next, E_next)
        if topk_next.shape[0] != T:
            raise OracleInputError("both layers must cover the same tokens")
        X = np.zeros((E, E_next), dtype=np.int64)
        for t in range(T):
            for i in topk[t]:
                for j in topk_next[t]:
                    X[int(i), int(j)] += 1
        out["transition"] = X
    return out


# ----------------------------------------------------------- dispatch plan

def dispatch_plan(topk: np.ndarray, gates: Optional[np.ndarray], expert_rank: np.ndarray,
                  G: int, ranks_per_node: int, src_offsets=None) -> dict:
    """Deduplicated dispatch plan: every token goes to every rank that holds
    at least one of its experts exactly once ([EC] abstract: deduplicated
    dispatch, one visit per GPU however many of the token's experts it
    holds).

    With one replica per expert the rank of task (t, e) is forced,
    r_t^e = p(e) ([CB] Problem Formulation).  R_t = {p(e) : e in D_t} is the
    token's set of destination ranks; one send row per (t, r in R_t).

    Reading (the pages give no buffer layout): rows are ordered by
    (source rank s_t, destination rank r, token t), so each (s, r) block is
    one all-to-all message and is contiguous per source.

    row_weight(t, r) is the token's gate mass on rank r, a float32 running sum
    over ascending slot j starting from 0 (reading: the routed probabilities
    travel with the hidden rows, [CE] footnote 3, and the combine applies
    them).

    Counters: N (rows), T*k (assignments), local_rows (#(t, r) with r = s_t),
    local_assign (#(t, j) with p(D_t[j]) = s_t), node_rows = sum_t |N_t| with
    N_t = {node(r) : r in R_t}, V = sum_t |N_t minus {node(s_t)}| (the
    cross-node volume of [CB] Problem Formulation), max rows received by one
    rank, and a reserved 0.  node(r) = r div ranks_per_node.
    """
    topk = np.asarray(topk)
    expert_rank = np.asarray(expert_rank)
    T, k = topk.shape
    E = expert_rank.shape[0]
    validate_routing(topk, E)
    validate_placement(expert_rank, E, G)
    if G % ranks_per_node != 0:
        raise OracleInputError("ranks_per_node must divide G")
    s_of = source_rank_of_tokens(T, G, src_offsets)

    def p(e):
        return int(expert_rank[int(e)])

    rows = []
    for t in range(T):
        for r in sorted({p(e) for e in topk[t]}):
            rows.append((int(s_of[t]), r, t))
    rows.sort()
    index = {}
    for i, (s, r, t) in enumerate(rows):
        index[(t, r)] = i
    N = len(rows)

    S = np.zeros((G, G), dtype=np.int64)
    for (s, r, t) in rows:
        S[s, r] += 1
    send_offsets = np.zeros(G * G + 1, dtype=np.int64)
    flat = S.reshape(-1)
    for q in range(G * G):
        send_offsets[q + 1] = send_offsets[q] + flat[q]

    row_token = np.array([t for (s, r, t) in rows], dtype=np.int64)
    row_weight = np.zeros(N, dtype=np.float32)
    if gates is not None:
        gates = np.asarray(gates, dtype=np.float32)
        for i, (s, r, t) in enumerate(rows):
            a = np.float32(0.0)
            for j in range(k):
                if p(topk[t, j]) == r:
                    a = np.float32(a + gates[t, j])
            row_weight[i] = a

    token_rows = np.full((T, k), -1, dtype=np.int64)
    slot_row = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        for q, r in enumerate(sorted({p(e) for e in topk[t]})):
            token_rows[t, q] = index[(t, r)]
        for j in range(k):
            slot_row[t, j] = index[(t, p(topk[t, j]))]

    local_rows = sum(1 for (s, r, t) in rows if r == s)
    local_assign = 0
    node_rows = 0
    V = 0
    for t in range(T):
        s = int(s_of[t])
        local_assign += sum(1 for e in topk[t] if p(e) == s)
        nodes = {p(e) // ranks_per_node for e in topk[t]}
        node_rows += len(nodes)
        V += len(nodes - {s // ranks_per_node})
    max_recv = int(S.sum(axis=0).max()) if G > 0 else 0
    counters = np.array([N, T * k, local_rows, local_assign, node_rows, V, max_recv, 0],
                        dtype=np.int64)
    return {"send_counts": S, "send_offsets": send_offsets, "row_token": row_token,
            "row_weight": row_weight, "token_rows": token_rows, "slot_row": slot_row,
            "counters": counters, "N": N}


# ---------------------------------------------------------------- permute

def permute_rows(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """Send buffer: row i is a bit copy of x[row_token[i]] (the dispatched
    hidden state of [CE] footnote 3).  Works on any dtype, bf16 included as
    uint16 bit patterns."""
    return np.asarray(x)[np.asarray(row_token, dtype=np.int64)]


def scatter_rows(x: np.ndarray, dest: np.ndarray, out_rows: int) -> np.ndarray:
    """out[dest[t]] = x[t] for every t with dest[t] >= 0 (a one-row-per-token
    move, e.g. the token shuffle); untouched rows stay zero."""
    x = np.asarray(x)
    out = np.zeros((out_rows,) + x.shape[1:], dtype=x.dtype)
    for t in range(x.shape[0]):
        if int(dest[t]) >= 0:
            out[int(dest[t])] = x[t]
    return out


# ---------------------------------------------------------------- bf16

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """A bf16 value is the upper half of the float32 with the same bits."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (8 significant bits), nearest, ties to an
    even last bit; result as uint16 bit patterns.

    Written from the definition: the two bf16 neighbours of x are the value
    with the low 16 bits cleared (toward zero) and the next one away from
    zero; the nearer one wins, a tie goes to the one whose last kept bit is 0.
    Magnitudes at or past the midpoint between the largest finite bf16 and
    2^128 become infinity.  NaN stays NaN (quiet), infinities stay.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lo = bits >> 16                                   # neighbour toward zero
    mag_lo = ((lo & 0x7FFF) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    exp_field = ((lo >> 7) & 0xFF).astype(np.int64)
    # spacing of bf16 values in lo's binade (subnormals share binade 1)
    ulp = np.ldexp(1.0, np.maximum(exp_field, 1) - 127 - 7)
    mag_hi = mag_lo + ulp                             # 2^128 past the largest finite
    a = np.abs(x.astype(np.float64))
    with np.errstate(invalid="ignore"):           # inf/NaN lanes are replaced below
        d_lo = a - mag_lo
        d_hi = mag_hi - a
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((lo & 1) == 0))
    # lo + 1 is the next magnitude; a carry into the exponent is exact,
    # and 0x7F7F + 1 = 0x7F80 is infinity.
    out = np.where(take_lo, lo, lo + 1)
    out = np.where(np.isinf(x), lo, out)
    out = np.where(np.isnan(x), lo | 0x0040, out)     # quiet NaN, payload kept
    return (out & 0xFFFF).astype(np.uint16)


def _as_f64(z: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f32(z).astype(np.float64)
    return np.asarray(z, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- combine

def combine(Z: np.ndarray, z_dtype: str, slot_row: np.ndarray, gates: np.ndarray,
            out_dtype: str) -> np.ndarray:
    """Weighted combine back to token order: y_t = sum_j w_tj * Z[row of
    (t, p(D_t[j]))] (the hidden-state combine of [CE] footnote 3; with the
    deduplicated dispatch of [EC] every assignment of t on rank r reads the
    single row (t, r)).

    Sum in float64, rounded once to float32; a bf16 output is the bf16
    rounding of that float32 value.  ``Z`` holds the expert-side rows, indexed
    by ``slot_row`` [T, k].
    """
    slot_row = np.asarray(slot_row, dtype=np.int64)
    gates = np.asarray(gates, dtype=np.float32)
    T, k = slot_row.shape
    Zf = _as_f64(Z, z_dtype)
    y = np.zeros((T, Zf.shape[1]), dtype=np.float64)
    for j in range(k):
        y += gates[:, j].astype(np.float64)[:, None] * Zf[slot_row[:, j]]
    y32 = y.astype(np.float32)
    return bf16_round(y32) if out_dtype == "bf16" else y32


def combine_unweighted(Z: np.ndarray, z_dtype: str, token_rows: np.ndarray,
                       out_dtype: str) -> np.ndarray:
    """y_t = sum over the token's rows (one per rank in R_t) of Z[row]: the
    combine for an expert side that already applied the gates."""
    token_rows = np.asarray(token_rows, dtype=np.int64)
    T, k = token_rows.shape
    Zf = _as_f64(Z, z_dtype)
    y = np.zeros((T, Zf.shape[1]), dtype=np.float64)
    for t in range(T):
        for q in range(k):
            if token_rows[t, q] >= 0:
                y[t] += Zf[token_rows[t, q]]
    y32 = y.astype(np.float32)
    return bf16_round(y32) if out_dtype == "bf16" else y32


# ---------------------------------------------------------- token shuffle

def shuffle_predict(topk: np.ndarray, transition: np.ndarray, expert_rank_next: np.ndarray,
                    G: int) -> dict:
    """Predict the rank holding each token's next-layer experts and order the
    tokens by it ([EC] abstract: token shuffling, tokens reordered by the rank
    forecast for their next-layer experts).

    Readings: the prediction scores rank r by the transition counts from the
    token's current experts into the next-layer experts placed on r,
    score_t[r] = sum_{i in D_t} sum_{j : p'(j) = r} X[i][j], raw integer
    counts; pred_t = the highest-scoring rank, lowest rank on ties (an
    all-zero score gives rank 0); no capacity limit, so shard sizes vary.
    The new order is stable: tokens keep ascending t within a rank.
    """
    topk = np.asarray(topk)
    X = np.asarray(transition, dtype=np.int64)
    E, E_next = X.shape
    validate_routing(topk, E)
    validate_placement(expert_rank_next, E_next, G)
    T = topk.shape[0]
    M = np.zeros((E, G), dtype=np.int64)
    for i in range(E):
        for j in range(E_next):
            M[i, int(expert_rank_next[j])] += X[i, j]
    pred = np.empty(T, dtype=np.int64)
    for t in range(T):
        score = np.zeros(G, dtype=np.int64)
        for i in topk[t]:
            score += M[int(i)]
        best = 0
        for r in range(1, G):
            if score[r] > score[best]:
                best = r
        pred[t] = best
    # stable counting sort by predicted rank
    counts = np.zeros(G, dtype=np.int64)
    for t in range(T):
        counts[pred[t]] += 1
    shard_offsets = np.zeros(G + 1, dtype=np.int64)
    for r in range(G):
        shard_offsets[r + 1] = shard_offsets[r] + counts[r]
    fill = shard_offsets[:G].copy()
    dest_pos = np.empty(T, dtype=np.int64)
    perm = np.empty(T, dtype=np.int64)
    for t in range(T):
        dest_pos[t] = fill[pred[t]]
        perm[fill[pred[t]]] = t
        fill[pred[t]] += 1
    return {"pred_rank": pred, "dest_pos": dest_pos, "perm": perm,
            "shard_offsets": shard_offsets, "rank_score": M}


def dispatch_plan_gathered(topk: np.ndarray, gates: Optional[np.ndarray], perm: np.ndarray,
                           expert_rank: np.ndarray, G: int, ranks_per_node: int,
                           src_offsets=None) -> dict:
    """The plan of a shuffled batch ([EC] abstract: tokens move to the rank
    predicted for their next-layer experts, and that layer dispatches from
    there): position p holds token perm[p], so the routing in the new order
    is topk[perm], gates[perm], and the plan is dispatch_plan on it.  Returns
    the plan with the gathered routing under "topk_out" / "gates_out"."""
    perm = np.asarray(perm, dtype=np.int64)
    topk_s = np.asarray(topk)[perm]
    gates_s = None if gates is None else np.asarray(gates)[perm]
    out = dict(dispatch_plan(topk_s, gates_s, expert_rank, G, ranks_per_node,
                             src_offsets=src_offsets))
    out["topk_out"] = topk_s
    out["gates_out"] = gates_s
    return out


def two_layer_pipeline(topk1: np.ndarray, topk2: np.ndarray, gates2: np.ndarray,
                       x: np.ndarray, expert_rank2: np.ndarray, E: int, E2: int,
                       G: int, ranks_per_node: int) -> dict:
    """Two consecutive MoE layers with token shuffling ([EC] abstract):
    statistics of layer 1 with the layer-1 -> layer-2 transitions, prediction
    of each token's layer-2 rank, the shuffle (tokens and their layer-2
    routing move together), then the layer-2 deduplicated plan with the new
    shards as source ranks, and the layer-2 permute.

    Reading: the transition counts come from the same batch (in-sample).
    """
    T = topk1.shape[0]
    stats = coact_stats(topk1, E, topk2, E2)
    sh = shuffle_predict(topk1, stats["transition"], expert_rank2, G)
    perm = sh["perm"]
    x_s = np.asarray(x)[perm]
    topk2_s = np.asarray(topk2)[perm]
    gates2_s = np.asarray(gates2)[perm]
    plan_before = dispatch_plan(topk2, gates2, expert_rank2, G, ranks_per_node)
    plan = dispatch_plan(topk2_s, gates2_s, expert_rank2, G, ranks_per_node,
                         src_offsets=sh["shard_offsets"])
    send = permute_rows(x_s, plan["row_token"])
    k2 = topk2.shape[1]
    return {"stats": stats, "shuffle": sh, "x_shuffled": x_s, "topk2_shuffled": topk2_s,
            "gates2_shuffled": gates2_s, "plan": plan, "send": send,
            "local_share_before": plan_before["counters"][3] / (T * k2),
            "local_share_after": plan["counters"][3] / (T * k2)}


def shuffle_dispatch(x: np.ndarray, perm: np.ndarray, token_rows: np.ndarray,
                     n_send_rows: int) -> tuple:
    """The shuffle's token move and the next layer's dispatch in one pass:
    shuffled position p holds token perm[p], and that row is also written to
    every send row the next layer's plan gives position p (token_rows is
    indexed by shuffled position).  Returns (x_shuffled, send); send rows no
    position targets stay zero.  Written from the definitions:
    x_s[p] = x[perm[p]], send[token_rows[p, q]] = x[perm[p]]."""
    x = np.asarray(x)
    perm = np.asarray(perm, dtype=np.int64)
    token_rows = np.asarray(token_rows, dtype=np.int64)
    x_s = np.zeros_like(x)
    send = np.zeros((n_send_rows,) + x.shape[1:], dtype=x.dtype)
    for p in range(x.shape[0]):
        row = x[int(perm[p])]
        x_s[p] = row
        for q in range(token_rows.shape[1]):
            r = int(token_rows[p, q])
            if r >= 0:
                send[r] = row
    return x_s, send


# ------------------------------------------------ destination-side expansion

def expert_plan(topk: np.ndarray, gates: Optional[np.ndarray], expert_rank: np.ndarray, G: int,
                slot_row: np.ndarray, n_send_rows: int) -> dict:
    """Per-expert grouped layout on the destination side.

    Every assignment (t, j) -- token t, slot j, expert e = D_t[j], rank
    r = p(e) -- gets one expert row.  Reading: rows are ordered by
    (rank r, expert e, token t), i.e. each rank's received tokens expanded
    into one contiguous block per local expert (ascending expert id), tokens
    ascending inside a block -- the layout a grouped expert GEMM consumes
    ([CE] training stack: grouped GEMM after the alltoall dispatch; footnote
    3: the routed probabilities travel with the rows, so each expert row
    carries its gate).

    Outputs: erow [T, k] (expert row of each slot), expert_first[e] and
    expert_count[e], rank_offsets [G+1], erow_weight / erow_slot / erow_src
    per expert row (gate, t*k + j, and the send row the slot was dispatched
    in), and row_dest [n_send_rows, k]: for send row (t, r), the expert rows
    of t's slots on r in ascending slot order, then -1.
    """
    topk = np.asarray(topk)
    expert_rank = np.asarray(expert_rank)
    T, k = topk.shape
    E = expert_rank.shape[0]
    validate_routing(topk, E)
    validate_placement(expert_rank, E, G)
    keys = sorted((int(expert_rank[int(topk[t, j])]), int(topk[t, j]), t, j)
                  for t in range(T) for j in range(k))
    erow = np.full((T, k), -1, dtype=np.int64)
    erow_weight = np.zeros(T * k, dtype=np.float32)
    erow_slot = np.full(T * k, -1, dtype=np.int64)
    erow_src = np.full(T * k, -1, dtype=np.int64)
    for i, (r, e, t, j) in enumerate(keys):
        erow[t, j] = i
        erow_slot[i] = t * k + j
        erow_src[i] = int(slot_row[t, j])
        if gates is not None:
            erow_weight[i] = np.float32(gates[t, j])
    expert_count = np.zeros(E, dtype=np.int64)
    for (r, e, t, j) in keys:
        expert_count[e] += 1
    expert_first = np.zeros(E, dtype=np.int64)
    rank_offsets = np.zeros(G + 1, dtype=np.int64)
    pos = 0
    for r in range(G):
        rank_offsets[r] = pos
        for e in range(E):
            if int(expert_rank[e]) == r:
                expert_first[e] = pos
                pos += int(expert_count[e])
    rank_offsets[G] = pos
    row_dest = np.full((n_send_rows, k), -1, dtype=np.int64)
    for t in range(T):
        used = {}
        for j in range(k):
            i = int(slot_row[t, j])
            q = used.get(i, 0)
            row_dest[i, q] = erow[t, j]
            used[i] = q + 1
    return {"erow": erow, "expert_first": expert_first, "expert_count": expert_count,
            "rank_offsets": rank_offsets, "erow_weight": erow_weight, "erow_slot": erow_slot,
            "erow_src": erow_src, "row_dest": row_dest}


def partial_combine(Y: np.ndarray, y_dtype: str, erow: np.ndarray, gates: np.ndarray,
                    slot_row: np.ndarray, n_send_rows: int, out_dtype: str) -> np.ndarray:
    """The expert side's reply rows: for send row (t, r),
    Z[(t, r)] = sum_{j : p(D_t[j]) = r} w_tj * Y[erow(t, j)]
    (the expert outputs of t on rank r, weighted by their gates), summed in
    float64 and rounded once.  Rows no slot maps to stay zero."""
    erow = np.asarray(erow, dtype=np.int64)
    slot_row = np.asarray(slot_row, dtype=np.int64)
    T, k = erow.shape
    Yf = _as_f64(Y, y_dtype)
    Z = np.zeros((n_send_rows, Yf.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            Z[slot_row[t, j]] += float(np.float32(gates[t, j])) * Yf[erow[t, j]]
    Z32 = Z.astype(np.float32)
    return bf16_round(Z32) if out_dtype == "bf16" else Z32


def moe_output(x: np.ndarray, x_dtype: str, topk: np.ndarray, gates: np.ndarray,
               expert_scale: np.ndarray) -> np.ndarray:
    """Plain MoE layer output for experts that scale their input row by a
    per-expert constant: y_t = sum_j w_tj * c_{D_t[j]} * x_t, in float64.
    The reference the dispatched path must reproduce (routing and expert
    parameters are untouched by the dispatch, [EC] abstract)."""
    xf = _as_f64(x, x_dtype)
    T, k = topk.shape
    y = np.zeros_like(xf)
    for t in range(T):
        for j in range(k):
            y[t] += float(np.float32(gates[t, j])) * float(expert_scale[int(topk[t, j])]) * xf[t]
    return y


# ------------------------------------------------------------ backward

def permute_scaled(x: np.ndarray, x_dtype: str, dest: np.ndarray, scale: np.ndarray,
                   out_rows: int, out_dtype: str) -> np.ndarray:
    """out[dest[t, q]] = scale[dest[t, q]] * x[t], the product formed exactly
    (float64) and rounded once to float32, then to bf16 for a bf16 output.
    The adjoint of the weighted combine with respect to its rows: the
    gradient of each dispatched row is its gate mass times the gradient of
    its token's output (the inverse all-to-alls of [CE] footnote 3 and the
    backward passes of [EC] abstract).  Untargeted rows stay zero."""
    xf = _as_f64(x, x_dtype)
    dest = np.asarray(dest, dtype=np.int64)
    if dest.ndim == 1:
        dest = dest[:, None]
    out = np.zeros((out_rows, xf.shape[1]), dtype=np.float64)
    for t in range(dest.shape[0]):
        for q in range(dest.shape[1]):
            r = int(dest[t, q])
            if r >= 0:
                out[r] = float(np.float32(scale[r])) * xf[t]
    o32 = out.astype(np.float32)
    return bf16_round(o32) if out_dtype == "bf16" else o32


def row_dot(a: np.ndarray, a_dtype: str, b: np.ndarray, b_dtype: str,
            rows: np.ndarray) -> np.ndarray:
    """out[t, q] = <a[t], b[rows[t, q]]> (0 where rows[t, q] < 0), summed in
    float64, rounded once to float32.  With a = dY and b the rows a slot
    reads, this is the gradient of the output with respect to that slot's
    gate weight."""
    af = _as_f64(a, a_dtype)
    bf = _as_f64(b, b_dtype)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros(rows.shape, dtype=np.float64)
    for t in range(rows.shape[0]):
        for q in range(rows.shape[1]):
            if rows[t, q] >= 0:
                out[t, q] = float(np.dot(af[t], bf[rows[t, q]]))
    return out.astype(np.float32)


# ------------------------------------------------- EMA statistics, placement

def ema_update(state: np.ndarray, x: np.ndarray, beta: float) -> np.ndarray:
    """Exponential moving average of per-step statistics ([CB] Stage 1: the
    planner works from EMAs of co-selection counts and expert loads; the
    decay is not given -- reading: a caller parameter).  float32 state;
    new = beta * state + (1 - beta) * x, each product and the sum rounded to
    float32 in that order."""
    b = np.float32(beta)
    ob = np.float32(np.float32(1.0) - b)
    s = np.asarray(state, dtype=np.float32)
    xv = np.asarray(x).astype(np.float32)
    return (s * b + xv * ob).astype(np.float32)


def colocated_coactivation(C: np.ndarray, expert_rank: np.ndarray) -> float:
    """Sum of C[i][j] over unordered pairs i < j placed on the same rank:
    the co-activation a placement keeps inside ranks."""
    E = len(expert_rank)
    tot = 0.0
    for i in range(E):
        for j in range(i + 1, E):
            if int(expert_rank[i]) == int(expert_rank[j]):
                tot += float(C[i][j])
    return tot


def place_experts(C: np.ndarray, load: np.ndarray, G: int, eps: float) -> np.ndarray:
    """Co-activation placement ([EC] abstract: experts often selected
    together go on the same GPU; [CB] Stage 1: maximise co-activation kept
    inside ranks under a workload limit).  The pages give no algorithm;
    reading -- grow one rank at a time:

    * every rank holds exactly E/G experts; the workload limit is
      L = (1 + eps) * sum(load) / G;
    * ranks are filled in order 0..G-1; each step adds to the current rank
      the unplaced expert with the largest summed co-activation with the
      rank's experts so far, ties broken by the larger total co-activation
      sum_{f != e} C[e][f], then the lower id (so an empty rank is seeded
      with the most co-activated expert left); candidates whose load keeps
      the rank within L are preferred when there are any.
    Sums are float64 over float32 inputs, in ascending expert order."""
    C = np.asarray(C, dtype=np.float32)
    load = np.asarray(load, dtype=np.float32)
    E = C.shape[0]
    if E % G != 0:
        raise OracleInputError("E must be divisible by G")
    cap = E // G
    limit = (1.0 + eps) * sum(float(v) for v in load) / G
    total = []
    for e in range(E):
        t = 0.0
        for f in range(E):
            if f != e:
                t += float(C[e][f])
        total.append(t)
    rank = [-1] * E
    for r in range(G):
        members = []
        rload = 0.0
        while len(members) < cap:
            cands = [e for e in range(E) if rank[e] < 0]
            fits = [e for e in cands if rload + float(load[e]) <= limit]
            pool = fits if fits else cands
            best = None
            for e in pool:
                aff = 0.0
                for f in sorted(members):
                    aff += float(C[e][f])
                key = (-aff, -total[e], e)
                if best is None or key < best[0]:
                    best = (key, e)
            e = best[1]
            rank[e] = r
            members.append(e)
            rload += float(load[e])
    return np.array(rank, dtype=np.int32)


def shuffle_balanced(topk: np.ndarray, transition: np.ndarray, expert_rank_next: np.ndarray,
                     G: int) -> dict:
    """Token shuffle with equal shards: every rank receives exactly T/G
    tokens, as the reduce-scatter that carries the shuffle ([EC] abstract)
    hands each rank a fixed share.

    Reading (the pages do not say how a full rank is handled): tokens are
    taken in token order; each takes the highest-scoring rank (score_t[r] as
    in shuffle_predict, ties to the lower rank) that still has room.  The new
    order is stable, as in shuffle_predict."""
    topk = np.asarray(topk)
    T = topk.shape[0]
    if T % G != 0:
        raise OracleInputError("equal shards need T divisible by G")
    cap = T // G
    M = shuffle_predict(topk, transition, expert_rank_next, G)["rank_score"]
    taken = [0] * G
    pred = np.empty(T, dtype=np.int64)
    for t in range(T):
        score = np.zeros(G, dtype=np.int64)
        for i in topk[t]:
            score += M[int(i)]
        prefs = sorted(range(G), key=lambda r: (-int(score[r]), r))
        for r in prefs:
            if taken[r] < cap:
                pred[t] = r
                taken[r] += 1
                break
    fill = [r * cap for r in range(G)]
    dest_pos = np.empty(T, dtype=np.int64)
    perm = np.empty(T, dtype=np.int64)
    for t in range(T):
        dest_pos[t] = fill[pred[t]]
        perm[fill[pred[t]]] = t
        fill[pred[t]] += 1
    return {"pred_rank": pred, "dest_pos": dest_pos, "perm": perm,
            "shard_offsets": np.arange(G + 1, dtype=np.int64) * cap}
