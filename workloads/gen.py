"""Seeded synthetic router outputs for the five dispatch workloads.

No production router traces are available, so every workload is drawn from
``numpy.random.default_rng(seed)`` (PCG64) with a fixed recipe.  Draw order in
every recipe: structure (expert pairs / clusters / placement), then the
per-token choices, then the router logits, then the hidden rows ``x``.

Router model (shared by all workloads): logits are N(0,1) per (token, expert)
plus a bias on the experts of the token's chosen pair/cluster/group; top-k is
the k largest logits (stable order, ties to the lower expert id); the gate
weights are the softmax over the k selected logits, computed in float64 and
stored as float32.

The hidden rows are N(0,1) float32, kept as float32 for the small fp32
workload and rounded to bf16 (round-to-nearest-even, done by torch's CPU cast)
for the bf16 workloads.  bf16 rows are returned as their uint16 bit patterns
because numpy has no bf16 type.

Workloads (T tokens, H hidden, E experts, k per token, G logical ranks):
  1: T=2048  H=128 fp32, E=8,   k=2, G=4  (1 node of 4), 4 fixed pairs (+2.0)
  2: T=16384 H=2048 bf16, E=64, k=2, G=8  (1 node), 32 fixed pairs (+2.5),
     placement co-locates 24 of the 32 pairs
  3: T=65536 H=4096 bf16, E=128, k=6, G=32 (4 nodes of 8), 64 six-expert
     clusters drawn Zipf(1.1) (+2.0), each cluster on <=2 ranks
  4: T=32768 H=7168 bf16, E=256, k=8, G=64 (8 nodes of 8), 128 eight-expert
     groups (+1.5), 20% of tokens unbiased; correlated and uniform placement
  5: two MoE layers, T=65536 H=4096 bf16, E=64, k=2, G=8; the layer-2 pair is
     a fixed map of the layer-1 pair with probability 0.7, else uniform
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# name, T, H, dtype, E, k, G, ranks_per_node
CONFIGS = {
    1: dict(T=2048, H=128, dtype="f32", E=8, k=2, G=4, ranks_per_node=4),
    2: dict(T=16384, H=2048, dtype="bf16", E=64, k=2, G=8, ranks_per_node=8),
    3: dict(T=65536, H=4096, dtype="bf16", E=128, k=6, G=32, ranks_per_node=8),
    4: dict(T=32768, H=7168, dtype="bf16", E=256, k=8, G=64, ranks_per_node=8),
    5: dict(T=65536, H=4096, dtype="bf16", E=64, k=2, G=8, ranks_per_node=8),
}

_X_CHUNK_ROWS = 4096


@dataclass
class Workload:
    cfg: int
    T: int
    H: int
    dtype: str  # "bf16" or "f32"
    E: int
    k: int
    G: int
    ranks_per_node: int
    topk: np.ndarray  # int32 [T, k]
    gates: np.ndarray  # float32 [T, k]
    expert_rank: np.ndarray  # int32 [E], the placement this workload runs
    alt_expert_rank: Optional[np.ndarray] = None  # second placement, if any
    x: Optional[np.ndarray] = None  # uint16 bf16 bits or float32, [T, H]
    # second MoE layer (workload 5 only)
    topk2: Optional[np.ndarray] = None
    gates2: Optional[np.ndarray] = None
    expert_rank2: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def row_bytes(self) -> int:
        return self.H * (2 if self.dtype == "bf16" else 4)


def uniform_contiguous(E: int, G: int) -> np.ndarray:
    """Expert e lives on rank e // (E/G): the contiguous equal split."""
    assert E % G == 0
    return (np.arange(E) // (E // G)).astype(np.int32)


def _route(rng, T, E, k, bias_sets, bias):
    """Draw logits N(0,1)+bias on each token's set, take top-k and gates.

    ``bias_sets`` is an int array [T, m] of the experts to bias per token, or
    ``None`` entries (rows with -1) for unbiased tokens.
    """
    logits = rng.standard_normal((T, E))
    rows = np.repeat(np.arange(T), bias_sets.shape[1])
    cols = bias_sets.reshape(-1)
    ok = cols >= 0
    logits[rows[ok], cols[ok]] += bias
    topk = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, topk, axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w /= w.sum(axis=1, keepdims=True)
    return topk.astype(np.int32), w.astype(np.float32)


def _hidden(rng, T, H, dtype):
    """N(0,1) rows; bf16 workloads are rounded by torch's CPU cast (RNE)."""
    if dtype == "f32":
        return rng.standard_normal((T, H), dtype=np.float32)
    import torch

    out = np.empty((T, H), dtype=np.uint16)
    for a in range(0, T, _X_CHUNK_ROWS):
        b = min(T, a + _X_CHUNK_ROWS)
        chunk = rng.standard_normal((b - a, H), dtype=np.float32)
        out[a:b] = torch.from_numpy(chunk).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out


def expert_outputs(rows: int, H: int, dtype: str, seed: int = 1) -> np.ndarray:
    """Stand-in expert outputs Z [rows, H]: an independent N(0,1) buffer."""
    rng = np.random.default_rng(seed)
    return _hidden(rng, rows, H, dtype)


def device_normal(rows: int, H: int, dtype: str, seed: int, device="cuda"):
    """N(0,1) [rows, H] drawn on the device by torch's seeded generator
    (Philox), cast to bf16 by torch (RNE) or kept fp32.  Used for the large
    stand-in expert outputs, where a host draw would dominate run time."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((rows, H), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device=device)
    step = max(1, (1 << 26) // max(H, 1))
    for a in range(0, rows, step):
        b = min(rows, a + step)
        out[a:b] = torch.randn((b - a, H), generator=g, device=device, dtype=torch.float32)
    return out


def make(cfg: int, T: Optional[int] = None, H: Optional[int] = None, seed: int = 0,
         with_x: bool = True) -> Workload:
    """Build workload ``cfg`` (1..5); ``T``/``H`` override the sizes for
    smaller test cases that keep the same structure."""
    c = dict(CONFIGS[cfg])
    if T is not None:
        c["T"] = T
    if H is not None:
        c["H"] = H
    T, H, E, k, G = c["T"], c["H"], c["E"], c["k"], c["G"]
    rng = np.random.default_rng(seed)
    meta = {}
    alt = None
    topk2 = gates2 = er2 = None

    if cfg == 1:
        pairs = rng.permutation(E).reshape(E // 2, 2)
        choice = rng.integers(0, pairs.shape[0], size=T)
        topk, gates = _route(rng, T, E, k, pairs[choice], 2.0)
        er = uniform_contiguous(E, G)
        meta["pairs"] = pairs
    elif cfg == 2:
        pairs = rng.permutation(E).reshape(32, 2)
        po = rng.permutation(32)
        base = np.empty(E, dtype=np.int64)
        for i in range(24):  # 24 pairs, 4 per rank, on ranks 0..5
            base[pairs[po[i]]] = i // 4
        for i in range(24, 32):  # 8 pairs split across ranks 6 and 7
            base[pairs[po[i], 0]] = 6
            base[pairs[po[i], 1]] = 7
        relabel = rng.permutation(G)
        er = relabel[base].astype(np.int32)
        alt = uniform_contiguous(E, G)
        choice = rng.integers(0, 32, size=T)
        topk, gates = _route(rng, T, E, k, pairs[choice], 2.5)
        meta["pairs"] = pairs
    elif cfg == 3:
        er = (rng.permutation(E) // (E // G)).astype(np.int32)  # 4 experts/rank
        on_rank = [np.flatnonzero(er == r) for r in range(G)]
        clusters = np.empty((64, 6), dtype=np.int64)
        for cl in range(64):
            a = cl % G
            b = (a + 1 + rng.integers(0, G - 1)) % G
            two = rng.choice(on_rank[b], size=2, replace=False)
            clusters[cl] = np.concatenate([on_rank[a], two])
        sigma = rng.permutation(64)
        zipf = (np.arange(64) + 1.0) ** -1.1
        q = rng.choice(64, size=T, p=zipf / zipf.sum())
        topk, gates = _route(rng, T, E, k, clusters[sigma[q]], 2.0)
        alt = uniform_contiguous(E, G)
        meta["clusters"] = clusters
    elif cfg == 4:
        er = (rng.permutation(E) // (E // G)).astype(np.int32)  # 4 experts/rank
        on_rank = [np.flatnonzero(er == r) for r in range(G)]
        groups = np.empty((128, 8), dtype=np.int64)
        for g in range(128):
            a = g % G
            b = (a + 1 + rng.integers(0, G - 1)) % G
            groups[g] = np.concatenate([on_rank[a], on_rank[b]])
        unbiased = rng.random(T) < 0.2
        gsel = rng.integers(0, 128, size=T)
        sets = groups[gsel].copy()
        sets[unbiased] = -1
        topk, gates = _route(rng, T, E, k, sets, 1.5)
        alt = uniform_contiguous(E, G)
        meta["groups"] = groups
    elif cfg == 5:
        p1 = rng.permutation(E).reshape(32, 2)
        p2 = rng.permutation(E).reshape(32, 2)
        phi = rng.permutation(32)
        c1 = rng.integers(0, 32, size=T)
        keep = rng.random(T) < 0.7
        c2r = rng.integers(0, 32, size=T)
        c2 = np.where(keep, phi[c1], c2r)
        topk, gates = _route(rng, T, E, k, p1[c1], 2.5)
        topk2, gates2 = _route(rng, T, E, k, p2[c2], 2.5)
        er = uniform_contiguous(E, G)
        er2 = uniform_contiguous(E, G)
        meta.update(pairs1=p1, pairs2=p2, phi=phi)
    else:
        raise ValueError(f"unknown workload {cfg}")

    x = _hidden(rng, T, H, c["dtype"]) if with_x else None
    return Workload(cfg=cfg, T=T, H=H, dtype=c["dtype"], E=E, k=k, G=G,
                    ranks_per_node=c["ranks_per_node"], topk=topk, gates=gates,
                    expert_rank=er, alt_expert_rank=alt, x=x, topk2=topk2,
                    gates2=gates2, expert_rank2=er2, meta=meta)
