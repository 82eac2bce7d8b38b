#!/usr/bin/env python3
"""Benchmark of the co-activation-aware MoE dispatch path on one MI355X.

One step = one pass of the whole path over one batch:
  workload 5 (default; two MoE layers, T=65536, H=4096 bf16, E=64, k=2, G=8):
    layer-1 co-activation stats (+ transitions) -> shuffle prediction ->
    layer-2 dedup plan over the shuffled order -> the token rows moved to
    their shuffled places and into the layer-2 send rows in one pass ->
    combine
  workloads 1-4: stats -> plan -> permute -> combine of one layer.
Inputs are seeded synthetic routings already resident in HBM when timing
starts.  The timed region runs K batches (default 200, so that filling the
pipeline costs about 1 us per batch) with two in flight: each batch's
routing-only phase (statistics, prediction, plan) runs on a second stream
beside the previous batch's combine (workload 5) or its whole move (k >= 6);
the same K batches run one after another are reported beside it.  Prints ONE
JSON line.  Its value is dispatched rows per second of the whole step (every
stage, batches back to back); permute+combine HBM GB/s with its share of peak
(the metric's second half) and the dominant kernel's roofline fraction ride
along, with the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--placement", default="main", choices=["main", "alt"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536)
    ap.add_argument("--no-copy-probe", action="store_true")
    ap.add_argument("--no-expert-side", action="store_true")
    return ap.parse_args()


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def counter_traffic(workload: int, stage: str):
    """HBM bytes per launch of `stage` from the committed rocprofv3 counter
    summary, or None when there is none or a kernel source changed since the
    counters were taken."""
    import hashlib
    from pathlib import Path

    root = Path(__file__).resolve().parent
    summary = root / "profiles" / f"hbm_counters_workload{workload}.md"
    if not summary.exists():
        return None
    lines = [ln.strip() for ln in summary.read_text().splitlines() if ln.strip().startswith("{")]
    if not lines:
        return None
    rec = json.loads(lines[-1])
    for path, digest in rec["sources"].items():
        if hashlib.sha256((root / path).read_bytes()).hexdigest()[:16] != digest:
            return None
    k = rec["kernels"].get(stage)
    return None if k is None else k["read_bytes"] + k["write_bytes"]


def expert_side(step, w, steps: int, device_normal) -> dict:
    """Destination side after the step's dispatch (outside the timed step):
    expert layout, expansion of the received rows into expert rows, reply
    rows from stand-in expert outputs, the reply combine, and the backward
    mirror of all of it.  Per-kernel times from HIP events, with
    algorithmic bytes."""
    import torch

    from co_activation_amd.pipeline import ExpertSideBackward, ExpertSideStep, StageTimers

    side = ExpertSideStep(step)
    bw = ExpertSideBackward(side)
    y_expert = device_normal(side.T * side.k, w.H, w.dtype, seed=2)
    dy = device_normal(side.T, w.H, w.dtype, seed=3)
    d_expert_in = device_normal(side.T * side.k, w.H, w.dtype, seed=4)

    def once(timers=None):
        side.dispatch(timers)
        side.reply_and_combine(y_expert, timers)
        bw.run(dy, y_expert, d_expert_in, timers)

    once()
    torch.cuda.synchronize()
    timers = StageTimers(side.STAGES + bw.STAGES, steps)
    for _ in range(steps):
        once(timers)
    torch.cuda.synchronize()
    if int(side.d_err.item()) != 0:
        return {"error": f"device data errors {int(side.d_err.item())}"}
    ms = timers.median_ms()
    N = int(step.plan.counters[0].item())
    k = side.k
    TK, rb, T = side.T * k, w.row_bytes, side.T
    # each received row read once, each expert row written once, one index per expert row
    bytes_ = {"expand": N * rb + TK * rb + 4 * TK,
              "partial_combine": TK * rb + 4 * TK + N * rb + 4 * N * k,
              "reply_combine": N * rb + T * rb + 4 * T * k,
              "grad_replies": T * rb + N * rb + 4 * T * k,
              "grad_expert_out": N * rb + TK * rb + 4 * N * k + 4 * TK,
              "grad_gates": T * rb + TK * rb + 8 * TK,
              "grad_send": TK * rb + N * rb + 4 * N * k,
              "grad_tokens": N * rb + T * rb + 4 * T * k}
    out = {"rows_expert": TK, "stage_us": {n: round(1e3 * v, 2) for n, v in ms.items()},
           "gbps": {n: round(b / (ms[n] * 1e-3) / 1e9, 1) for n, b in bytes_.items()},
           "algorithmic_bytes": bytes_}
    return out


def placement_planner(w) -> dict:
    """Co-activation placement for the benchmark's dispatched layer: one
    step of statistics folded into the moving averages, a plan, and the
    rows the dispatch needs under it versus the contiguous split."""
    import numpy as np
    import torch

    from co_activation_amd import ops
    from co_activation_amd.placement import PlacementPlanner

    topk = w.topk2 if w.cfg == 5 else w.topk
    dev = "cuda"
    tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).to(dev)
    planner = PlacementPlanner(w.E, w.G, beta=0.9, eps=0.1, period=1, device=dev)
    st = ops.coact_stats(tk, w.E)
    planner.observe(st)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    er = planner.plan()
    plan_ms = 1e3 * (time.perf_counter() - t0)
    rows = {}
    for name, p in (("contiguous", np.arange(w.E) // (w.E // w.G)), ("planned", er)):
        pl = ops.dispatch_plan(tk, None, torch.from_numpy(np.ascontiguousarray(p, dtype=np.int32))
                               .to(dev), w.G, w.ranks_per_node)
        c = pl.counters.cpu().numpy()
        rows[name] = {"rows": int(c[0]), "local_assign": int(c[3]), "cross_node_V": int(c[5])}
    return {"layer": "layer 2" if w.cfg == 5 else "layer", "beta": 0.9, "eps": 0.1,
            "plan_host_ms": plan_ms, "dispatch": rows,
            "rows_removed_frac": 1.0 - rows["planned"]["rows"] / rows["contiguous"]["rows"]}


def shuffle_modes(w, x, z, steps: int) -> dict:
    """The two-layer step with the free shuffle (shards sized by the
    prediction) and with equal shards: shuffle time, layer-2 local share and
    the largest shard, per mode."""
    import numpy as np
    import torch

    from co_activation_amd.pipeline import StageTimers, TwoLayerStep

    dev = "cuda"

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    out = {}
    for name, bal in (("free", False), ("balanced", True)):
        st = TwoLayerStep(i32(w.topk), i32(w.topk2), torch.from_numpy(w.gates2).to(dev),
                          i32(w.expert_rank2), x, z, w.G, w.ranks_per_node, E1=w.E, balanced=bal)
        st.run()
        timers = StageTimers(("shuffle_predict",), steps)
        for _ in range(steps):
            st.run(timers)
        torch.cuda.synchronize()
        c = st.plan.counters.cpu().numpy()
        off = st.shuffle["shard_offsets"].cpu().numpy()
        out[name] = {"shuffle_predict_us": 1e3 * timers.median_ms()["shuffle_predict"],
                     "local_share": float(c[3]) / (w.T * w.k),
                     "largest_shard": int(np.diff(off).max()), "rows": int(c[0])}
        del st
    return out


def cpu_baseline(w, sample_tokens: int) -> dict:
    """The CPU oracle on the first `sample_tokens` tokens of the same
    workload, single-threaded; rows/s of the same step definition."""
    import numpy as np

    import oracle
    from workloads import expert_outputs

    Ts = max(w.G, (min(sample_tokens, w.T) // w.G) * w.G)
    sl = slice(0, Ts)
    try:  # keep any BLAS call the oracle makes on one thread, as reported
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except ImportError:
        limit = None
    t0 = time.perf_counter()
    if w.cfg == 5:
        res = oracle.two_layer_pipeline(w.topk[sl], w.topk2[sl], w.gates2[sl], w.x[sl],
                                        w.expert_rank2, w.E, w.E, w.G, w.ranks_per_node)
        plan, gates = res["plan"], res["gates2_shuffled"]
    else:
        oracle.coact_stats(w.topk[sl], w.E)
        plan = oracle.dispatch_plan(w.topk[sl], w.gates[sl], w.expert_rank, w.G, w.ranks_per_node)
        oracle.permute_rows(w.x[sl], plan["row_token"])
        gates = w.gates[sl]
    t_mid = time.perf_counter()
    N = int(plan["N"])
    Z = expert_outputs(N, w.H, w.dtype, seed=1)  # input generation, not timed
    t1 = time.perf_counter()
    oracle.combine(Z, w.dtype, plan["slot_row"], gates, w.dtype)
    t2 = time.perf_counter()
    secs = (t_mid - t0) + (t2 - t1)
    if limit is not None:
        limit.restore_original_limits()
    return {"value": N / secs, "unit": "dispatched rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {Ts} of {w.T} tokens of the same workload (full H={w.H}); "
                      f"{N} rows; {secs:.1f} s single-threaded numpy on {_cpu_model()} "
                      f"({os.cpu_count()} host threads visible)"}


def main() -> int:
    args = _args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the engine models "
                                   "the expert-parallel group inside one GPU and has no "
                                   "multi-GPU exchange", "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import co_activation_amd
    from co_activation_amd.pipeline import (ExpertSideStep, GraphPipeline, GraphStep, LayerStep,
                                            Pipeline, StageTimers, TwoLayerStep)
    from workloads import make
    from workloads.gen import device_normal

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no HIP device"}))
        return 1
    if not co_activation_amd.is_built():
        from co_activation_amd.build import build
        build()
    co_activation_amd.lib()

    w = make(args.workload)
    dev = "cuda"

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def xdev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x = xdev(w.x)
    cap = w.T * min(w.k, w.G)
    z = device_normal(cap, w.H, w.dtype, seed=1)
    if w.cfg == 5:
        def make_step(x, z):
            return TwoLayerStep(i32(w.topk), i32(w.topk2), torch.from_numpy(w.gates2).to(dev),
                                i32(w.expert_rank2), x, z, w.G, w.ranks_per_node, E1=w.E)
        workload = (f"two MoE layers with token shuffle: T={w.T} H={w.H} bf16 E={w.E} k={w.k} "
                    f"G={w.G} (1 node of {w.ranks_per_node}); layer-1 stats+transitions, shuffle "
                    f"predict, layer-2 dedup plan, shuffle move fused with the layer-2 permute, "
                    f"combine")
    else:
        er = w.expert_rank if args.placement == "main" else w.alt_expert_rank

        def make_step(x, z):
            return LayerStep(i32(w.topk), torch.from_numpy(w.gates).to(dev), i32(er), x, z, w.G,
                             w.ranks_per_node)
        workload = (f"one MoE layer: T={w.T} H={w.H} {w.dtype} E={w.E} k={w.k} G={w.G} "
                    f"({w.G // w.ranks_per_node} nodes of {w.ranks_per_node}), {args.placement} "
                    f"placement; stats, dedup plan, permute, combine")

    # Attainable copy bandwidth (1 GiB device-to-device), outside the timed region.
    copy_gbs = None
    if not args.no_copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(5):
            e0.record()
            b.copy_(a)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        copy_gbs = 2 * (1 << 30) / (statistics.median(times) * 1e-3) / 1e9
        del a, b

    # Two batches in flight: each step object owns its inputs and outputs.
    step = make_step(x, z)
    step_b = make_step(x.clone(), z.clone())
    pipe = Pipeline([step, step_b])

    pipe.run(max(args.warmup, 2))
    torch.cuda.synchronize()
    for st in (step, step_b):
        if int(st.d_err.item()) != 0:
            print(json.dumps({"error": f"device data errors {int(st.d_err.item())}"}))
            return 1

    # Stage breakdown (events around every stage, all on one stream so that
    # each stage is timed alone), outside the timed region.  Before each step
    # a 512 MiB read evicts the step's data from L2 and the 256 MB Infinity
    # Cache, so every stage starts cold.  (A write would leave dirty lines
    # whose write-back the next stage would pay for.)
    flush = torch.ones(512 << 18, dtype=torch.int32, device=dev)
    stages = StageTimers(step.STAGES, args.steps)
    for _ in range(args.steps):
        flush.sum()
        step.run(stages, overlap=False)
    torch.cuda.synchronize()
    del flush
    stage_ms = stages.median_ms()
    stage_min = {n: min(stages.durations_ms(n)) for n in stage_ms}
    stage_p90 = {n: float(np.percentile(stages.durations_ms(n), 90)) for n in stage_ms}
    moves = ("shuffle_dispatch",) if "shuffle_dispatch" in stage_ms else ("permute",)
    dom = max(moves + ("combine",), key=lambda n: stage_ms[n])

    # Timed region: K batches through the two-step pipeline (each batch's
    # routing-only phase beside the previous batch's combine); events only
    # around the dominant kernel.
    timers = StageTimers((dom,), args.steps)
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e_start.record()
    pipe.run(args.steps, timers)
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = e_start.elapsed_time(e_end)
    ms_per_step = gpu_ms / args.steps
    dom_all = timers.durations_ms(dom)
    dom_ms = statistics.mean(dom_all)
    for st in (step, step_b):
        if int(st.d_err.item()) != 0:
            print(json.dumps({"error": f"device data errors {int(st.d_err.item())}"}))
            return 1

    # The same K batches one after another on one step (no batch overlap).
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record()
    for _ in range(args.steps):
        step.run()
    s1.record()
    torch.cuda.synchronize()
    seq_ms = s0.elapsed_time(s1) / args.steps

    # The same step captured once as a HIP graph and replayed (outside the
    # timed region above): the host enqueues one launch per step.
    graph = GraphStep(step)
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record()
    for _ in range(args.steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graph

    # The pipeline captured as a graph of ten batches and replayed: what a
    # caller whose host paces the eager loop (small layers) would use.
    gbatches = 10
    gpipe = GraphPipeline(pipe, gbatches)
    reps = max(1, args.steps // gbatches)
    torch.cuda.synchronize()
    g0.record()
    for _ in range(reps):
        gpipe.replay()
    g1.record()
    torch.cuda.synchronize()
    gpipe_ms = g0.elapsed_time(g1) / (reps * gbatches)
    del gpipe

    counters = step.plan.counters.cpu().numpy()
    N = int(counters[0])
    T, k = w.T, w.k
    rb = w.row_bytes
    bytes_perm = (T + N) * rb + 4 * T * k
    bytes_comb = N * rb + T * rb + 4 * T * k + 4 * N
    kernels = {"permute": bytes_perm, "combine": bytes_comb}
    # the shuffle's move fused with the layer-2 permute: each row read once,
    # written to its shuffled place and its send rows; dest_pos and token_rows
    kernels["shuffle_dispatch"] = (2 * T + N) * rb + 4 * T + 4 * T * k
    mv = moves[0]
    pc_gbs = (kernels[mv] + bytes_comb) / ((stage_ms[mv] + stage_ms["combine"]) * 1e-3) / 1e9
    achieved = kernels[dom] / (dom_ms * 1e-3) / 1e9
    achieved_alone = kernels[dom] / (stage_ms[dom] * 1e-3) / 1e9

    line = {
        "metric": "dispatched rows/s and permute+combine HBM GB/s (% of peak) at 1 MI355X",
        "value": N / (ms_per_step * 1e-3),
        "unit": "dispatched rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded router logits, N(0,1) rows)",
        "config": {"workload": workload, "tokens": T, "hidden": w.H, "experts": w.E, "top_k": k,
                   "logical_ranks": w.G, "dispatched_rows": N},
        "dispatched_rows_per_s_of_move_kernel": N / (stage_ms[mv] * 1e-3),
        "permute_combine_gbps": pc_gbs,
        "permute_combine_pct_of_hbm_peak": 100.0 * pc_gbs / HBM_PEAK_GBS,
        "stage_us_median": {n: 1e3 * v for n, v in stage_ms.items()},
        "stage_us_min": {n: 1e3 * v for n, v in stage_min.items()},
        "stage_us_p90": {n: 1e3 * v for n, v in stage_p90.items()},
        "stage_gbps": {n: b / (stage_ms[n] * 1e-3) / 1e9
                       for n, b in ((mv, kernels[mv]), ("combine", bytes_comb))},
        "schedule": ("two batches in flight: each batch's " +
                     ("statistics and plan" if w.cfg != 5 else
                      "statistics, shuffle prediction and layer-2 plan") +
                     " on a second stream beside the previous batch's " +
                     ("combine" if pipe.beside == "combine" else "permute and combine")),
        "counters": {"rows": N, "assignments": int(counters[1]), "local_rows": int(counters[2]),
                     "local_assign": int(counters[3]), "node_rows": int(counters[4]),
                     "cross_node_V": int(counters[5]), "max_recv_rows": int(counters[6])},
        "copy_probe_gbps": copy_gbs,
        "wall_s_timed": wall,
        "sequential": {"ms_per_step": seq_ms, "dispatched_rows_per_s": N / (seq_ms * 1e-3)},
        "graph_replay": {"ms_per_step": graph_ms,
                         "dispatched_rows_per_s": int(counters[0]) / (graph_ms * 1e-3)},
        "graph_pipeline": {"batches_per_graph": gbatches, "ms_per_step": gpipe_ms,
                           "dispatched_rows_per_s": N / (gpipe_ms * 1e-3)},
        "roofline": {"bound": "hbm", "kernel": dom, "kernel_us": 1e3 * dom_ms,
                     "kernel_us_median": 1e3 * statistics.median(dom_all),
                     "algorithmic_bytes": kernels[dom], "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(w.cfg, dom),
                     "kernel_us_alone": 1e3 * stage_ms[dom],
                     "frac_alone": achieved_alone / HBM_PEAK_GBS},
    }
    if not args.no_expert_side:
        line["expert_side"] = expert_side(step, w, args.steps, device_normal)
        line["placement"] = placement_planner(w)
        if w.cfg == 5:
            line["shuffle_modes"] = shuffle_modes(w, x, z, args.steps)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
