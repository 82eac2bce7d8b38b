"""bench.py's JSON line on a real device: the fields and their meaning (the
value is dispatched rows per second of the whole step, the roofline's
fraction is its achieved rate over the peak, the CPU baseline names its
sample and threads), and the per-workload records and measured ceilings the
default run adds.  Runs the benchmark as a child process, short."""

import json
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parents[1]


def test_bench_line_contract(built_lib):
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--steps", "10", "--warmup", "2",
                        "--no-expert-side", "--cpu-sample-tokens", "512"],
                       cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    assert d["metric"] == "dispatched rows/s and permute+combine HBM GB/s (% of peak) at 1 MI355X"
    assert d["unit"] == "dispatched rows/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 10 and d["warmup"] == 2
    assert d["scaling"] == "weak" and d["vs_baseline"] is None and d["dtype"] == "bf16"
    assert "workload" in d["config"] and "model" not in d["config"]
    N = d["config"]["dispatched_rows"]
    assert N == d["counters"]["rows"] > 0
    assert d["value"] == pytest.approx(N / (d["ms_per_step"] * 1e-3), rel=1e-9)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["kernel"] == "shuffle_dispatch"
    assert rf["achieved"] == pytest.approx(rf["algorithmic_bytes"] / (rf["kernel_us"] * 1e-6) / 1e9)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert 0.3 < rf["frac"] < 1.0
    assert rf["traffic"] is None or 0.9 < rf["traffic"] / rf["algorithmic_bytes"] < 1.2
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0
    assert cb["unit"] == d["unit"] and "512" in cb["sample"]
    # measured ceilings, and the dominant kernel placed against its read/write mix
    g = d["ceilings"]["gbps"]
    for key in ("read", "write", "copy"):
        assert 1000 < g[key] < 8000, (key, g[key])
    assert rf["mix_bound_us"] == pytest.approx(
        (rf["read_bytes"] / (g["read"] * 1e9) + rf["write_bytes"] / (g["write"] * 1e9)) * 1e6)
    assert rf["read_bytes"] + rf["write_bytes"] == rf["algorithmic_bytes"]
    assert 0.3 < rf["frac_of_mix_bound"] < 1.05
    for f in range(1, 9):
        assert 1000 < g[f"fanout{f}"] < 8000, (f, g[f"fanout{f}"])
        assert 1000 < g[f"fanin{f}"] < 8000, (f, g[f"fanin{f}"])
    # the fused dispatch writes about 2.8x what it reads: inside the fan-out probe's range
    assert rf["same_mix_bound_us"] > 0 and 0.3 < rf["frac_of_same_mix_bound"] < 1.1
    fr = d["stage_frac_of_same_mix_bound"]
    assert set(fr) == {"shuffle_dispatch", "combine"} and all(0.3 < v < 1.1 for v in fr.values())
    # workloads 1-4 beside the headline, each measured the same way
    ws = d["workloads"]
    assert sorted(ws) == ["1", "2", "3", "4"]
    for key, o in ws.items():
        n = o["counters"]["rows"]
        assert o["value"] == pytest.approx(n / (o["ms_per_step"] * 1e-3), rel=1e-9)
        assert o["config"]["dispatched_rows"] == n
        assert o["roofline"]["kernel"] in ("permute", "combine")
        assert o["roofline"]["frac"] == pytest.approx(o["roofline"]["achieved"] / 8000.0)
        assert o["cpu_baseline"]["kind"] == "oracle" and o["cpu_baseline"]["value"] > 0
        if key != "1":
            assert "alt_placement" in o and o["alt_placement"]["counters"]["rows"] > 0
    assert ws["3"]["counters"]["cross_node_V"] > 0 and ws["4"]["counters"]["cross_node_V"] > 0
    assert ws["1"]["counters"]["cross_node_V"] == 0 and ws["2"]["counters"]["cross_node_V"] == 0
