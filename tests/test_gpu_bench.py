"""bench.py's JSON line on a real device: the fields and their meaning (the
value is dispatched rows per second of the whole step, the roofline's
fraction is its achieved rate over the peak, the CPU baseline names its
sample and threads).  Runs the benchmark as a child process, short."""

import json
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parents[1]


def test_bench_line_contract(built_lib):
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--steps", "20", "--warmup", "2",
                        "--no-expert-side", "--no-copy-probe", "--cpu-sample-tokens", "512"],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    assert d["metric"] == "dispatched rows/s and permute+combine HBM GB/s (% of peak) at 1 MI355X"
    assert d["unit"] == "dispatched rows/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 2
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
