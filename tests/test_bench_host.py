"""bench.py's command-line contract on a machine without a GPU: more than one
GPU (by flag or by a launcher's WORLD_SIZE) is refused with a JSON message and
exit status 2, before anything touches a device; without a HIP device the one
line it prints is a JSON error, not a traceback."""

import json
import os
import subprocess
import sys
from pathlib import Path

import pytest
import torch

ROOT = Path(__file__).resolve().parents[1]


def _bench(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    return r.returncode, lines


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      (["--gpus", "2"], {"WORLD_SIZE": "2"}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    rc, lines = _bench(args, env)
    assert rc == 2
    assert len(lines) == 1
    msg = json.loads(lines[0])
    assert "error" in msg and "one GPU" in msg["error"]


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a machine without a HIP device")
def test_without_a_device_the_line_is_a_json_error():
    rc, lines = _bench(["--steps", "1", "--warmup", "0", "--no-cpu-baseline"])
    assert rc == 1
    assert len(lines) == 1
    assert "error" in json.loads(lines[0])
