"""Build libmoe_coact.so (HIP, gfx950) in the package directory.

Usage: python -m co_activation_amd.build  (or co_activation_amd.build.build())
Compiles every source under csrc/ with hipcc into _build/ and links the
shared library next to this file; also builds libmoe_hbm_probe.so, the
bandwidth probes the benchmark measures its ceilings with, from probe/.
Always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libmoe_coact.so"
PROBE_SRC = PKG / "probe" / "hbm_probe.hip"
PROBE_LIB = PKG / "libmoe_hbm_probe.so"
ARCH = os.environ.get("MOE_COACT_ARCH", "gfx950")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> Path:
    hipcc = _hipcc()
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))
    inc = ["-I", str(ROOT / "include"), "-I", str(CSRC)]

    def compile_one(src: Path) -> Path:
        obj = BUILD / (src.name + ".o")
        if src.suffix == ".hip":
            cmd = [hipcc, *HIP_FLAGS, *inc, "-c", str(src), "-o", str(obj)]
        else:
            cmd = [hipcc, "-O2", "-std=c++17", "-fPIC", *inc, "-c", str(src), "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB.with_suffix(".so.tmp")
    cmd = [hipcc, *HIP_FLAGS, *inc, "-shared", str(PROBE_SRC), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
