"""Helpers shared by the GPU tests: host <-> device moves and the comparison
rules (bit-exact integers, fp32 bound, bf16 ulp bound)."""

import sys

import numpy as np
import torch

import oracle

DEV = "cuda"


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run names it."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def i32(a) -> torch.Tensor:
    return dev(np.asarray(a, dtype=np.int32))


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def x_tensor(w) -> torch.Tensor:
    return dev(w.x)


def assert_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} mismatches, first at {bad[:5]}: "
                           f"got {got.reshape(-1)[bad[:5]]} want {want.reshape(-1)[bad[:5]]}")


def f32_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in float32 units in the last place (same-sign ordering)."""
    def key(x):
        i = np.asarray(x, np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(key(a) - key(b))


def bf16_ulps(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    def key(x):
        i = np.asarray(x, np.uint16).astype(np.int64)
        return np.where(i & 0x8000, -(i & 0x7FFF), i)
    return np.abs(key(a_bits) - key(b_bits))


def combine_scale(Z, z_dtype, slot_row, gates):
    """sum_j |w_tj| |Z[slot_row[t, j]]| per element: the size of the terms."""
    Zf = oracle.bf16_to_f32(Z) if z_dtype == "bf16" else np.asarray(Z, np.float32)
    scale = np.zeros((slot_row.shape[0], Zf.shape[1]), np.float64)
    for j in range(slot_row.shape[1]):
        scale += np.abs(gates[:, j:j + 1].astype(np.float64)) * np.abs(Zf[slot_row[:, j]])
    return scale


# Elements held to the fp32 bound instead of 1 bf16 ulp (cancellation), per
# check: (what, count, elements).  Reported by the tests that gather them.
FALLBACKS = []


def check_combine(y_gpu: torch.Tensor, Z: np.ndarray, z_dtype: str, slot_row: np.ndarray,
                  gates: np.ndarray, out_dtype: str, what=""):
    """check_combine_host on the device output y_gpu; returns it on the host."""
    y = host(y_gpu)
    check_combine_host(y, Z, z_dtype, slot_row, gates, out_dtype, what)
    return y


def check_combine_host(y: np.ndarray, Z: np.ndarray, z_dtype: str, slot_row: np.ndarray,
                       gates: np.ndarray, out_dtype: str, what=""):
    """fp32 output: |y - y_ref| <= 1e-5 * sum_j |w_tj| |Z_row| per element.
    bf16 output: within 1 bf16 ulp of the oracle's fp32 result rounded once;
    where the weighted sum cancels no fp32 accumulation order can promise
    that, and the element is held to the fp32 bound instead -- only where the
    sum is at least 2^7 times smaller than its terms' magnitude
    sum_j |w_tj| |Z_row| (a rounding error of the kernel's fp32 sum, at most a
    few 2^-24 of that magnitude, can exceed 1 bf16 ulp of the result only
    there).  The number of such elements is recorded in FALLBACKS.  Plain
    numpy: safe to run on several threads at once."""
    ref32 = oracle.combine(Z, z_dtype, slot_row, gates, "f32")
    scale = combine_scale(Z, z_dtype, slot_row, gates)
    if out_dtype == "f32":
        err = np.abs(y.astype(np.float64) - ref32.astype(np.float64))
        ok = err <= 1e-5 * scale + 1e-30
        assert ok.all(), f"{what}: {np.count_nonzero(~ok)} elements outside 1e-5 relative"
    else:
        ref = oracle.bf16_round(ref32)
        d = bf16_ulps(y, ref)
        yf = oracle.bf16_to_f32(y).astype(np.float64)
        near = np.abs(yf - ref32.astype(np.float64)) <= 1e-5 * scale
        ok = (d <= 1) | near
        assert ok.all(), (f"{what}: {np.count_nonzero(~ok)} elements beyond 1 bf16 ulp and "
                          f"the fp32 bound; worst {d[~ok].max()} ulp")
        fb = d > 1
        n_fb = int(np.count_nonzero(fb))
        if n_fb:
            assert (np.abs(yf[fb]) <= 2.0 ** -7 * scale[fb]).all(), (
                f"{what}: an element beyond 1 bf16 ulp whose sum does not cancel")
        FALLBACKS.append((what, n_fb, int(d.size)))
