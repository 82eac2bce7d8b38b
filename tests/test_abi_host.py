"""CPU-side checks of the C ABI: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host (negative status,
nothing enqueued, no HIP call made)."""

import ctypes
import re
from pathlib import Path

import pytest

from co_activation_amd import _lib

HEADER = Path(__file__).resolve().parents[1] / "include" / "moe_coact.h"

NULL = None
FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on these paths


def _declared():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_and_exports_agree(built_lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(built_lib, n), n


def test_status_strings(built_lib):
    for code in _lib.STATUS:
        assert built_lib.moe_status_string(code)
    assert built_lib.moe_status_string(12345) == b"unknown status"


def test_workspace_queries(built_lib):
    n = ctypes.c_size_t()
    assert built_lib.moe_dispatch_plan_workspace_size(65536, 8, ctypes.byref(n)) == 0
    assert n.value >= (65536 // 256 + 8) * (8 + 4) * 4 and n.value % 256 == 0
    assert built_lib.moe_dispatch_plan_workspace_size(10, 65, ctypes.byref(n)) == -2
    assert built_lib.moe_dispatch_plan_workspace_size(10, 8, None) == -1
    assert built_lib.moe_shuffle_predict_workspace_size(4096, 64, 8, ctypes.byref(n)) == 0
    assert n.value > 4096 * 4
    assert built_lib.moe_shuffle_predict_workspace_size(4096, 257, 8, ctypes.byref(n)) == -2


def test_stats_rejects(built_lib):
    f = built_lib.moe_coact_stats
    W = (FAKE, 1 << 24, NULL)  # workspace, its bytes, stream
    assert f(FAKE, 10, 9, 8, NULL, 0, 0, FAKE, NULL, NULL, NULL, NULL, *W) == -2  # k > 8
    assert f(FAKE, 10, 2, 257, NULL, 0, 0, FAKE, NULL, NULL, NULL, NULL, *W) == -2  # E > 256
    assert f(FAKE, -1, 2, 8, NULL, 0, 0, FAKE, NULL, NULL, NULL, NULL, *W) == -2
    assert f(FAKE, 10, 2, 8, NULL, 0, 0, NULL, NULL, NULL, NULL, NULL, *W) == -1  # counts
    assert f(FAKE, 10, 2, 8, NULL, 0, 0, FAKE, NULL, FAKE, NULL, NULL, *W) == -1  # ochiai w/o pairs
    assert f(FAKE, 10, 2, 8, NULL, 2, 8, FAKE, NULL, NULL, FAKE, NULL, *W) == -1  # no topk_next
    assert f(FAKE, 10, 2, 8, FAKE, 0, 8, FAKE, NULL, NULL, FAKE, NULL, *W) == -2  # k_next 0
    assert f(FAKE, 2**30, 2, 8, NULL, 0, 0, FAKE, NULL, NULL, NULL, NULL, *W) == -2  # T*k
    assert f(FAKE, 10, 2, 8, NULL, 0, 0, FAKE, FAKE, NULL, NULL, NULL, NULL, 1 << 24, NULL) == -1
    assert f(FAKE, 10, 2, 8, NULL, 0, 0, FAKE, FAKE, NULL, NULL, NULL, FAKE + 4, 1 << 24,
             NULL) == -4                                                          # alignment
    n = ctypes.c_size_t()
    assert built_lib.moe_coact_stats_workspace_size(10, 8, 1, 0, ctypes.byref(n)) == 0
    assert f(FAKE, 10, 2, 8, NULL, 0, 0, FAKE, FAKE, NULL, NULL, NULL, FAKE, n.value - 16,
             NULL) == -5                                                          # too small


def test_stats_workspace_sizes(built_lib):
    """Up to 128 splits of at least 256 tokens; each split holds a partial of
    the counted bins (the pair triangle i <= j, the transitions) as 16-bit
    counters while a split has fewer than 2^16 tokens, else 32-bit, each
    slice of rows padded to 16 bytes and each split's row to an odd number of
    256-byte units."""
    n = ctypes.c_size_t()
    q = built_lib.moe_coact_stats_workspace_size

    def within(splits, bins, bytes_per_bin, slices):
        lo = splits * bins * bytes_per_bin
        return lo <= n.value <= lo + splits * (slices * 16 + 512) + 256

    assert q(32768, 256, 1, 0, ctypes.byref(n)) == 0
    assert within(128, 256 * 257 // 2, 2, 3)                  # 128 splits of 256 tokens
    assert q(65536, 64, 1, 64, ctypes.byref(n)) == 0
    assert within(128, 64 * 65 // 2 + 64 * 64, 2, 2)          # pairs and transitions
    assert q(2048, 8, 0, 0, ctypes.byref(n)) == 0
    assert within(8, 8, 2, 1)
    assert q(1 << 24, 8, 0, 0, ctypes.byref(n)) == 0
    assert n.value == 128 * 256                               # 2^17 tokens a split: 32-bit,
    assert q(0, 8, 1, 0, ctypes.byref(n)) == 0 and n.value >= 36 * 2  # one 256-byte row
    assert q(10, 257, 1, 0, ctypes.byref(n)) == -2
    assert q(10, 8, 1, 0, None) == -1


def _plan(lib, **kw):
    a = dict(topk=FAKE, gates=NULL, T=64, k=2, E=8, er=FAKE, G=4, Rn=4, src=NULL, cap=128,
             sc=FAKE, so=FAKE, rt=FAKE, rw=NULL, tr=FAKE, sr=NULL, cn=FAKE, derr=NULL, ws=FAKE,
             wsb=1 << 20)
    a.update(kw)
    return lib.moe_dispatch_plan(a["topk"], a["gates"], a["T"], a["k"], a["E"], a["er"], a["G"],
                                 a["Rn"], a["src"], a["cap"], a["sc"], a["so"], a["rt"], a["rw"],
                                 a["tr"], a["sr"], a["cn"], a["derr"], a["ws"], a["wsb"], NULL)


def test_plan_rejects(built_lib):
    L = built_lib
    assert _plan(L, G=65) == -2
    assert _plan(L, G=0) == -2
    assert _plan(L, Rn=3) == -2          # does not divide G
    assert _plan(L, T=63) == -2          # equal shards need T % G == 0
    assert _plan(L, k=0) == -2
    assert _plan(L, E=300) == -2
    assert _plan(L, cap=-1) == -2
    assert _plan(L, er=NULL) == -1
    assert _plan(L, ws=NULL) == -1
    assert _plan(L, tr=NULL) == -1
    assert _plan(L, rt=NULL) == -1
    assert _plan(L, ws=FAKE + 4) == -4   # workspace alignment
    assert _plan(L, wsb=16) == -5        # workspace too small


def test_noalloc_plan_rejects(built_lib):
    """The allocation-free plan checks its arguments like the workspace plan
    and refuses inputs whose per-tile scratch exceeds its fixed array, all
    before any HIP call."""
    L = built_lib
    f = L.moe_dispatch_plan_noalloc

    def call(T=64, k=2, E=8, G=4, Rn=4, er=FAKE, tr=FAKE, cap=128):
        return f(FAKE, NULL, T, k, E, er, G, Rn, NULL, cap, FAKE, FAKE, FAKE, NULL, tr, NULL, FAKE,
                 NULL, NULL)
    assert call(G=65) == -2
    assert call(Rn=3) == -2
    assert call(T=63) == -2
    assert call(er=NULL) == -1
    assert call(tr=NULL) == -1
    limit = _lib.NOALLOC_SCRATCH_BYTES
    n = ctypes.c_size_t()
    for T, G in ((3_931_136, 64), (4_000_000, 64), (22_367_488, 8), (22_400_000, 8)):
        assert L.moe_dispatch_plan_workspace_size(T, G, ctypes.byref(n)) == 0
        if n.value > limit:
            assert call(T=T, k=1, E=G, G=G, Rn=G, cap=T) == -5   # beyond the scratch array
        else:
            assert T in (3_931_136, 22_367_488)                  # the largest that fit


def test_gathered_plan_rejects(built_lib):
    L = built_lib
    f = L.moe_dispatch_plan_gathered
    # topk, gates, perm, T, k, E, er, G, Rn, src, cap, sc, so, rt, rw, tr, sr, cn,
    # topk_out, gates_out, d_err, ws, ws_bytes, stream
    base = [FAKE, FAKE, FAKE, 64, 2, 8, FAKE, 4, 4, NULL, 128, FAKE, FAKE, FAKE, FAKE, FAKE, NULL,
            FAKE, FAKE + 4096, FAKE + 8192, NULL, FAKE, 1 << 20, NULL]
    def call(**kw):
        a = list(base)
        idx = {"perm": 2, "T": 3, "k": 4, "topk_out": 18, "gates_out": 19, "ws_bytes": 22}
        for key, v in kw.items():
            a[idx[key]] = v
        return f(*a)
    assert call(perm=NULL) == -1                  # no order
    assert call(topk_out=NULL) == -1              # nowhere to put the routing
    assert call(gates_out=NULL) == -1             # gates given, no gates_out
    assert call(topk_out=FAKE) == -2              # in place
    assert call(gates_out=FAKE) == -2             # in place
    assert call(k=9) == -2
    assert call(ws_bytes=16) == -5


def test_permute_combine_shuffle_reject(built_lib):
    L = built_lib
    assert L.moe_permute(FAKE, 8, 0, FAKE, 1, FAKE, 8, NULL, NULL, NULL) == -2
    assert L.moe_permute(FAKE, 8, 16, FAKE, 9, FAKE, 8, NULL, NULL, NULL) == -2
    assert L.moe_permute(FAKE, 8, 6, FAKE, 1, FAKE, 8, NULL, NULL, NULL) == -4
    assert L.moe_permute(FAKE + 2, 8, 16, FAKE, 1, FAKE, 8, NULL, NULL, NULL) == -4
    assert L.moe_permute(NULL, 8, 16, FAKE, 1, FAKE, 8, NULL, NULL, NULL) == -1
    assert L.moe_permute(NULL, 0, 16, NULL, 1, NULL, 0, NULL, NULL, NULL) == 0   # empty: no-op
    sdp = L.moe_shuffle_dispatch
    assert sdp(FAKE, 8, 16, FAKE, FAKE, 9, FAKE, FAKE, 16, NULL, NULL) == -2   # k > 8
    assert sdp(FAKE, 8, 0, FAKE, FAKE, 2, FAKE, FAKE, 16, NULL, NULL) == -2    # row_bytes
    assert sdp(FAKE, 8, 16, NULL, FAKE, 2, FAKE, FAKE, 16, NULL, NULL) == -1   # dest_pos
    assert sdp(FAKE, 8, 6, FAKE, FAKE, 2, FAKE, FAKE, 16, NULL, NULL) == -4    # not whole words
    assert sdp(NULL, 0, 16, NULL, NULL, 2, NULL, NULL, 0, NULL, NULL) == 0     # empty: no-op
    g = L.moe_gather
    assert g(FAKE, 8, 0, FAKE, 8, FAKE, NULL, NULL, NULL) == -2     # row_bytes
    assert g(FAKE, -1, 16, FAKE, 8, FAKE, NULL, NULL, NULL) == -2   # x_rows
    assert g(FAKE, 8, 16, FAKE, 1 << 31, FAKE, NULL, NULL, NULL) == -2
    assert g(FAKE, 8, 6, FAKE, 8, FAKE, NULL, NULL, NULL) == -4     # not whole words
    assert g(FAKE, 8, 16, FAKE, 8, FAKE + 2, NULL, NULL, NULL) == -4
    assert g(FAKE, 8, 16, NULL, 8, FAKE, NULL, NULL, NULL) == -1    # src
    assert g(NULL, 8, 16, FAKE, 8, FAKE, NULL, NULL, NULL) == -1    # x
    assert g(NULL, 0, 16, NULL, 0, NULL, NULL, NULL, NULL) == 0     # empty: no-op
    # launches of 2^32 or more work-items are refused before anything runs
    big = 1 << 24
    assert L.moe_permute(FAKE, big, 4096, FAKE, 1, FAKE, big, NULL, NULL, NULL) == -2
    assert L.moe_permute(FAKE, big // 2, 16384, FAKE, 2, FAKE, big, NULL, NULL, NULL) == -2
    assert sdp(FAKE, big // 2, 8192, FAKE, FAKE, 2, FAKE, FAKE, big, NULL, NULL) == -2
    assert g(FAKE, big, 8192, FAKE, big // 2, FAKE, NULL, NULL, NULL) == -2
    assert L.moe_combine(FAKE, 1, big, 1 << 20, FAKE, 2, NULL, big // 64, FAKE, 1, NULL, NULL,
                         NULL) == -2
    assert L.moe_combine(FAKE, 7, 8, 64, FAKE, 2, NULL, 8, FAKE, 1, NULL, NULL, NULL) == -3
    assert L.moe_combine(FAKE, 1, 8, 60, FAKE, 2, NULL, 8, FAKE, 1, NULL, NULL, NULL) == -4  # 120 B
    assert L.moe_combine(FAKE, 1, 8, 64, FAKE, 0, NULL, 8, FAKE, 1, NULL, NULL, NULL) == -2
    assert L.moe_combine(FAKE, 1, 8, 64, NULL, 2, NULL, 8, FAKE, 1, NULL, NULL, NULL) == -1
    assert L.moe_combine(FAKE + 8, 1, 8, 64, FAKE, 2, NULL, 8, FAKE, 1, NULL, NULL, NULL) == -4
    ep = L.moe_expert_plan
    args = [FAKE, NULL, 64, 2, 8, FAKE, 4, FAKE, 128, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL,
            FAKE, NULL, FAKE, 1 << 20, NULL]
    assert ep(*args[:3], 9, *args[4:]) == -2                       # k > 8
    assert ep(*args[:6], 65, *args[7:]) == -2                      # G > 64
    assert ep(*args[:7], NULL, *args[8:]) == -1                    # slot_row
    assert ep(*args[:16], NULL, *args[17:]) == -1                  # row_dest
    assert ep(*args[:19], 16, NULL) == -5                          # workspace
    n = ctypes.c_size_t()
    assert L.moe_expert_plan_workspace_size(65536, 256, ctypes.byref(n)) == 0
    assert n.value >= 256 * 256 * 4
    ps = L.moe_permute_scaled
    assert ps(FAKE, 2, 8, 64, FAKE, 1, FAKE, FAKE, 1, 8, NULL, NULL, NULL) == -3
    assert ps(FAKE, 1, 8, 64, FAKE, 9, FAKE, FAKE, 1, 8, NULL, NULL, NULL) == -2
    assert ps(FAKE, 1, 8, 64, FAKE, 1, NULL, FAKE, 1, 8, NULL, NULL, NULL) == -1
    assert ps(FAKE, 1, 8, 60, FAKE, 1, FAKE, FAKE, 1, 8, NULL, NULL, NULL) == -4
    rd = L.moe_row_dot
    assert rd(FAKE, 1, 8, 64, FAKE, 5, 8, FAKE, 1, FAKE, NULL, NULL, NULL) == -3
    assert rd(FAKE, 1, 8, 64, FAKE, 1, 8, FAKE, 0, FAKE, NULL, NULL, NULL) == -2
    assert rd(FAKE, 1, 8, 64, FAKE, 1, 8, NULL, 1, FAKE, NULL, NULL, NULL) == -1
    assert rd(FAKE, 0, 8, 4, FAKE, 1, 8, FAKE, 1, FAKE, NULL, NULL, NULL) == -4  # bf16 side, H=4
    sp = L.moe_shuffle_predict
    assert sp(FAKE, 8, 2, 8, FAKE, 8, FAKE, 65, FAKE, FAKE, NULL, FAKE, NULL, FAKE, 1 << 20, NULL) == -2
    assert sp(FAKE, 8, 2, 8, NULL, 8, FAKE, 4, FAKE, FAKE, NULL, FAKE, NULL, FAKE, 1 << 20, NULL) == -1
    assert sp(FAKE, 8, 2, 8, FAKE, 8, FAKE, 4, FAKE, FAKE, NULL, FAKE, NULL, FAKE + 16, 1 << 20, NULL) == -4
    assert sp(FAKE, 8, 2, 8, FAKE, 8, FAKE, 4, FAKE, FAKE, NULL, FAKE, NULL, FAKE, 64, NULL) == -5


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No CPU fallback: without the built library every call raises."""
    monkeypatch.setattr(_lib, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_binding_rejects_a_stream_of_another_device(monkeypatch):
    """The binding hands the kernels the current stream; tensors on another
    device than that stream's are refused before any call."""
    import types

    import torch

    from co_activation_amd import ops

    streams = {1: types.SimpleNamespace(cuda_stream=0x1234)}
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 1)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda idx=None: streams[idx])
    assert ops._stream(types.SimpleNamespace(device=torch.device("cuda", 1))) == 0x1234
    with pytest.raises(ValueError, match="current device"):
        ops._stream(types.SimpleNamespace(device=torch.device("cuda", 0)))


def test_probe_library_rejects(built_lib):
    """The bandwidth-probe library (include/moe_hbm_probe.h) loads and checks
    its arguments on the host before any launch."""
    from co_activation_amd import hbm_probe
    f = hbm_probe._load().moe_probe_stream
    assert f(3, 0, FAKE, FAKE, 1024, FAKE, NULL) == -2       # no such mode
    assert f(0, 4, FAKE, FAKE, 1024, FAKE, NULL) == -2       # no such shape
    assert f(2, 0, FAKE, FAKE, 1000, FAKE, NULL) == -2       # not a multiple of 16 bytes
    assert f(2, 0, FAKE, FAKE, 0, FAKE, NULL) == -2
    assert f(0, 0, NULL, FAKE, 1024, FAKE, NULL) == -1       # read needs src
    assert f(0, 0, FAKE, NULL, 1024, NULL, NULL) == -1       # read needs sink
    assert f(1, 0, NULL, NULL, 1024, NULL, NULL) == -1       # write needs dst
    assert f(2, 0, FAKE + 8, FAKE, 1024, NULL, NULL) == -4   # alignment
    g = hbm_probe._load().moe_probe_fanout
    D = FAKE + 4096
    assert g(4, FAKE, D, 1024, 1024, 2, 0, NULL) == -2   # no such shape
    assert g(0, FAKE, D, 1024, 1024, 0, 0, NULL) == -2   # fan-out below 1
    assert g(0, FAKE, D, 1024, 1024, 65, 0, NULL) == -2  # fan-out above 64
    assert g(0, FAKE, D, 1024, 1024, 2, 1, NULL) == -2   # cap of one block
    assert g(0, FAKE, D, 1024, 1024, 2, 33, NULL) == -2  # cap above 32
    assert g(0, FAKE, D, 1000, 1008, 2, 0, NULL) == -2   # not a multiple of 16 bytes
    assert g(0, FAKE, D, 1024, 1008, 2, 0, NULL) == -2   # regions would overlap
    assert g(0, FAKE, D, 1024, 1032, 2, 0, NULL) == -2   # stride not a multiple of 16
    assert g(0, NULL, FAKE, 1024, 1024, 2, 0, NULL) == -1
    assert g(0, FAKE, NULL, 1024, 1024, 2, 0, NULL) == -1
    assert g(0, FAKE, FAKE + 4100, 1024, 1024, 2, 0, NULL) == -4   # alignment
    h = hbm_probe._load().moe_probe_fanin  # (shape, src, stride, dst, bytes, fan, cap, stream)
    assert h(4, D, 1024, FAKE, 1024, 2, 0, NULL) == -2   # no such shape
    assert h(0, D, 1024, FAKE, 1024, 0, 0, NULL) == -2   # fan-in below 1
    assert h(0, D, 1008, FAKE, 1024, 2, 0, NULL) == -2   # regions would overlap
    assert h(0, D, 1024, FAKE, 1024, 2, 1, NULL) == -2   # cap of one block
    assert h(0, NULL, 1024, FAKE, 1024, 2, 0, NULL) == -1
    assert h(0, D, 1024, NULL, 1024, 2, 0, NULL) == -1
    assert h(0, D + 4, 1024, FAKE, 1024, 2, 0, NULL) == -4  # alignment


def test_fanout_bound_arithmetic():
    """fanout_bound_us: at a whole fan-out it is the probe's own time for the
    same bytes, between two it is linear in the time per byte read; the
    fan-in bound mirrors it, and the same-mix bound picks by direction."""
    from co_activation_amd.hbm_probe import fanin_bound_us, fanout_bound_us, same_mix_bound_us
    g = {f"fanout{f}": 6000.0 - 100 * f for f in range(1, 9)}
    g.update({f"fanin{f}": 7000.0 - 50 * f for f in range(1, 9)})
    ceil = {"gbps": g}
    W = 2e8
    assert fanin_bound_us(5 * W, W, ceil) == pytest.approx(6 * W / (g["fanin5"] * 1e9) * 1e6)
    assert same_mix_bound_us(5 * W, W, ceil) == fanin_bound_us(5 * W, W, ceil)
    assert same_mix_bound_us(W, 5 * W, ceil) == fanout_bound_us(W, 5 * W, ceil)
    R = 1e9
    assert fanout_bound_us(R, 3 * R, ceil) == pytest.approx(4 * R / (g["fanout3"] * 1e9) * 1e6)
    assert fanout_bound_us(R, 8 * R, ceil) == pytest.approx(9 * R / (g["fanout8"] * 1e9) * 1e6)
    lo = fanout_bound_us(R, 3 * R, ceil)
    hi = fanout_bound_us(R, 4 * R, ceil)
    assert fanout_bound_us(R, 3.25 * R, ceil) == pytest.approx(lo + 0.25 * (hi - lo))
    assert fanout_bound_us(R, 0.5 * R, ceil) is None and fanout_bound_us(R, 9 * R, ceil) is None


def test_overlapping_outputs_rejected(built_lib):
    """An output sharing bytes with an input is refused with MOE_ERR_SHAPE
    before any launch (blocks would read rows others already overwrote)."""
    L = built_lib
    RB = 256  # row bytes
    # permute: x = 8 rows at FAKE, out = 8 rows starting inside x
    assert L.moe_permute(FAKE, 8, RB, FAKE + 8192, 1, FAKE + 4 * RB, 8, NULL, NULL, NULL) == -2
    assert L.moe_permute(FAKE, 8, RB, FAKE + 8192, 1, FAKE, 8, NULL, NULL, NULL) == -2  # in place
    # gather: out ends inside x
    assert L.moe_gather(FAKE + 2 * RB, 8, RB, FAKE + 8192, 4, FAKE, NULL, NULL, NULL) == -2
    # shuffle dispatch: x_out over x, send over x, send over x_out
    sd = L.moe_shuffle_dispatch
    big = FAKE + (1 << 20)
    assert sd(FAKE, 8, RB, big, big + 64, 2, FAKE, big + 4096, 16, NULL, NULL) == -2
    assert sd(FAKE, 8, RB, big, big + 64, 2, big + 4096, FAKE + RB, 16, NULL, NULL) == -2
    assert sd(FAKE, 8, RB, big, big + 64, 2, big + 4096, big + 4096 + RB, 16, NULL, NULL) == -2
    # combine: y over z (bf16, H = 128: 256-byte rows)
    assert L.moe_combine(FAKE, 1, 8, 128, big, 2, NULL, 4, FAKE + RB, 1, NULL, NULL, NULL) == -2
    # backward: scaled permute out over x; row dot out over a
    assert L.moe_permute_scaled(FAKE, 1, 8, 128, big, 1, big + 64, FAKE, 1, 8, NULL, NULL,
                                NULL) == -2
    assert L.moe_row_dot(FAKE, 1, 8, 128, big, 1, 8, big + 4096, 1, FAKE + 16, NULL, NULL,
                         NULL) == -2


def test_bound_call_converts_once_and_checks_status(built_lib):
    """ops.Bound: the arguments are converted to the entry point's ctypes
    once; a replay that the library refuses on the host raises MoeError (here
    width 0, refused before anything is enqueued)."""
    import ctypes

    import torch

    from co_activation_amd import _lib, ops
    args = (FAKE, 8, 256, FAKE + 8192, 0, FAKE + 16384, 8, NULL, NULL)
    b = ops.Bound("moe_permute", args, torch.device("cuda", 0))
    assert len(b.args) == len(args) and isinstance(b.args[0], ctypes.c_void_p)
    assert isinstance(b.args[1], ctypes.c_int64) and b.args[4].value == 0
    with pytest.raises(_lib.MoeError, match="MOE_ERR_SHAPE"):
        b(0)
