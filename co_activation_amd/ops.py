"""torch-facing wrappers of the C ABI (argument marshalling only).

Every function takes device tensors, checks dtype / contiguity / device /
shape, passes raw pointers and ``torch.cuda.current_stream()`` (which must
be on the tensors' device) to the library, and returns the output tensors.
All compute happens in the HIP kernels; outputs may be preallocated through
``out=`` to keep allocations out of a timed loop.  Device-side data errors are OR-ed into ``d_err`` (an int32
tensor of one element); ``raise_on_errors`` reads it back.

``coact_stats``, ``dispatch_plan``, ``permute``, ``combine``,
``shuffle_predict`` and ``shuffle_dispatch`` also take ``bind=True``: they check their arguments as usual but, instead of calling
the library, return ``(result, Bound)``, the call with its arguments already
converted, which a loop that the host paces replays on a stream with no
further checks (the buffers are read and written in place at each replay).
"""

from __future__ import annotations

import ctypes
import math
from typing import NamedTuple, Optional

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_F32, check

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


def _stream(ref: torch.Tensor) -> int:
    """The current stream, which must belong to the device holding ``ref``:
    the kernels run on the stream's device and would otherwise be handed
    another device's pointers."""
    idx = ref.device.index
    cur = torch.cuda.current_device()
    if idx != cur:
        raise ValueError(f"tensors are on {ref.device} but the current device is cuda:{cur}; "
                         "call under torch.cuda.device(...)")
    return torch.cuda.current_stream(idx).cuda_stream


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


try:  # the raw hipStream_t of a device's current stream, without a Stream object
    _raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover
    def _raw_stream(idx):
        return torch.cuda.current_stream(idx).cuda_stream


class Bound:
    """One library call whose arguments an ops function has checked, with
    the arguments converted once.  ``bound(stream)`` enqueues it on
    ``stream`` (a hipStream_t as an int); ``bound()`` on the current stream
    of the device it was bound on.  The buffers are the ones given at bind
    time: keep them alive and do not replace them."""

    __slots__ = ("name", "fn", "args", "device")

    def __init__(self, name: str, args: tuple, device: torch.device):
        self.name = name
        self.fn = getattr(_lib.lib(), name)
        self.args = tuple(t(a) for t, a in zip(self.fn.argtypes, args))
        self.device = device.index

    def __call__(self, stream: Optional[int] = None) -> None:
        if stream is None:
            stream = _raw_stream(self.device)
        st = self.fn(*self.args, stream)
        if st != 0:
            check(self.name, st)


def _run(name: str, args: tuple, ref: torch.Tensor, bind: bool):
    """Calls entry point ``name`` with ``args`` and the current stream of
    ``ref``'s device, or with ``bind`` returns the call as a ``Bound``."""
    if bind:
        return Bound(name, args, ref.device)
    check(name, getattr(_lib.lib(), name)(*args, _stream(ref)))
    return None


def _want(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _same_device(ref: torch.Tensor, *ts) -> None:
    """Every given tensor lives on ref's device (the kernels run there and
    would otherwise be handed another device's pointers)."""
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"all tensors of a call must be on {ref.device}, "
                             f"got one on {t.device}")


def _err_word(d_err: Optional[torch.Tensor], ref: torch.Tensor):
    """The device error word: None, or one int32 element on ref's device."""
    if d_err is None:
        return None
    _want(d_err, "d_err", torch.int32)
    if d_err.numel() != 1:
        raise ValueError("d_err must be a single int32 element")
    _same_device(ref, d_err)
    return d_err


def _alloc(out: Optional[dict], key: str, shape, dtype, device) -> torch.Tensor:
    if out is not None and out.get(key) is not None:
        return _want(out[key], key, dtype, shape)
    return torch.empty(shape, dtype=dtype, device=device)


def new_error_word(device="cuda") -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device)


def decode_errors(bits: int) -> list:
    return [name for b, name in _lib.DERR_BITS.items() if bits & b]


def raise_on_errors(d_err: torch.Tensor) -> None:
    bits = int(d_err.item())
    if bits:
        raise RuntimeError(f"device data errors: {decode_errors(bits)}")


# ----------------------------------------------------------------- stats

def stats_workspace_bytes(T: int, E: int, pairs: bool = True, E_next: int = 0) -> int:
    n = ctypes.c_size_t()
    check("moe_coact_stats_workspace_size",
          _lib.lib().moe_coact_stats_workspace_size(T, E, int(pairs), E_next, ctypes.byref(n)))
    return n.value


def coact_stats(topk: torch.Tensor, E: int, topk_next: Optional[torch.Tensor] = None,
                E_next: Optional[int] = None, *, pairs: bool = True, ochiai: bool = True,
                out: Optional[dict] = None, ws: Optional[torch.Tensor] = None,
                d_err: Optional[torch.Tensor] = None, bind: bool = False):
    """moe_coact_stats: expert_count [E], pair_count [E,E], ochiai [E,E],
    transition [E,E_next] (when topk_next is given).  ws: the workspace
    (uint8, at least stats_workspace_bytes); allocated here when not given."""
    _want(topk, "topk", torch.int32)
    T, k = topk.shape
    dev = topk.device
    res = {"expert_count": _alloc(out, "expert_count", (E,), torch.int32, dev)}
    if pairs:
        res["pair_count"] = _alloc(out, "pair_count", (E, E), torch.int32, dev)
        if ochiai:
            res["ochiai"] = _alloc(out, "ochiai", (E, E), torch.float32, dev)
    k2 = 0
    if topk_next is not None:
        _want(topk_next, "topk_next", torch.int32)
        if topk_next.shape[0] != T:
            raise ValueError("topk_next must cover the same tokens")
        k2 = topk_next.shape[1]
        res["transition"] = _alloc(out, "transition", (E, E_next), torch.int32, dev)
    need = stats_workspace_bytes(T, E, pairs, E_next if topk_next is not None else 0)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _want(ws, "ws", torch.uint8)
    err = _err_word(d_err, topk)
    _same_device(topk, topk_next, ws, res.get("pair_count"), res.get("ochiai"),
                 res.get("transition"), res["expert_count"])
    b = _run("moe_coact_stats",
             (_p(topk), T, k, E, _p(topk_next), k2, E_next or 0, _p(res["expert_count"]),
              _p(res.get("pair_count")), _p(res.get("ochiai")), _p(res.get("transition")),
              _p(err), _p(ws), ws.numel()), topk, bind)
    return (res, b) if bind else res


# ----------------------------------------------------------------- plan

class Plan(NamedTuple):
    send_counts: torch.Tensor   # [G, G] int32
    send_offsets: torch.Tensor  # [G*G+1] int32
    row_token: torch.Tensor     # [row_capacity] int32
    row_weight: Optional[torch.Tensor]  # [row_capacity] float32
    token_rows: torch.Tensor    # [T, k] int32
    slot_row: Optional[torch.Tensor]    # [T, k] int32
    counters: torch.Tensor      # [8] int64


def plan_workspace_bytes(T: int, G: int) -> int:
    n = ctypes.c_size_t()
    check("moe_dispatch_plan_workspace_size",
          _lib.lib().moe_dispatch_plan_workspace_size(T, G, ctypes.byref(n)))
    return n.value


def dispatch_plan(topk: torch.Tensor, gates: Optional[torch.Tensor], expert_rank: torch.Tensor,
                  G: int, ranks_per_node: int, src_offsets: Optional[torch.Tensor] = None, *,
                  row_capacity: Optional[int] = None, with_weights: bool = True,
                  with_slot_row: bool = True, out: Optional[dict] = None,
                  ws: Optional[torch.Tensor] = None,
                  d_err: Optional[torch.Tensor] = None, perm: Optional[torch.Tensor] = None,
                  topk_out: Optional[torch.Tensor] = None,
                  gates_out: Optional[torch.Tensor] = None, bind: bool = False):
    """moe_dispatch_plan.  row_capacity defaults to T * min(k, G).

    With ``perm`` (moe_dispatch_plan_gathered): the plan of the batch in the
    order perm, position p holding token perm[p]; the routing in that order
    is written to ``topk_out`` (and ``gates_out`` when gates are given),
    which the caller provides."""
    _want(topk, "topk", torch.int32)
    T, k = topk.shape
    E = expert_rank.numel()
    _want(expert_rank, "expert_rank", torch.int32, (E,))
    if gates is not None:
        _want(gates, "gates", torch.float32, (T, k))
    if src_offsets is not None:
        _want(src_offsets, "src_offsets", torch.int32, (G + 1,))
    cap = T * min(k, G) if row_capacity is None else int(row_capacity)
    dev = topk.device
    sc = _alloc(out, "send_counts", (G, G), torch.int32, dev)
    so = _alloc(out, "send_offsets", (G * G + 1,), torch.int32, dev)
    rt = _alloc(out, "row_token", (cap,), torch.int32, dev)
    rw = _alloc(out, "row_weight", (cap,), torch.float32, dev) if with_weights else None
    tr = _alloc(out, "token_rows", (T, k), torch.int32, dev)
    sr = _alloc(out, "slot_row", (T, k), torch.int32, dev) if with_slot_row else None
    cn = _alloc(out, "counters", (8,), torch.int64, dev)
    need = plan_workspace_bytes(T, G)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _want(ws, "ws", torch.uint8)
    err = _err_word(d_err, topk)
    if perm is None:
        _same_device(topk, gates, expert_rank, src_offsets, sc, so, rt, rw, tr, sr, cn, ws, perm,
                     topk_out, gates_out)
        b = _run("moe_dispatch_plan",
                 (_p(topk), _p(gates), T, k, E, _p(expert_rank), G, ranks_per_node,
                  _p(src_offsets), cap, _p(sc), _p(so), _p(rt), _p(rw), _p(tr), _p(sr), _p(cn),
                  _p(err), _p(ws), ws.numel()), topk, bind)
        plan = Plan(sc, so, rt, rw, tr, sr, cn)
        return (plan, b) if bind else plan
    _want(perm, "perm", torch.int32, (T,))
    if topk_out is None or (gates is not None and gates_out is None):
        raise ValueError("a gathered plan writes the routing in the new order: give topk_out "
                         "(and gates_out with gates)")
    _want(topk_out, "topk_out", torch.int32, (T, k))
    if gates is not None:
        _want(gates_out, "gates_out", torch.float32, (T, k))
    _same_device(topk, gates, expert_rank, src_offsets, sc, so, rt, rw, tr, sr, cn, ws, perm,
                 topk_out, gates_out)
    b = _run("moe_dispatch_plan_gathered",
             (_p(topk), _p(gates), _p(perm), T, k, E, _p(expert_rank), G, ranks_per_node,
              _p(src_offsets), cap, _p(sc), _p(so), _p(rt), _p(rw), _p(tr), _p(sr), _p(cn),
              _p(topk_out), _p(gates_out), _p(err), _p(ws), ws.numel()), topk, bind)
    plan = Plan(sc, so, rt, rw, tr, sr, cn)
    return (plan, b) if bind else plan


def dispatch_plan_noalloc(topk: torch.Tensor, gates: Optional[torch.Tensor],
                          expert_rank: torch.Tensor, G: int, ranks_per_node: int,
                          src_offsets: Optional[torch.Tensor] = None, *, out: dict,
                          d_err: Optional[torch.Tensor] = None) -> Plan:
    """moe_dispatch_plan_noalloc: moe_dispatch_plan with the library's fixed
    device scratch instead of a workspace.  The caller passes every output in
    ``out`` (keys as ``Plan``'s fields; row_weight and slot_row may be
    None), so this call allocates nothing.  Calls that overlap on one device
    race on the shared scratch."""
    _want(topk, "topk", torch.int32)
    T, k = topk.shape
    E = expert_rank.numel()
    _want(expert_rank, "expert_rank", torch.int32, (E,))
    if gates is not None:
        _want(gates, "gates", torch.float32, (T, k))
    if src_offsets is not None:
        _want(src_offsets, "src_offsets", torch.int32, (G + 1,))
    sc = _want(out["send_counts"], "send_counts", torch.int32, (G, G))
    so = _want(out["send_offsets"], "send_offsets", torch.int32, (G * G + 1,))
    rt = _want(out["row_token"], "row_token", torch.int32)
    if rt.dim() != 1:
        raise ValueError("row_token must be one-dimensional")
    cap = rt.shape[0]
    rw = out.get("row_weight")
    if rw is not None:
        _want(rw, "row_weight", torch.float32, (cap,))
    tr = _want(out["token_rows"], "token_rows", torch.int32, (T, k))
    sr = out.get("slot_row")
    if sr is not None:
        _want(sr, "slot_row", torch.int32, (T, k))
    cn = _want(out["counters"], "counters", torch.int64, (8,))
    err = _err_word(d_err, topk)
    _same_device(topk, gates, expert_rank, src_offsets, sc, so, rt, rw, tr, sr, cn)
    st = _lib.lib().moe_dispatch_plan_noalloc(
        _p(topk), _p(gates), T, k, E, _p(expert_rank), G, ranks_per_node, _p(src_offsets), cap,
        _p(sc), _p(so), _p(rt), _p(rw), _p(tr), _p(sr), _p(cn), _p(err), _stream(topk))
    check("moe_dispatch_plan_noalloc", st)
    return Plan(sc, so, rt, rw, tr, sr, cn)


# ----------------------------------------------------------------- permute

def permute(x: torch.Tensor, dest: torch.Tensor, out_rows: int, *,
            out: Optional[torch.Tensor] = None, n_valid: Optional[torch.Tensor] = None,
            d_err: Optional[torch.Tensor] = None, bind: bool = False):
    """moe_permute: out[dest[t, q]] = x[t] (bit copy).  dest is [T, width] or
    [T] int32; out has out_rows rows shaped like x's rows; n_valid (an int32
    device element, e.g. a plan's row count) limits the tokens moved."""
    _want(x, "x")
    _want(dest, "dest", torch.int32)
    T = x.shape[0]
    width = 1 if dest.dim() == 1 else dest.shape[1]
    if dest.shape[0] != T:
        raise ValueError("dest must have one row per token")
    row_shape = tuple(x.shape[1:])
    row_bytes = x.element_size() * (x[0].numel() if T > 0 else int(torch.tensor(row_shape).prod()))
    if out is None:
        out = torch.empty((out_rows,) + row_shape, dtype=x.dtype, device=x.device)
    _want(out, "out", x.dtype)
    if tuple(out.shape[1:]) != row_shape or out.shape[0] < out_rows:
        raise ValueError("out rows must match x rows")
    if n_valid is not None:
        _want(n_valid, "n_valid", torch.int32)
    err = _err_word(d_err, x)
    _same_device(x, dest, out, n_valid)
    b = _run("moe_permute", (_p(x), T, row_bytes, _p(dest), width, _p(out), out_rows, _p(n_valid),
                             _p(err)), x, bind)
    return (out, b) if bind else out


def shuffle_dispatch(x: torch.Tensor, perm: torch.Tensor, token_rows: torch.Tensor,
                     send_rows: int, *, x_out: Optional[torch.Tensor] = None,
                     send: Optional[torch.Tensor] = None,
                     d_err: Optional[torch.Tensor] = None, bind: bool = False) -> tuple:
    """moe_shuffle_dispatch: x_out[p] = x[perm[p]] and
    send[token_rows[p, q]] = x[perm[p]] (bit copies); token_rows [T, k] is
    indexed by shuffled position.  Returns (x_out, send)."""
    _want(x, "x")
    _want(perm, "perm", torch.int32)
    _want(token_rows, "token_rows", torch.int32)
    T = x.shape[0]
    if perm.numel() != T or token_rows.dim() != 2 or token_rows.shape[0] != T:
        raise ValueError("perm and token_rows need one entry / row per position")
    k = token_rows.shape[1]
    row_shape = tuple(x.shape[1:])
    row_bytes = x.element_size() * math.prod(row_shape)
    if x_out is None:
        x_out = torch.empty_like(x)
    if send is None:
        send = torch.empty((send_rows,) + row_shape, dtype=x.dtype, device=x.device)
    _want(x_out, "x_out", x.dtype)
    _want(send, "send", x.dtype)
    if x_out.shape != x.shape or tuple(send.shape[1:]) != row_shape or send.shape[0] < send_rows:
        raise ValueError("x_out must match x; send needs send_rows rows shaped like x's rows")
    err = _err_word(d_err, x)
    _same_device(x, perm, token_rows, x_out, send)
    b = _run("moe_shuffle_dispatch", (_p(x), T, row_bytes, _p(perm), _p(token_rows), k, _p(x_out),
                                      _p(send), send_rows, _p(err)), x, bind)
    return ((x_out, send), b) if bind else (x_out, send)


def gather(x: torch.Tensor, src: torch.Tensor, *, out: Optional[torch.Tensor] = None,
           n_valid: Optional[torch.Tensor] = None,
           d_err: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_gather: out[i] = x[src[i]] (bit copy; rows with src < 0 are left
    as they are).  src is [n] int32; out has n rows shaped like x's rows."""
    _want(x, "x")
    _want(src, "src", torch.int32)
    if src.dim() != 1:
        raise ValueError("src must be one-dimensional")
    n = src.shape[0]
    row_shape = tuple(x.shape[1:])
    row_bytes = x.element_size() * math.prod(row_shape)
    if out is None:
        out = torch.empty((n,) + row_shape, dtype=x.dtype, device=x.device)
    _want(out, "out", x.dtype)
    if tuple(out.shape[1:]) != row_shape or out.shape[0] < n:
        raise ValueError("out must have n rows shaped like x's rows")
    if n_valid is not None:
        _want(n_valid, "n_valid", torch.int32)
    err = _err_word(d_err, x)
    _same_device(x, src, out, n_valid)
    st = _lib.lib().moe_gather(_p(x), x.shape[0], row_bytes, _p(src), n, _p(out), _p(n_valid),
                               _p(err), _stream(x))
    check("moe_gather", st)
    return out


# ----------------------------------------------------------------- combine

def combine(z: torch.Tensor, rows: torch.Tensor, row_weight: Optional[torch.Tensor] = None, *,
            out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
            n_valid: Optional[torch.Tensor] = None,
            d_err: Optional[torch.Tensor] = None, bind: bool = False):
    """moe_combine: y[t] = sum_q a(rows[t,q]) z[rows[t,q]], a = row_weight or 1."""
    _want(z, "z")
    if z.dtype not in _DT:
        raise TypeError("z must be float32 or bfloat16")
    _want(rows, "rows", torch.int32)
    T, k = rows.shape
    H = z.shape[1]
    if row_weight is not None:
        _want(row_weight, "row_weight", torch.float32)
        if row_weight.dim() != 1 or row_weight.numel() < z.shape[0]:
            raise ValueError("row_weight needs one weight per row of z (the kernel reads "
                             "row_weight[r] for every row id r < z.shape[0])")
    out_dtype = out_dtype or z.dtype
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=z.device)
    _want(out, "out", out_dtype, (T, H))
    if n_valid is not None:
        _want(n_valid, "n_valid", torch.int32)
    err = _err_word(d_err, z)
    _same_device(z, rows, row_weight, out, n_valid)
    b = _run("moe_combine", (_p(z), _DT[z.dtype], z.shape[0], H, _p(rows), k, _p(row_weight), T,
                             _p(out), _DT[out_dtype], _p(n_valid), _p(err)), z, bind)
    return (out, b) if bind else out


# ----------------------------------------------------------------- shuffle

def shuffle_workspace_bytes(T: int, E: int, G: int, balanced: bool = False) -> int:
    n = ctypes.c_size_t()
    fn = "moe_shuffle_balanced_workspace_size" if balanced else "moe_shuffle_predict_workspace_size"
    check(fn, getattr(_lib.lib(), fn)(T, E, G, ctypes.byref(n)))
    return n.value


def shuffle_predict(topk: torch.Tensor, transition: torch.Tensor, expert_rank_next: torch.Tensor,
                    G: int, *, balanced: bool = False, with_perm: bool = True,
                    out: Optional[dict] = None, ws: Optional[torch.Tensor] = None,
                    d_err: Optional[torch.Tensor] = None, bind: bool = False):
    """moe_shuffle_predict (or moe_shuffle_balanced with balanced=True):
    pred_rank [T], dest_pos [T], perm [T], shard_offsets [G+1]."""
    _want(topk, "topk", torch.int32)
    T, k = topk.shape
    E, E2 = transition.shape
    _want(transition, "transition", torch.int32)
    _want(expert_rank_next, "expert_rank_next", torch.int32, (E2,))
    dev = topk.device
    res = {
        "pred_rank": _alloc(out, "pred_rank", (T,), torch.int32, dev),
        "dest_pos": _alloc(out, "dest_pos", (T,), torch.int32, dev),
        "perm": _alloc(out, "perm", (T,), torch.int32, dev) if with_perm else None,
        "shard_offsets": _alloc(out, "shard_offsets", (G + 1,), torch.int32, dev),
    }
    need = shuffle_workspace_bytes(T, E, G, balanced)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _want(ws, "ws", torch.uint8)
    err = _err_word(d_err, topk)
    _same_device(topk, transition, expert_rank_next, ws, res["pred_rank"], res["dest_pos"],
                 res["perm"], res["shard_offsets"])
    b = _run("moe_shuffle_balanced" if balanced else "moe_shuffle_predict",
             (_p(topk), T, k, E, _p(transition), E2, _p(expert_rank_next), G, _p(res["pred_rank"]),
              _p(res["dest_pos"]), _p(res["perm"]), _p(res["shard_offsets"]), _p(err), _p(ws),
              ws.numel()), topk, bind)
    return (res, b) if bind else res


# ----------------------------------------------------------------- expert side

def expert_workspace_bytes(T: int, E: int) -> int:
    n = ctypes.c_size_t()
    check("moe_expert_plan_workspace_size",
          _lib.lib().moe_expert_plan_workspace_size(T, E, ctypes.byref(n)))
    return n.value


def expert_plan(topk: torch.Tensor, gates: Optional[torch.Tensor], expert_rank: torch.Tensor,
                G: int, slot_row: torch.Tensor, send_rows: int, *, with_slots: bool = True,
                out: Optional[dict] = None, ws: Optional[torch.Tensor] = None,
                d_err: Optional[torch.Tensor] = None) -> dict:
    """moe_expert_plan: erow [T,k], expert_first [E], expert_count [E],
    rank_offsets [G+1], erow_weight [T*k], erow_slot [T*k], erow_src [T*k],
    row_dest [send_rows, k]."""
    _want(topk, "topk", torch.int32)
    T, k = topk.shape
    E = expert_rank.numel()
    _want(expert_rank, "expert_rank", torch.int32, (E,))
    _want(slot_row, "slot_row", torch.int32, (T, k))
    if gates is not None:
        _want(gates, "gates", torch.float32, (T, k))
    dev = topk.device
    res = {
        "erow": _alloc(out, "erow", (T, k), torch.int32, dev),
        "expert_first": _alloc(out, "expert_first", (E,), torch.int32, dev),
        "expert_count": _alloc(out, "expert_count", (E,), torch.int32, dev),
        "rank_offsets": _alloc(out, "rank_offsets", (G + 1,), torch.int32, dev),
        "erow_weight": _alloc(out, "erow_weight", (T * k,), torch.float32, dev),
        "erow_slot": _alloc(out, "erow_slot", (T * k,), torch.int32, dev) if with_slots else None,
        "erow_src": _alloc(out, "erow_src", (T * k,), torch.int32, dev),
        "row_dest": _alloc(out, "row_dest", (send_rows, k), torch.int32, dev),
    }
    need = expert_workspace_bytes(T, E)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _want(ws, "ws", torch.uint8)
    err = _err_word(d_err, topk)
    _same_device(topk, gates, expert_rank, slot_row, ws, *res.values())
    st = _lib.lib().moe_expert_plan(
        _p(topk), _p(gates), T, k, E, _p(expert_rank), G, _p(slot_row), send_rows, _p(res["erow"]),
        _p(res["expert_first"]), _p(res["expert_count"]), _p(res["rank_offsets"]),
        _p(res["erow_weight"]), _p(res["erow_slot"]), _p(res["erow_src"]), _p(res["row_dest"]),
        _p(err), _p(ws), ws.numel(), _stream(topk))
    check("moe_expert_plan", st)
    return res


# ----------------------------------------------------------------- backward

def permute_scaled(x: torch.Tensor, dest: torch.Tensor, scale: torch.Tensor, out_rows: int, *,
                   out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                   n_valid: Optional[torch.Tensor] = None,
                   d_err: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_permute_scaled: out[dest[t, q]] = scale[dest[t, q]] * x[t]."""
    _want(x, "x")
    if x.dtype not in _DT:
        raise TypeError("x must be float32 or bfloat16")
    _want(dest, "dest", torch.int32)
    _want(scale, "scale", torch.float32)
    T, H = x.shape
    width = 1 if dest.dim() == 1 else dest.shape[1]
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = torch.empty((out_rows, H), dtype=out_dtype, device=x.device)
    _want(out, "out", out_dtype)
    if (scale.dim() != 1 or scale.numel() < out_rows or out.dim() != 2 or out.shape[0] < out_rows
            or out.shape[1] != H):
        raise ValueError("scale and out need out_rows rows")
    if n_valid is not None:
        _want(n_valid, "n_valid", torch.int32)
    err = _err_word(d_err, x)
    _same_device(x, dest, scale, out, n_valid)
    st = _lib.lib().moe_permute_scaled(_p(x), _DT[x.dtype], T, H, _p(dest), width, _p(scale),
                                       _p(out), _DT[out_dtype], out_rows, _p(n_valid), _p(err),
                                       _stream(x))
    check("moe_permute_scaled", st)
    return out


def row_dot(a: torch.Tensor, b: torch.Tensor, rows: torch.Tensor, *,
            out: Optional[torch.Tensor] = None, n_valid: Optional[torch.Tensor] = None,
            d_err: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_row_dot: out[t, q] = <a[t], b[rows[t, q]]> (float32)."""
    _want(a, "a")
    _want(b, "b")
    if a.dtype not in _DT or b.dtype not in _DT:
        raise TypeError("a and b must be float32 or bfloat16")
    _want(rows, "rows", torch.int32)
    T, H = a.shape
    if b.shape[1] != H or rows.shape[0] != T:
        raise ValueError("shapes of a, b and rows disagree")
    width = 1 if rows.dim() == 1 else rows.shape[1]
    if out is None:
        out = torch.empty((T, width), dtype=torch.float32, device=a.device)
    _want(out, "out", torch.float32)
    if out.numel() != T * width:
        raise ValueError(f"out must hold T x width = {T} x {width} values")
    if n_valid is not None:
        _want(n_valid, "n_valid", torch.int32)
    err = _err_word(d_err, a)
    _same_device(a, b, rows, out, n_valid)
    st = _lib.lib().moe_row_dot(_p(a), _DT[a.dtype], T, H, _p(b), _DT[b.dtype], b.shape[0],
                                _p(rows), width, _p(out), _p(n_valid), _p(err), _stream(a))
    check("moe_row_dot", st)
    return out


# ----------------------------------------------------------------- placement

def ema_update(state: torch.Tensor, x: torch.Tensor, beta: float) -> torch.Tensor:
    """moe_ema_update: state = beta * state + (1 - beta) * x, in place."""
    _want(state, "state", torch.float32)
    _want(x, "x", torch.int32)
    if state.numel() != x.numel():
        raise ValueError("state and x must have the same size")
    check("moe_ema_update", _lib.lib().moe_ema_update(_p(state), _p(x), state.numel(), float(beta),
                                                      _stream(state)))
    return state


def place_experts(coact, load, G: int, eps: float):
    """moe_place_experts on host arrays (numpy float32 [E,E] and [E]);
    returns a numpy int32 [E] placement."""
    import numpy as np

    C = np.ascontiguousarray(coact, dtype=np.float32)
    w = np.ascontiguousarray(load, dtype=np.float32)
    E = w.shape[0]
    if C.shape != (E, E):
        raise ValueError("coact must be [E, E]")
    out = np.empty(E, dtype=np.int32)
    check("moe_place_experts", _lib.lib().moe_place_experts(C.ctypes.data, w.ctypes.data, E, G,
                                                            float(eps), out.ctypes.data))
    return out
