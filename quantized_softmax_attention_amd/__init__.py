"""K-interval attention on AMD Instinct MI355X (gfx950).

A thin binding over libkia.so (C ABI in include/kia.h).  PyTorch only
supplies device memory and the current stream; every step of the operator
runs in the library's HIP kernels.  The functions keep the C names:

    o, stats = kia_forward(q, k, v, params)
    dq, dk, dv, ws = kia_backward(q, k, v, o, do, stats, params)
    o = kia_attention(q, k, v, params)          # the same two calls as an autograd op

with q, k, v, o, do fp32 CUDA tensors of shape [B, H, T, d], d in {64, 128}.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

from . import _lib
from ._lib import KiaExt, KiaParams, KiaStatsLayout, KiaWorkspaceLayout

CAL = {"minmax": 0, "fwm": 1, "fwm_untrunc": 2}
REC = {"lerp": 0, "nearest": 1, "exact": 2, "exp_bf16": 3, "exp_fp8": 4}
STE = {"weight": 0, "prob": 1}
RULE = {"full": 0, "detach": 1, "max_only": 2, "min_only": 3, "p1": 4}


class KiaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.load().kia_status_str(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


@dataclass(frozen=True)
class Params:
    """Operator flags; K is the number of intervals (K+1 grid values)."""
    K: int
    tau: float = 6.0
    calibration: str = "minmax"
    reconstruction: str = "lerp"
    surrogate: str = "weight"
    grad_rule: str = "full"

    def c(self) -> KiaParams:
        def pick(table, v):
            return table[v] if isinstance(v, str) else int(v)
        return KiaParams(int(self.K), float(self.tau), pick(CAL, self.calibration),
                         pick(REC, self.reconstruction), pick(STE, self.surrogate),
                         pick(RULE, self.grad_rule))


def _torch():
    import torch
    return torch


def _shape(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, T, d]")
    return tuple(int(x) for x in q.shape)


def _check(t, name, shape=None, device=None):
    """A contiguous fp32 GPU tensor (of the given shape, on the given device)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if shape is not None and tuple(t.shape) != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _nbytes(t):
    return t.numel() * t.element_size()


def _buffer(t, name, nbytes, device):
    """A contiguous GPU buffer of any dtype holding at least nbytes bytes."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, the call needs {nbytes}")


def _size_error(lib, query, cp, B, H, T, d, layout):
    """The status of the size query's checks (a size query returns 0 on error)."""
    out = layout()
    st = getattr(lib, query)(ctypes.byref(cp), B, H, T, d, ctypes.byref(out))
    return KiaError(st if st else 2, query)


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _ext(events, idx_dump):
    if events is None and idx_dump is None:
        return None
    ext = KiaExt()
    if events is not None:
        arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(int(e)) for e in events])
        ext.events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        ext.n_events = len(events)
        ext._keep = arr
    if idx_dump is not None:
        ext.idx_dump = ctypes.c_void_p(idx_dump.data_ptr())
    return ext


def kia_stats_bytes(params: Params, B, H, T, d) -> int:
    return int(_lib.load().kia_stats_bytes(ctypes.byref(params.c()), B, H, T, d))


def kia_workspace_bytes(params: Params, B, H, T, d) -> int:
    return int(_lib.load().kia_workspace_bytes(ctypes.byref(params.c()), B, H, T, d))


def kia_stats_layout_query(params: Params, B, H, T, d) -> KiaStatsLayout:
    out = KiaStatsLayout()
    st = _lib.load().kia_stats_layout_query(ctypes.byref(params.c()), B, H, T, d, ctypes.byref(out))
    if st:
        raise KiaError(st, "kia_stats_layout_query")
    return out


def kia_workspace_layout_query(params: Params, B, H, T, d) -> KiaWorkspaceLayout:
    out = KiaWorkspaceLayout()
    st = _lib.load().kia_workspace_layout_query(ctypes.byref(params.c()), B, H, T, d, ctypes.byref(out))
    if st:
        raise KiaError(st, "kia_workspace_layout_query")
    return out


def kia_forward(q, k, v, params: Params, o=None, stats=None, stream=None, events=None, idx_dump=None):
    """O = P V with K-interval weights.  Returns (o, stats); stats is a uint8
    device buffer holding the forward -> backward state.  Buffers passed in
    (o, stats, idx_dump) are checked for device, dtype, shape or size."""
    torch = _torch()
    B, H, T, d = _shape(q)
    dev = q.device
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, (B, H, T, d), dev)
    lib = _lib.load()
    cp = params.c()
    nbytes = int(lib.kia_stats_bytes(ctypes.byref(cp), B, H, T, d))
    if nbytes == 0:
        raise _size_error(lib, "kia_stats_layout_query", cp, B, H, T, d, KiaStatsLayout)
    if o is None:
        o = torch.empty_like(q)
    _check(o, "o", (B, H, T, d), dev)
    if stats is None:
        stats = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _buffer(stats, "stats", nbytes, dev)
    if idx_dump is not None:
        if idx_dump.dtype != torch.int32 or idx_dump.numel() != B * H * T * T:
            raise ValueError("idx_dump must be int32 with B*H*T*T elements")
        _buffer(idx_dump, "idx_dump", B * H * T * T * 4, dev)
    ext = _ext(events, idx_dump)
    with torch.cuda.device(dev):
        args = (ctypes.byref(cp), B, H, T, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                stats.data_ptr(), _nbytes(stats), _stream(stream, dev))
        st = lib.kia_forward_ext(*args, ctypes.byref(ext)) if ext is not None else lib.kia_forward(*args)
    if st:
        raise KiaError(st, "kia_forward")
    return o, stats


def kia_backward(q, k, v, o, do, stats, params: Params, dq=None, dk=None, dv=None, ws=None,
                 stream=None, events=None):
    """dQ, dK, dV of sum(do * o).  Returns (dq, dk, dv, ws); ws is the
    workspace (uint8 device buffer) whose tiles kia_workspace_layout_query
    describes.  Buffers passed in are checked like kia_forward's."""
    torch = _torch()
    B, H, T, d = _shape(q)
    dev = q.device
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, nm, (B, H, T, d), dev)
    lib = _lib.load()
    cp = params.c()
    sbytes = int(lib.kia_stats_bytes(ctypes.byref(cp), B, H, T, d))
    wbytes = int(lib.kia_workspace_bytes(ctypes.byref(cp), B, H, T, d))
    if sbytes == 0 or wbytes == 0:
        raise _size_error(lib, "kia_workspace_layout_query", cp, B, H, T, d, KiaWorkspaceLayout)
    _buffer(stats, "stats", sbytes, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, nm, (B, H, T, d), dev)
    if ws is None:
        ws = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    _buffer(ws, "ws", wbytes, dev)
    ext = _ext(events, None)
    with torch.cuda.device(dev):
        args = (ctypes.byref(cp), B, H, T, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                do.data_ptr(), stats.data_ptr(), _nbytes(stats), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                ws.data_ptr(), _nbytes(ws), _stream(stream, dev))
        st = lib.kia_backward_ext(*args, ctypes.byref(ext)) if ext is not None else lib.kia_backward(*args)
    if st:
        raise KiaError(st, "kia_backward")
    return dq, dk, dv, ws


class Step:
    """One forward + backward over fixed buffers, for loops that launch the
    same step many times.  The buffers are checked once, here, by one
    kia_forward and one kia_backward call (which also run the step); each
    later call passes the stored arguments straight to the C ABI
    (kia_forward_ext / kia_backward_ext when HIP events are given), on the
    stream that was current here (or `stream`).  Call it with the tensors'
    device current; the tensors are kept alive by the object."""

    def __init__(self, q, k, v, do, params: Params, o, stats, dq, dk, dv, ws, stream=None):
        kia_forward(q, k, v, params, o=o, stats=stats, stream=stream)
        kia_backward(q, k, v, o, do, stats, params, dq=dq, dk=dk, dv=dv, ws=ws, stream=stream)
        B, H, T, d = _shape(q)
        self._lib = _lib.load()
        self._cp = params.c()
        st = _stream(stream, q.device)
        cp = ctypes.byref(self._cp)
        self._fargs = (cp, B, H, T, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       stats.data_ptr(), _nbytes(stats), st)
        self._bargs = (cp, B, H, T, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                       stats.data_ptr(), _nbytes(stats), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       ws.data_ptr(), _nbytes(ws), st)
        self._keep = (q, k, v, do, o, stats, dq, dk, dv, ws)

    def __call__(self, events_f=None, events_b=None):
        lib = self._lib
        if events_f is None:
            st = lib.kia_forward(*self._fargs)
        else:
            st = lib.kia_forward_ext(*self._fargs, ctypes.byref(_ext(events_f, None)))
        if st:
            raise KiaError(st, "kia_forward")
        if events_b is None:
            st = lib.kia_backward(*self._bargs)
        else:
            st = lib.kia_backward_ext(*self._bargs, ctypes.byref(_ext(events_b, None)))
        if st:
            raise KiaError(st, "kia_backward")


def kia_backward_noalloc(q, k, v, o, do, stats, params: Params, dq=None, dk=None, dv=None, stream=None):
    """kia_backward without a workspace: the library takes it from its own
    per-device scratch (include/kia.h, kia_backward_noalloc) and allocates
    nothing.  Output buffers not passed in are allocated here, by the caller's
    side.  Returns (dq, dk, dv)."""
    torch = _torch()
    B, H, T, d = _shape(q)
    dev = q.device
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, nm, (B, H, T, d), dev)
    lib = _lib.load()
    cp = params.c()
    sbytes = int(lib.kia_stats_bytes(ctypes.byref(cp), B, H, T, d))
    if sbytes == 0:
        raise _size_error(lib, "kia_stats_layout_query", cp, B, H, T, d, KiaStatsLayout)
    _buffer(stats, "stats", sbytes, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, nm, (B, H, T, d), dev)
    with torch.cuda.device(dev):
        st = lib.kia_backward_noalloc(ctypes.byref(cp), B, H, T, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      o.data_ptr(), do.data_ptr(), stats.data_ptr(), _nbytes(stats),
                                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream(stream, dev))
    if st:
        raise KiaError(st, "kia_backward_noalloc")
    return dq, dk, dv


GEOMETRY_FIELDS = ("span", "h", "q_norm", "k_norm", "entropy_p", "entropy_soft", "tv", "top_mass")


def kia_geometry(q, k, stats, params: Params, geo=None, stream=None):
    """Score-geometry probe over the scores a kia_forward call with the same
    params left in stats.  Returns geo, fp32 [8, B, H, T], fields in the
    order of GEOMETRY_FIELDS."""
    torch = _torch()
    B, H, T, d = _shape(q)
    dev = q.device
    _check(q, "q", (B, H, T, d), dev)
    _check(k, "k", (B, H, T, d), dev)
    lib = _lib.load()
    cp = params.c()
    sbytes = int(lib.kia_stats_bytes(ctypes.byref(cp), B, H, T, d))
    if sbytes == 0:
        raise _size_error(lib, "kia_stats_layout_query", cp, B, H, T, d, KiaStatsLayout)
    _buffer(stats, "stats", sbytes, dev)
    if geo is None:
        geo = torch.empty((len(GEOMETRY_FIELDS), B, H, T), dtype=torch.float32, device=dev)
    _check(geo, "geo", (len(GEOMETRY_FIELDS), B, H, T), dev)
    with torch.cuda.device(dev):
        st = lib.kia_geometry(ctypes.byref(cp), B, H, T, d, q.data_ptr(), k.data_ptr(), stats.data_ptr(),
                              _nbytes(stats), geo.data_ptr(), _nbytes(geo), _stream(stream, dev))
    if st:
        raise KiaError(st, "kia_geometry")
    return geo


def kia_tiles_to_dense(B, H, T, tiles, key_major: bool, dense=None, stream=None):
    """Expand a tile buffer (a uint8/float view starting at the tiles) into a
    dense [B, H, T, T] fp32 tensor; non-causal entries keep dense's content
    (zeros when dense is allocated here)."""
    torch = _torch()
    dev = tiles.device
    n_t = (T + 31) // 32
    _buffer(tiles, "tiles", B * H * (n_t * (n_t + 1) // 2) * 32 * 32 * 4, dev)
    if dense is None:
        dense = torch.zeros((B, H, T, T), dtype=torch.float32, device=dev)
    _check(dense, "dense", (B, H, T, T), dev)
    with torch.cuda.device(dev):
        st = _lib.load().kia_tiles_to_dense(B, H, T, tiles.data_ptr(), 1 if key_major else 0,
                                            dense.data_ptr(), _stream(stream, dev))
    if st:
        raise KiaError(st, "kia_tiles_to_dense")
    return dense


def kia_attention(q, k, v, params: Params):
    """O = K-interval attention of q, k, v as a differentiable torch op: the
    forward calls kia_forward, the backward kia_backward with the saved
    stats (so dQ, dK, dV follow params' gradient rule and surrogate).  The
    incoming gradient is made contiguous; no other work happens here."""
    return _KiaAttention.apply(q, k, v, params)


def _make_function():
    torch = _torch()

    class KiaAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, params):
            o, stats = kia_forward(q, k, v, params)
            ctx.save_for_backward(q, k, v, o, stats)
            ctx.params = params
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, stats = ctx.saved_tensors
            dq, dk, dv, _ = kia_backward(q, k, v, o, do.contiguous(), stats, ctx.params)
            return dq, dk, dv, None

    return KiaAttention


class _Lazy:
    """The autograd Function class, built on first use (torch is imported
    only then)."""
    fn = None

    @classmethod
    def apply(cls, *args):
        if cls.fn is None:
            cls.fn = _make_function()
        return cls.fn.apply(*args)


_KiaAttention = _Lazy


def kia_abi_version() -> int:
    return int(_lib.load().kia_abi_version())


__all__ = ["Params", "KiaError", "kia_forward", "kia_backward", "kia_stats_bytes",
           "kia_workspace_bytes", "kia_stats_layout_query", "kia_workspace_layout_query",
           "kia_geometry", "GEOMETRY_FIELDS", "kia_tiles_to_dense", "kia_abi_version", "kia_attention", "Step"]
