"""Routed mixture-of-experts FFN layer for AMD MI355X (gfx950).

A thin ctypes binding over ``libcoli_moe.so`` -- the C ABI declared in
``include/coli_moe.h``.  Every step of the layer runs in the library's HIP
kernels; this module only marshals arguments (device pointers taken from
torch tensors, sizes, the current HIP stream) and turns error codes into
exceptions.  PyTorch provides device memory and streams, nothing else.

The entry points keep the C names:

  coli_moe_workspace_bytes(shape, int4=False) -> int
  coli_moe_route(shape, x, w_router, bias, routing, ws, stream=None)
  coli_moe_ffn(shape, x, routing, weights, y, residual=None, y_bf16=None, ws, stream=None)
  coli_moe_ffn_int4(shape, x, routing, weights_int4, y, residual=None, y_bf16=None, ws, stream=None)
  coli_moe_dense_workspace_bytes(shape) -> int
  coli_moe_dense_ffn(shape, x, dense_weights, y, residual=None, y_bf16=None, ws, stream=None)
  coli_moe_bank_fill(shape, host_tensors, bank_tensors, experts=None, int4=False, group=32,
                     copy_stream, wait_event=None, ready_event=None)
  coli_moe_bank_acquire(compute_stream, ready_event) / coli_moe_bank_release(compute_stream, free_event)
  coli_index_topk_workspace_bytes(rows, L, k) -> int
  coli_index_topk(scores, k, idx, tail=0, lens=None, ws=None, stream=None)
  coli_moe_status_str(code) -> str

If the library has not been built the import still works, but every call
raises ``ColiError`` -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoli_moe.so")

COLI_F32, COLI_BF16 = 0, 1
STATUS_NAMES = {0: "COLI_OK", 1: "COLI_E_NULL", 2: "COLI_E_SHAPE", 3: "COLI_E_DTYPE",
                4: "COLI_E_ALIGN", 5: "COLI_E_WORKSPACE", 6: "COLI_E_DEVICE",
                7: "COLI_E_LAUNCH", 8: "COLI_E_ALIAS", 9: "COLI_E_MEMORY"}
EXPORTED = ("coli_moe_workspace_bytes", "coli_moe_route", "coli_moe_ffn", "coli_moe_ffn_int4",
            "coli_moe_route_timed", "coli_moe_ffn_timed", "coli_moe_ffn_int4_timed",
            "coli_moe_dense_workspace_bytes", "coli_moe_dense_ffn",
            "coli_moe_bank_fill", "coli_moe_bank_acquire", "coli_moe_bank_release",
            "coli_index_topk_workspace_bytes", "coli_index_topk", "coli_moe_ffn_noalloc",
            "coli_moe_status_str", "coli_moe_version")
ROUTE_STAGES = ("router", "topk", "perm")
FFN_STAGES = ("gate_up", "down", "combine")


class ColiError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {STATUS_NAMES.get(code, code)}"
        try:
            msg += f" ({coli_moe_status_str(code)})"
        except Exception:   # library missing: keep the code only
            pass
        super().__init__(msg)


class CShape(C.Structure):
    _fields_ = [("T", C.c_int32), ("D", C.c_int32), ("E", C.c_int32), ("K", C.c_int32),
                ("F", C.c_int32), ("dtype", C.c_int32)]


class CRouting(C.Structure):
    _fields_ = [("ids", C.c_void_p), ("w", C.c_void_p), ("count", C.c_void_p),
                ("offset", C.c_void_p), ("perm", C.c_void_p), ("inv", C.c_void_p)]


class CWeights(C.Structure):
    _fields_ = [("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p),
                ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p)]


class CWeightsInt4(C.Structure):
    _fields_ = [("gate_q", C.c_void_p), ("up_q", C.c_void_p), ("down_q", C.c_void_p),
                ("gate_s", C.c_void_p), ("up_s", C.c_void_p), ("down_s", C.c_void_p),
                ("group", C.c_int32),
                ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p)]


class CDenseWeights(C.Structure):
    _fields_ = [("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p)]


_lib = None


def lib():
    """Load libcoli_moe.so (raises ColiError-like RuntimeError if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(there is no fallback implementation)")
        L = C.CDLL(LIB_PATH)
        vp, sz = C.c_void_p, C.c_size_t
        sp = C.POINTER(CShape)
        L.coli_moe_workspace_bytes.restype = sz
        L.coli_moe_workspace_bytes.argtypes = [sp, C.c_int]
        L.coli_moe_route.restype = C.c_int
        L.coli_moe_route.argtypes = [sp, vp, vp, vp, C.POINTER(CRouting), vp, sz, vp]
        L.coli_moe_ffn.restype = C.c_int
        L.coli_moe_ffn.argtypes = [sp, vp, C.POINTER(CRouting), C.POINTER(CWeights), vp, vp, vp,
                                   vp, sz, vp]
        L.coli_moe_ffn_int4.restype = C.c_int
        L.coli_moe_ffn_int4.argtypes = [sp, vp, C.POINTER(CRouting), C.POINTER(CWeightsInt4),
                                        vp, vp, vp, vp, sz, vp]
        ev = C.POINTER(C.c_void_p)
        L.coli_moe_route_timed.restype = C.c_int
        L.coli_moe_route_timed.argtypes = L.coli_moe_route.argtypes + [ev, C.c_int32]
        L.coli_moe_ffn_timed.restype = C.c_int
        L.coli_moe_ffn_timed.argtypes = L.coli_moe_ffn.argtypes + [ev, C.c_int32]
        L.coli_moe_ffn_int4_timed.restype = C.c_int
        L.coli_moe_ffn_int4_timed.argtypes = L.coli_moe_ffn_int4.argtypes + [ev, C.c_int32]
        L.coli_moe_dense_workspace_bytes.restype = sz
        L.coli_moe_dense_workspace_bytes.argtypes = [sp]
        L.coli_moe_dense_ffn.restype = C.c_int
        L.coli_moe_dense_ffn.argtypes = [sp, vp, C.POINTER(CDenseWeights), vp, vp, vp, vp, sz, vp]
        L.coli_moe_bank_fill.restype = C.c_int
        L.coli_moe_bank_fill.argtypes = [sp, C.c_int32, C.c_int32, C.POINTER(C.c_void_p),
                                         C.POINTER(C.c_void_p), C.POINTER(C.c_int32), C.c_int32,
                                         vp, vp, vp]
        L.coli_moe_bank_acquire.restype = C.c_int
        L.coli_moe_bank_acquire.argtypes = [vp, vp]
        L.coli_moe_bank_release.restype = C.c_int
        L.coli_moe_bank_release.argtypes = [vp, vp]
        L.coli_index_topk_workspace_bytes.restype = sz
        L.coli_index_topk_workspace_bytes.argtypes = [C.c_int32, C.c_int32, C.c_int32]
        L.coli_index_topk.restype = C.c_int
        L.coli_index_topk.argtypes = [vp, C.c_int32, C.c_int32, C.c_int64, vp, C.c_int32, C.c_int32,
                                      vp, vp, sz, vp]
        L.coli_moe_ffn_noalloc.restype = C.c_int
        L.coli_moe_ffn_noalloc.argtypes = [sp, vp, C.POINTER(CRouting), C.POINTER(CWeights), vp, vp,
                                           vp, vp]
        L.coli_moe_status_str.restype = C.c_char_p
        L.coli_moe_status_str.argtypes = [C.c_int]
        L.coli_moe_version.restype = C.c_int32
        L.coli_moe_version.argtypes = []
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# argument containers
# ---------------------------------------------------------------------------

@dataclass
class Shape:
    T: int
    D: int
    E: int
    K: int
    F: int
    dtype: int = COLI_BF16

    def c(self) -> CShape:
        return CShape(self.T, self.D, self.E, self.K, self.F, self.dtype)


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None stays NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the C ABI must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class Routing:
    """Routing tensors (device, int32 / fp32), see coli_moe_routing."""
    ids: object
    w: object
    count: object
    offset: object
    perm: object
    inv: object

    @staticmethod
    def empty(T: int, E: int, K: int, device="cuda"):
        import torch
        i32 = dict(dtype=torch.int32, device=device)
        return Routing(ids=torch.empty((T, K), **i32),
                       w=torch.empty((T, K), dtype=torch.float32, device=device),
                       count=torch.empty(E, **i32), offset=torch.empty(E + 1, **i32),
                       perm=torch.empty(T * K, **i32), inv=torch.empty(T * K, **i32))

    def c(self) -> CRouting:
        return CRouting(*[_ptr(getattr(self, k)) for k in
                          ("ids", "w", "count", "offset", "perm", "inv")])


@dataclass
class Weights:
    gate: object
    up: object
    down: object
    s_gate: object
    s_up: object
    s_down: object

    def c(self) -> CWeights:
        return CWeights(*[_ptr(getattr(self, k)) for k in
                          ("gate", "up", "down", "s_gate", "s_up", "s_down")])


@dataclass
class WeightsInt4:
    gate_q: object
    up_q: object
    down_q: object
    gate_s: object
    up_s: object
    down_s: object
    group: int
    s_gate: object
    s_up: object
    s_down: object

    def c(self) -> CWeightsInt4:
        return CWeightsInt4(_ptr(self.gate_q), _ptr(self.up_q), _ptr(self.down_q),
                            _ptr(self.gate_s), _ptr(self.up_s), _ptr(self.down_s), self.group,
                            _ptr(self.s_gate), _ptr(self.s_up), _ptr(self.s_down))


def _check(code: int, where: str):
    if code != 0:
        raise ColiError(code, where)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def coli_moe_status_str(code: int) -> str:
    return lib().coli_moe_status_str(code).decode()


def coli_moe_version() -> int:
    return lib().coli_moe_version()


def coli_moe_workspace_bytes(shape: Shape, int4: bool = False) -> int:
    cs = shape.c()
    return lib().coli_moe_workspace_bytes(C.byref(cs), 1 if int4 else 0)


def _nbytes(ws, ws_bytes):
    if ws_bytes is not None:
        return ws_bytes
    return ws.numel() * ws.element_size() if ws is not None else 0


def _events(events):
    """A list of hipEvent_t handles (ints) -> (void** array, count); None -> (None, 0)."""
    if not events:
        return None, 0
    arr = (C.c_void_p * len(events))(*events)
    return arr, len(events)


def coli_moe_route(shape: Shape, x, w_router, bias, routing: Routing, ws, ws_bytes=None,
                   stream=None, events=None) -> None:
    """Route T tokens; ``events`` (hipEvent_t handles) selects the timed variant."""
    cs, cr = shape.c(), routing.c()
    args = [C.byref(cs), _ptr(x), _ptr(w_router), _ptr(bias), C.byref(cr), _ptr(ws),
            _nbytes(ws, ws_bytes), _stream(stream)]
    if events:
        _check(lib().coli_moe_route_timed(*args, *_events(events)), "coli_moe_route_timed")
    else:
        _check(lib().coli_moe_route(*args), "coli_moe_route")


def coli_moe_ffn(shape: Shape, x, routing: Routing, weights: Weights, y, residual=None,
                 y_bf16=None, ws=None, ws_bytes=None, stream=None, events=None) -> None:
    cs, cr, cw = shape.c(), routing.c(), weights.c()
    args = [C.byref(cs), _ptr(x), C.byref(cr), C.byref(cw), _ptr(residual), _ptr(y),
            _ptr(y_bf16), _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)]
    if events:
        _check(lib().coli_moe_ffn_timed(*args, *_events(events)), "coli_moe_ffn_timed")
    else:
        _check(lib().coli_moe_ffn(*args), "coli_moe_ffn")


def coli_moe_ffn_int4(shape: Shape, x, routing: Routing, weights: WeightsInt4, y, residual=None,
                      y_bf16=None, ws=None, ws_bytes=None, stream=None, events=None) -> None:
    cs, cr, cw = shape.c(), routing.c(), weights.c()
    args = [C.byref(cs), _ptr(x), C.byref(cr), C.byref(cw), _ptr(residual), _ptr(y),
            _ptr(y_bf16), _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)]
    if events:
        _check(lib().coli_moe_ffn_int4_timed(*args, *_events(events)), "coli_moe_ffn_int4_timed")
    else:
        _check(lib().coli_moe_ffn_int4(*args), "coli_moe_ffn_int4")


# ---------------------------------------------------------------------------
# dense FFN layers, the expert bank, index selection
# ---------------------------------------------------------------------------

@dataclass
class DenseWeights:
    gate: object
    up: object
    down: object

    def c(self) -> CDenseWeights:
        return CDenseWeights(_ptr(self.gate), _ptr(self.up), _ptr(self.down))


def coli_moe_dense_workspace_bytes(shape: Shape) -> int:
    cs = shape.c()
    return lib().coli_moe_dense_workspace_bytes(C.byref(cs))


def coli_moe_dense_ffn(shape: Shape, x, weights: DenseWeights, y, residual=None, y_bf16=None,
                       ws=None, ws_bytes=None, stream=None) -> None:
    cs, cw = shape.c(), weights.c()
    _check(lib().coli_moe_dense_ffn(C.byref(cs), _ptr(x), C.byref(cw), _ptr(residual), _ptr(y),
                                    _ptr(y_bf16), _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)),
           "coli_moe_dense_ffn")


def _event_handle(ev, record_on=None):
    """torch.cuda.Event (or a raw hipEvent_t int, or None) -> handle.

    torch creates an event's handle when it is first recorded.  An event the
    library will record (record_on = that stream) is recorded there once
    first, which creates it; an event to wait for that was never recorded has
    nothing to wait for and is passed as NULL."""
    if ev is None or isinstance(ev, int):
        return ev
    if ev.cuda_event == 0:
        if record_on is None:
            return None
        ev.record(record_on)
    return ev.cuda_event


def coli_moe_bank_fill(shape: Shape, host, bank, experts=None, int4: bool = False, group: int = 32,
                       copy_stream=None, wait_event=None, ready_event=None) -> None:
    """Copy the listed experts (host ints; None = all) of `host` tensors (pinned) into `bank`."""
    n_t = 6 if int4 else 3
    if len(host) != n_t or len(bank) != n_t:
        raise ValueError(f"{n_t} tensors expected")
    cs = shape.c()
    h = (C.c_void_p * n_t)(*[_ptr(t) for t in host])
    b = (C.c_void_p * n_t)(*[_ptr(t) for t in bank])
    if experts is None:
        ex, n = None, 0
    else:
        ex = (C.c_int32 * len(experts))(*[int(e) for e in experts])
        n = len(experts)
    import torch
    cstream = copy_stream if copy_stream is not None else torch.cuda.current_stream()
    _check(lib().coli_moe_bank_fill(C.byref(cs), 1 if int4 else 0, group, h, b, ex, n,
                                    _stream(cstream), _event_handle(wait_event),
                                    _event_handle(ready_event, cstream)), "coli_moe_bank_fill")


def coli_moe_bank_acquire(compute_stream, ready_event) -> None:
    _check(lib().coli_moe_bank_acquire(_stream(compute_stream), _event_handle(ready_event)),
           "coli_moe_bank_acquire")


def coli_moe_bank_release(compute_stream, free_event) -> None:
    import torch
    cstream = compute_stream if compute_stream is not None else torch.cuda.current_stream()
    _check(lib().coli_moe_bank_release(_stream(cstream), _event_handle(free_event, cstream)),
           "coli_moe_bank_release")


def coli_index_topk_workspace_bytes(rows: int, L: int, k: int) -> int:
    return lib().coli_index_topk_workspace_bytes(rows, L, k)


def coli_index_topk(scores, k: int, idx, tail: int = 0, lens=None, ws=None, ws_bytes=None,
                    stream=None, L: Optional[int] = None, ld: Optional[int] = None) -> None:
    """scores: fp32 [rows][ld] device tensor (L columns used); idx: int32 [rows][k]."""
    rows = scores.shape[0]
    ld = scores.stride(0) if ld is None else ld
    L = scores.shape[1] if L is None else L
    _check(lib().coli_index_topk(scores.data_ptr(), rows, L, ld, _ptr(lens), k, tail, _ptr(idx),
                                 _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)),
           "coli_index_topk")


NOALLOC_SCRATCH_BYTES = 32 << 20


def coli_moe_ffn_noalloc(shape: Shape, x, routing: Routing, weights: Weights, y, residual=None,
                         y_bf16=None, stream=None) -> None:
    """coli_moe_ffn with the library's own per-GPU scratch array as workspace."""
    cs, cr, cw = shape.c(), routing.c(), weights.c()
    _check(lib().coli_moe_ffn_noalloc(C.byref(cs), _ptr(x), C.byref(cr), C.byref(cw), _ptr(residual),
                                      _ptr(y), _ptr(y_bf16), _stream(stream)), "coli_moe_ffn_noalloc")
