"""ctypes front end of the CPU oracle (``oracle/liboracle.so``).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the product package
never does.  The oracle shares no code with the HIP library.

Arrays are numpy arrays; bf16 tensors are ``uint16`` bit patterns, fp16 scale
tensors are ``uint16`` bit patterns, int4 tensors are packed ``uint8`` (low
nibble = even reduction index).  All arithmetic happens in the C library in
double precision; this module only marshals arguments.

Page citations used in this directory:
  [glm5next]  "Add GLM-5.3-Flash (glm5next) support with ROCmFP mix qtypes
              (105/106)", sections "Architecture" and "MoE FFN".
  [glm53-hip] "feat(glm53): add device-resident HIP backend for MI350P",
              section "Key changes" (offset-binary int4, deterministic top-k).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, INT4 = 0, 1, 2


class OrcMat(C.Structure):
    _fields_ = [("kind", C.c_int), ("data", C.c_void_p),
                ("scales", C.c_void_p), ("group", C.c_int)]


def build(force: bool = False) -> str:
    """Compile liboracle.so with the Makefile beside this file."""
    args = ["make", "-s", "-C", _HERE]
    if force:
        args.insert(1, "-B")
    subprocess.run(args, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        d, i64, i32 = C.c_double, C.c_int64, C.c_int
        vp = C.c_void_p
        mp = C.POINTER(OrcMat)
        L.oracle_sigmoid.restype = d
        L.oracle_sigmoid.argtypes = [d]
        L.oracle_silu.restype = d
        L.oracle_silu.argtypes = [d]
        L.oracle_swiglu.restype = d
        L.oracle_swiglu.argtypes = [d, d]
        L.oracle_bf16_to_double.restype = d
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_fp16_to_double.restype = d
        L.oracle_fp16_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_from_double.restype = C.c_uint16
        L.oracle_bf16_from_double.argtypes = [d]
        L.oracle_mat_elem.restype = d
        L.oracle_mat_elem.argtypes = [mp, i64, i64, i64, i64, i64]
        L.oracle_router_logits.restype = i32
        L.oracle_router_logits.argtypes = [i64, i64, i64, mp, mp, vp, vp]
        L.oracle_select_topk.restype = i32
        L.oracle_select_topk.argtypes = [i64, i64, i32, vp, vp, vp]
        L.oracle_permutation.restype = i32
        L.oracle_permutation.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp]
        L.oracle_expert_hidden.restype = i32
        L.oracle_expert_hidden.argtypes = [i64, i64, vp, mp, mp, i64, i64, vp]
        L.oracle_expert_down.restype = i32
        L.oracle_expert_down.argtypes = [i64, i64, vp, mp, i64, i64, vp]
        L.oracle_moe_ffn.restype = i32
        L.oracle_moe_ffn.argtypes = [i64, i64, i64, i32, i64, mp, vp, vp,
                                     mp, mp, mp, mp, mp, mp, vp, vp, i64, vp]
        L.oracle_residual_layer.restype = i32
        L.oracle_residual_layer.argtypes = [i64, i64, i64, i32, i64, vp, mp, vp,
                                            mp, mp, mp, mp, mp, mp,
                                            vp, vp, vp, vp, vp, vp]
        L.oracle_dense_ffn.restype = i32
        L.oracle_dense_ffn.argtypes = [i64, i64, i64, mp, mp, mp, mp, vp, vp]
        L.oracle_index_topk.restype = i32
        L.oracle_index_topk.argtypes = [i64, i64, i64, vp, vp, i64, i64, vp]
        L.oracle_num_threads.restype = i32
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


# --------------------------------------------------------------------------
# operand wrapping
# --------------------------------------------------------------------------

class Mat:
    """A stacked operand [n_mat][rows][K] in one of the three encodings.

    ``Mat.f32(a)``  float32 array;  ``Mat.bf16(bits)`` uint16 bf16 bits;
    ``Mat.int4(q, s, group)`` packed nibbles + fp16 scale bits.
    Keeps references to the arrays so they outlive the C call.
    """

    def __init__(self, kind, data, scales=None, group=0):
        self.kind = kind
        self.data = np.ascontiguousarray(data)
        self.scales = None if scales is None else np.ascontiguousarray(scales)
        self.group = int(group)
        self.s = OrcMat(kind, self.data.ctypes.data,
                        None if self.scales is None else self.scales.ctypes.data,
                        self.group)

    @staticmethod
    def f32(a):
        a = np.asarray(a)
        assert a.dtype == np.float32
        return Mat(F32, a)

    @staticmethod
    def bf16(bits):
        bits = np.asarray(bits)
        assert bits.dtype == np.uint16
        return Mat(BF16, bits)

    @staticmethod
    def int4(q, s, group):
        q = np.asarray(q)
        s = np.asarray(s)
        assert q.dtype == np.uint8 and s.dtype == np.uint16
        return Mat(INT4, q, s, group)

    @staticmethod
    def auto(a):
        """float32 -> F32, uint16 -> BF16 bits."""
        a = np.asarray(a)
        if a.dtype == np.float32:
            return Mat.f32(a)
        if a.dtype == np.uint16:
            return Mat.bf16(a)
        raise TypeError(f"unsupported operand dtype {a.dtype}")

    def ref(self):
        return C.byref(self.s)


def _as_mat(a):
    return a if isinstance(a, Mat) else Mat.auto(a)


def _p(a):
    return a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def sigmoid(z: float) -> float:
    return lib().oracle_sigmoid(float(z))


def silu(a: float) -> float:
    return lib().oracle_silu(float(a))


def swiglu(g: float, u: float) -> float:
    return lib().oracle_swiglu(float(g), float(u))


def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(int(b))


def fp16_to_double(h: int) -> float:
    return lib().oracle_fp16_to_double(int(h))


def bf16_from_double(v: float) -> int:
    return lib().oracle_bf16_from_double(float(v))


def mat_elem(m: Mat, mat: int, rows: int, K: int, row: int, k: int) -> float:
    return lib().oracle_mat_elem(m.ref(), mat, rows, K, row, k)


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------

def router_logits(x, wr, bias, T, D, E):
    x, wr = _as_mat(x), _as_mat(wr)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    z = np.empty((T, E), np.float64)
    _check(lib().oracle_router_logits(T, D, E, x.ref(), wr.ref(), _p(bias), _p(z)),
           "router_logits")
    return z


def select_topk(z, K):
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, E = z.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    _check(lib().oracle_select_topk(T, E, K, _p(z), _p(ids), _p(w)), "select_topk")
    return ids, w


def permutation(ids, E):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    count = np.empty(E, np.int32)
    offset = np.empty(E + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    inv = np.empty(T * K, np.int32)
    _check(lib().oracle_permutation(T, E, K, _p(ids), _p(count), _p(offset),
                                    _p(perm), _p(inv)), "permutation")
    return count, offset, perm, inv


def expert_hidden(xrow, gate, up, e, D, F, n_mat):
    xrow = np.ascontiguousarray(xrow, dtype=np.float64)
    gate, up = _as_mat(gate), _as_mat(up)
    h = np.empty(F, np.float64)
    _check(lib().oracle_expert_hidden(D, F, _p(xrow), gate.ref(), up.ref(), n_mat, e,
                                      _p(h)), "expert_hidden")
    return h


def expert_down(h, down, e, D, F, n_mat):
    h = np.ascontiguousarray(h, dtype=np.float64)
    down = _as_mat(down)
    o = np.empty(D, np.float64)
    _check(lib().oracle_expert_down(D, F, _p(h), down.ref(), n_mat, e, _p(o)),
           "expert_down")
    return o


def moe_ffn(x, ids, w, gate, up, down, s_gate, s_up, s_down, T, D, E, K, F,
            residual=None, tokens=None):
    """y[i] for token tokens[i] (all tokens when ``tokens`` is None)."""
    x = _as_mat(x)
    mats = [_as_mat(a) for a in (gate, up, down, s_gate, s_up, s_down)]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.float64)
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        n = len(tokens)
    else:
        n = T
    y = np.empty((n, D), np.float64)
    _check(lib().oracle_moe_ffn(
        T, D, E, K, F, x.ref(), _p(ids), _p(w), *[m.ref() for m in mats],
        None if residual is None else _p(residual),
        None if tokens is None else _p(tokens), n, _p(y)), "moe_ffn")
    return y


def moe_layer(x, wr, bias, gate, up, down, s_gate, s_up, s_down, T, D, E, K, F,
              residual=None, tokens=None):
    """Route all T tokens, then the FFN for ``tokens`` (default all).

    Returns a dict with z, ids, w, count, offset, perm, inv and y.
    """
    z = router_logits(x, wr, bias, T, D, E)
    ids, w = select_topk(z, K)
    count, offset, perm, inv = permutation(ids, E)
    y = moe_ffn(x, ids, w, gate, up, down, s_gate, s_up, s_down, T, D, E, K, F,
                residual=residual, tokens=tokens)
    return dict(z=z, ids=ids, w=w, count=count, offset=offset, perm=perm, inv=inv, y=y)


def residual_layer(x, wr, bias, gate, up, down, s_gate, s_up, s_down, D, E, K, F):
    """One layer of the stacked chain on rows ``x`` (float64 [n][D]).

    The layer input is bf16_rne(x); returns (xin_bf16, ids, w, z, y, x_next).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = x.shape[0]
    wr = _as_mat(wr)
    mats = [_as_mat(a) for a in (gate, up, down, s_gate, s_up, s_down)]
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    xin = np.empty((n, D), np.uint16)
    ids = np.empty((n, K), np.int32)
    w = np.empty((n, K), np.float64)
    z = np.empty((n, E), np.float64)
    y = np.empty((n, D), np.float64)
    xn = np.empty((n, D), np.float64)
    _check(lib().oracle_residual_layer(n, D, E, K, F, _p(x), wr.ref(), _p(bias),
                                       *[m.ref() for m in mats], _p(xin), _p(ids),
                                       _p(w), _p(z), _p(y), _p(xn)), "residual_layer")
    return xin, ids, w, z, y, xn


def dense_ffn(x, gate, up, down, T, D, F, residual=None):
    """Dense FFN layer: y = residual + W_down swiglu(W_gate x, W_up x) for all T rows."""
    x = _as_mat(x)
    mats = [_as_mat(a) for a in (gate, up, down)]
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.float64)
    y = np.empty((T, D), np.float64)
    _check(lib().oracle_dense_ffn(T, D, F, x.ref(), *[m.ref() for m in mats],
                                  None if residual is None else _p(residual), _p(y)),
           "dense_ffn")
    return y


def index_topk(scores, k, tail=0, lens=None):
    """Selected positions per row of ``scores`` (float32 [rows][L]), ascending, -1 padded."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    rows, L = scores.shape
    if lens is not None:
        lens = np.ascontiguousarray(lens, dtype=np.int32)
    idx = np.empty((rows, k), np.int32)
    _check(lib().oracle_index_topk(rows, L, L, _p(scores) if rows else None,
                                   None if lens is None else _p(lens), k, tail,
                                   _p(idx) if rows else None), "index_topk")
    return idx


def sigma_gap(z, K):
    """Per row: sigmoid(8th largest logit) - sigmoid(9th largest), via the oracle's
    own ranking and sigmoid (used to filter generated inputs)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, E = z.shape
    ids, _ = select_topk(z, K + 1) if E > K else (None, None)
    if ids is None:
        return np.full(T, np.inf)
    out = np.empty(T)
    for t in range(T):
        chosen = ids[t]
        zz = sorted(((z[t, e], -int(e)) for e in chosen), reverse=True)
        out[t] = sigmoid(zz[K - 1][0]) - sigmoid(zz[K][0])
    return out
