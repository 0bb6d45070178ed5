"""Seeded synthetic inputs for the routed-MoE workloads (``synth/libsynth.so``).

Shared by the oracle side (tests) and the GPU side (tests, smoke check,
benchmark).  It holds none of the layer's arithmetic: random streams,
storage rounding, nibble packing and the Zipf bias ranking only.

Workloads (shapes of the GLM-5.3-Flash MoE layer: 288 routed experts, top-8,
one shared expert, 42 MoE layers -- "Add GLM-5.3-Flash (glm5next) support with
ROCmFP mix qtypes (105/106)", section "Architecture"; model width 2048 and
expert width 768 are the workload definition's, the pages do not give them):

  tiny     T=8,    D=128,  F=64,  fp32 everything, bias U(-0.1, 0.1)
  decode   T=64,   D=2048, F=768, bf16, bias U(-0.1, 0.1)
  prefill  T=4096, D=2048, F=768, bf16, bias -1.1*ln(rank) (Zipf popularity)
  int4     T=512,  D=2048, F=768, int4 experts (group 32, fp16 scales
           U(0.005, 0.02), nibbles U{0..15}), router + shared expert bf16
  stacked  T=256,  D=2048, F=768, bf16, 42 layers with independent weights
  int4_decode  T=64, D=2048, F=768, int4 experts as in int4 (decode batch)

Dense FFN layers (the model's first layers run a dense FFN, same section):
  dense_decode   T=64,   D=2048, F=6912, bf16
  dense_prefill  T=4096, D=2048, F=6912, bf16
(the pages give no dense width; 6912 = 9 x 768 is the hidden width a token
activates in an MoE layer: 8 routed experts and the shared one.)

Index selection of the sparse attention ("MLA/DSA": top-2048 of the indexer
scores, the last kpool = 4 tokens always kept), fp32 scores ~ N(0, 1):
  index_topk         2048 query rows (a prefill chunk) over a 32768-entry
                     cache, causal: row i sees its first 30721 + i entries
  index_topk_decode  64 query rows, each over a full 32768-entry cache

Value recipe: x ~ N(0,1); router, gate, up ~ N(0, 1/D); down ~ N(0, 1/F);
shared expert likewise; seed 0.  Token rows can be redrawn ("attempts") so
that the gap between the 8th and 9th router probability exceeds 1e-3; the
attempt per token is chosen by a committed script with the oracle and stored
in ``tests/golden/gap_attempts.json``.
"""
from __future__ import annotations

import ctypes as C
import json
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
GAP_ATTEMPTS_PATH = os.path.join(_ROOT, "tests", "golden", "gap_attempts.json")

# tensor ids of the random streams
X, WR, BIAS, GATE, UP, DOWN, SGATE, SUP, SDOWN = 1, 2, 3, 4, 5, 6, 7, 8, 9
GATE_Q, UP_Q, DOWN_Q, GATE_S, UP_S, DOWN_S = 10, 11, 12, 13, 14, 15
DGATE, DUP, DDOWN, SCORES = 16, 17, 18, 19

CONFIGS = {
    "tiny": dict(cid=1, T=8, D=128, E=288, K=8, F=64, dtype="f32", bias="uniform",
                 layers=1, int4=False),
    "decode": dict(cid=2, T=64, D=2048, E=288, K=8, F=768, dtype="bf16", bias="uniform",
                   layers=1, int4=False),
    "prefill": dict(cid=3, T=4096, D=2048, E=288, K=8, F=768, dtype="bf16", bias="zipf",
                    layers=1, int4=False),
    "int4": dict(cid=4, T=512, D=2048, E=288, K=8, F=768, dtype="bf16", bias="uniform",
                 layers=1, int4=True, group=32),
    "stacked": dict(cid=5, T=256, D=2048, E=288, K=8, F=768, dtype="bf16", bias="uniform",
                    layers=42, int4=False),
    "int4_decode": dict(cid=6, T=64, D=2048, E=288, K=8, F=768, dtype="bf16", bias="uniform",
                        layers=1, int4=True, group=32),
}
DENSE_CONFIGS = {
    "dense_decode": dict(cid=7, T=64, D=2048, F=6912, dtype="bf16"),
    "dense_prefill": dict(cid=8, T=4096, D=2048, F=6912, dtype="bf16"),
}
INDEX_CONFIGS = {
    "index_topk": dict(cid=9, rows=2048, L=32768, k=2048, tail=4, lens="causal"),
    "index_topk_decode": dict(cid=10, rows=64, L=32768, k=2048, tail=4, lens="full"),
}
ZIPF_S = 1.1
GAP_MIN = 1e-3


def build(force: bool = False) -> str:
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
        u64, i64, d, vp = C.c_uint64, C.c_int64, C.c_double, C.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64, u64, u64]
        L.synth_normal.restype = None
        L.synth_normal.argtypes = [u64, i64, i64, i64, d, C.c_int, vp]
        L.synth_x_rows.restype = None
        L.synth_x_rows.argtypes = [u64, i64, i64, vp, C.c_int, vp]
        L.synth_uniform_f32.restype = None
        L.synth_uniform_f32.argtypes = [u64, i64, d, d, vp]
        L.synth_uniform_fp16.restype = None
        L.synth_uniform_fp16.argtypes = [u64, i64, i64, d, d, vp]
        L.synth_nibbles.restype = None
        L.synth_nibbles.argtypes = [u64, i64, i64, vp]
        L.synth_zipf_bias.restype = None
        L.synth_zipf_bias.argtypes = [u64, i64, d, vp]
        L.synth_bf16.restype = C.c_uint16
        L.synth_bf16.argtypes = [d]
        L.synth_fp16.restype = C.c_uint16
        L.synth_fp16.argtypes = [d]
        L.synth_num_threads.restype = C.c_int
        L.synth_num_threads.argtypes = []
        _lib = L
    return _lib


def key(cfg: dict, layer: int, tensor: int, seed: int = 0) -> int:
    return lib().synth_key(seed, cfg["cid"], layer, tensor)


def _kind(dtype):
    return 0 if dtype == "f32" else 1


def _np_dtype(dtype):
    return np.float32 if dtype == "f32" else np.uint16


def normal(k: int, rows: int, cols: int, scale: float, dtype: str, row0: int = 0):
    out = np.empty((rows, cols), _np_dtype(dtype))
    lib().synth_normal(k, rows, cols, row0, scale, _kind(dtype), out.ctypes.data)
    return out


def x_rows(cfg: dict, attempts=None, layer: int = 0, seed: int = 0, dtype=None):
    T, D = cfg["T"], cfg["D"]
    dtype = dtype or cfg["dtype"]
    out = np.empty((T, D), _np_dtype(dtype))
    att = None
    if attempts is not None:
        att = np.ascontiguousarray(attempts, dtype=np.int32)
        assert att.shape == (T,)
    lib().synth_x_rows(key(cfg, layer, X, seed), T, D,
                       None if att is None else att.ctypes.data, _kind(dtype), out.ctypes.data)
    return out


def bias(cfg: dict, layer: int = 0, seed: int = 0):
    E = cfg["E"]
    out = np.empty(E, np.float32)
    if cfg["bias"] == "zipf":
        lib().synth_zipf_bias(key(cfg, layer, BIAS, seed), E, ZIPF_S, out.ctypes.data)
    else:
        lib().synth_uniform_f32(key(cfg, layer, BIAS, seed), E, -0.1, 0.1, out.ctypes.data)
    return out


def int4_matrix(cfg: dict, layer: int, qtensor: int, stensor: int, n_mat: int, rows: int,
                K: int, seed: int = 0):
    G = cfg["group"]
    q = np.empty((n_mat, rows, K // 2), np.uint8)
    s = np.empty((n_mat, rows, K // G), np.uint16)
    lib().synth_nibbles(key(cfg, layer, qtensor, seed), n_mat * rows, K, q.ctypes.data)
    lib().synth_uniform_fp16(key(cfg, layer, stensor, seed), n_mat * rows, K // G, 0.005, 0.02,
                             s.ctypes.data)
    return q, s


def layer_weights(cfg: dict, layer: int = 0, seed: int = 0) -> dict:
    """Router, bias, routed experts and shared expert of one layer."""
    D, E, F, dt = cfg["D"], cfg["E"], cfg["F"], cfg["dtype"]
    sd, sf = 1.0 / math.sqrt(D), 1.0 / math.sqrt(F)
    W = dict(
        wr=normal(key(cfg, layer, WR, seed), E, D, sd, dt),
        bias=bias(cfg, layer, seed),
        s_gate=normal(key(cfg, layer, SGATE, seed), F, D, sd, dt),
        s_up=normal(key(cfg, layer, SUP, seed), F, D, sd, dt),
        s_down=normal(key(cfg, layer, SDOWN, seed), D, F, sf, dt),
    )
    if cfg["int4"]:
        W["gate_q"], W["gate_s"] = int4_matrix(cfg, layer, GATE_Q, GATE_S, E, F, D, seed)
        W["up_q"], W["up_s"] = int4_matrix(cfg, layer, UP_Q, UP_S, E, F, D, seed)
        W["down_q"], W["down_s"] = int4_matrix(cfg, layer, DOWN_Q, DOWN_S, E, D, F, seed)
    else:
        W["gate"] = normal(key(cfg, layer, GATE, seed), E * F, D, sd, dt).reshape(E, F, D)
        W["up"] = normal(key(cfg, layer, UP, seed), E * F, D, sd, dt).reshape(E, F, D)
        W["down"] = normal(key(cfg, layer, DOWN, seed), E * D, F, sf, dt).reshape(E, D, F)
    return W


def load_attempts(name: str, path: str = GAP_ATTEMPTS_PATH):
    """Per-token redraw index for workload ``name`` from the stored table
    (zeros when the table or the entry is absent)."""
    cfg = CONFIGS[name]
    att = np.zeros(cfg["T"], np.int32)
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
        for t, a in table.get(name, {}).get("attempts", {}).items():
            att[int(t)] = int(a)
    return att


def workload(name: str, layer: int = 0, seed: int = 0, attempts="stored") -> dict:
    """x (layer 0 only) plus the weights of one layer of workload ``name``."""
    cfg = CONFIGS[name]
    W = layer_weights(cfg, layer, seed)
    if layer == 0:
        if isinstance(attempts, str) and attempts == "stored":
            attempts = load_attempts(name)
        W["x"] = x_rows(cfg, attempts, 0, seed)
    return W


def bf16_bits(v: float) -> int:
    return lib().synth_bf16(v)


def fp16_bits(v: float) -> int:
    return lib().synth_fp16(v)


def dense_weights(cfg: dict, layer: int = 0, seed: int = 0) -> dict:
    """gate, up [F][D] ~ N(0, 1/D) and down [D][F] ~ N(0, 1/F) of a dense FFN layer, plus x."""
    D, F, dt = cfg["D"], cfg["F"], cfg["dtype"]
    sd, sf = 1.0 / math.sqrt(D), 1.0 / math.sqrt(F)
    return dict(gate=normal(key(cfg, layer, DGATE, seed), F, D, sd, dt),
                up=normal(key(cfg, layer, DUP, seed), F, D, sd, dt),
                down=normal(key(cfg, layer, DDOWN, seed), D, F, sf, dt),
                x=x_rows(cfg, None, layer, seed))


def index_scores(cfg: dict, seed: int = 0):
    """fp32 scores [rows][L] ~ N(0, 1) and the per-row valid lengths."""
    rows, L = cfg["rows"], cfg["L"]
    scores = normal(key(cfg, 0, SCORES, seed), rows, L, 1.0, "f32")
    if cfg["lens"] == "causal":
        lens = (L - rows + 1 + np.arange(rows)).astype(np.int32)
    else:
        lens = np.full(rows, L, np.int32)
    return scores, lens
