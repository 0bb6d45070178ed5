"""CPU checks of the C ABI library: it loads, exports every function that
include/coli_moe.h declares, sizes workspaces, and rejects invalid arguments
on the host before any device work (fake device addresses are used; none is
ever dereferenced because every case fails validation first, and those cases
are skipped on hosts with a GPU)."""
import ctypes as C
import os
import re

import pytest

import sparse_moe_ffn_coli_amd as pkg
from sparse_moe_ffn_coli_amd import (COLI_BF16, COLI_F32, CRouting, CShape, CWeights,
                                     CWeightsInt4)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli_moe.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WS, E_DEVICE, E_LAUNCH, E_ALIAS = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coli_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pkg.lib()
    names = declared_functions()
    assert set(names) >= {"coli_moe_route", "coli_moe_ffn", "coli_moe_ffn_int4",
                          "coli_moe_workspace_bytes", "coli_moe_status_str"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(pkg.EXPORTED)


def test_status_strings():
    for code in range(10):
        s = pkg.coli_moe_status_str(code)
        assert isinstance(s, str) and s
    assert pkg.coli_moe_status_str(0) == "ok"
    assert pkg.coli_moe_version() >= 100


def _shape(T=64, D=2048, E=288, K=8, F=768, dt=COLI_BF16):
    return pkg.Shape(T, D, E, K, F, dt)


def test_workspace_sizes():
    s = _shape()
    n = pkg.coli_moe_workspace_bytes(s)
    R = 64 * 8
    assert n >= (R + 64) * 768 * 2 + R * 2048 * 2          # h and o in bf16
    assert pkg.coli_moe_workspace_bytes(_shape(T=4096)) > n
    assert pkg.coli_moe_workspace_bytes(_shape(K=9)) == 0   # invalid shape -> 0
    assert pkg.coli_moe_workspace_bytes(_shape(T=0)) > 0


# fake, 256-aligned device addresses; never dereferenced.  Every case below
# that passes them must fail a host check before the library reaches the
# device; so that a regression in those checks can never hand such addresses
# to a real GPU, the cases run only on hosts without one (counting devices
# does not initialise the GPU runtime).
BASE = 0x7F0000000000


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0


no_gpu = pytest.mark.skipif(_gpu_present(), reason="fake device addresses must not reach a GPU")


def fake(i, misalign=0):
    return BASE + i * (1 << 32) + misalign


def _routing(misalign=0):
    return CRouting(*(fake(20 + i, misalign if i == 0 else 0) for i in range(6)))


def _route(shape, x=fake(1), wr=fake(2), bias=fake(3), routing=None, ws=fake(4), ws_bytes=1 << 31):
    routing = routing if routing is not None else _routing()
    cs = shape if isinstance(shape, CShape) else shape.c()
    return pkg.lib().coli_moe_route(C.byref(cs), x, wr, bias, C.byref(routing), ws, ws_bytes, None)


def _weights(misalign=0):
    return CWeights(*(fake(40 + i, misalign if i == 2 else 0) for i in range(6)))


def _ffn(shape, x=fake(1), routing=None, w=None, residual=None, y=fake(5), y_bf16=None,
         ws=fake(4), ws_bytes=1 << 31):
    routing = routing if routing is not None else _routing()
    w = w if w is not None else _weights()
    cs = shape.c()
    return pkg.lib().coli_moe_ffn(C.byref(cs), x, C.byref(routing), C.byref(w), residual, y,
                                  y_bf16, ws, ws_bytes, None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(K=0), E_SHAPE), (dict(K=9), E_SHAPE), (dict(E=7), E_SHAPE), (dict(E=1025), E_SHAPE),
    (dict(D=100), E_SHAPE), (dict(F=96), E_SHAPE), (dict(T=-1), E_SHAPE), (dict(D=0), E_SHAPE),
    (dict(dt=2), E_DTYPE)])
def test_route_rejects_bad_shapes(kw, code):
    assert _route(_shape(**kw)) == code


@no_gpu
def test_route_rejects_null_misaligned_small_workspace():
    assert pkg.lib().coli_moe_route(None, fake(1), fake(2), fake(3), C.byref(_routing()),
                                    fake(4), 1 << 31, None) == E_NULL
    assert _route(_shape(), x=None) == E_NULL
    assert _route(_shape(), bias=None) == E_NULL
    assert _route(_shape(), routing=CRouting(0, 0, 0, 0, 0, 0)) == E_NULL
    assert _route(_shape(), x=fake(1, 2)) == E_ALIGN
    assert _route(_shape(), routing=_routing(misalign=8)) == E_ALIGN
    assert _route(_shape(), ws_bytes=16) == E_WS


@no_gpu
def test_ffn_rejects_bad_arguments():
    s = _shape()
    assert _ffn(_shape(K=0)) == E_SHAPE
    assert _ffn(s, y=None) == E_NULL
    assert _ffn(s, w=CWeights(0, 0, 0, 0, 0, 0)) == E_NULL
    assert _ffn(s, w=_weights(misalign=4)) == E_ALIGN
    assert _ffn(s, residual=fake(6, 8)) == E_ALIGN
    assert _ffn(_shape(dt=COLI_F32), y_bf16=fake(7)) == E_DTYPE     # bf16 copy of an fp32 layer
    assert _ffn(s, y=fake(1) + 1024) == E_ALIAS                      # y inside x
    assert _ffn(s, y_bf16=fake(5) + 4096) == E_ALIAS                 # y_bf16 inside y
    assert _ffn(s, residual=fake(5) + 256) == E_ALIAS                # partial overlap with y
    assert _ffn(s, ws_bytes=1000) == E_WS
    # outputs against every other buffer of the call
    assert _ffn(s, ws=fake(20) + 256) == E_ALIAS                     # workspace over ids
    assert _ffn(s, ws=fake(24) - 1024) == E_ALIAS                    # workspace runs into perm
    assert _ffn(s, residual=fake(4) + 4096) == E_ALIAS               # residual inside the workspace
    assert _ffn(s, y_bf16=fake(21)) == E_ALIAS                       # y_bf16 over the weights w
    assert _ffn(s, y=fake(42) + 512) == E_ALIAS                      # y over the down weights
    assert _ffn(s, residual=fake(5)) == E_DEVICE                     # in place is fine (no GPU: last check)


@no_gpu
def test_route_rejects_overlapping_outputs():
    s = _shape()
    r = _routing()
    r.perm = r.ids + 512                                             # perm overlaps ids
    assert _route(s, routing=r) == E_ALIAS
    assert _route(s, ws=fake(1) + 256) == E_ALIAS                    # workspace over x
    assert _route(s, ws=fake(22) - 512) == E_ALIAS                   # workspace runs into count
    r2 = _routing()
    r2.count = fake(3)                                               # count written over bias
    assert _route(s, routing=r2) == E_ALIAS
    assert _route(s) == E_DEVICE                                     # no GPU here: last check


@no_gpu
def test_int4_rejects_fp32_and_null():
    cs = _shape(dt=COLI_F32).c()
    w = CWeightsInt4(*([fake(50 + i) for i in range(6)] + [32] + [fake(60 + i) for i in range(3)]))
    assert pkg.lib().coli_moe_ffn_int4(C.byref(cs), fake(1), C.byref(_routing()), C.byref(w),
                                       None, fake(5), None, fake(4), 1 << 31, None) == E_DTYPE
    cs2 = _shape().c()
    assert pkg.lib().coli_moe_ffn_int4(C.byref(cs2), fake(1), C.byref(_routing()), None,
                                       None, fake(5), None, fake(4), 1 << 31, None) == E_NULL


@no_gpu
def test_int4_alias_checks_cover_every_weight():
    cs = _shape().c()
    ws = [fake(50 + i) for i in range(6)] + [32] + [fake(60 + i) for i in range(3)]

    def call(y=fake(5), ws_ptr=fake(4)):
        w = CWeightsInt4(*ws)
        return pkg.lib().coli_moe_ffn_int4(C.byref(cs), fake(1), C.byref(_routing()), C.byref(w),
                                           None, y, None, ws_ptr, 1 << 31, None)
    assert call() == E_DEVICE                                        # valid: reaches the device query
    assert call(y=fake(53) + 64) == E_ALIAS                          # y over the gate scales
    assert call(ws_ptr=fake(62) + 256) == E_ALIAS                    # workspace over the shared down
    assert call(y=fake(60)) == E_ALIAS                               # y over the shared gate


@no_gpu
def test_noalloc_rejects_shapes_beyond_its_scratch_array():
    big = _shape(T=4096)
    assert pkg.coli_moe_workspace_bytes(big) > pkg.NOALLOC_SCRATCH_BYTES
    cs = big.c()
    assert pkg.lib().coli_moe_ffn_noalloc(C.byref(cs), fake(1), C.byref(_routing()), C.byref(_weights()),
                                          None, fake(5), None, None) == E_WS
    cs = _shape(T=64).c()                                            # fits: reaches the device query
    assert pkg.lib().coli_moe_ffn_noalloc(C.byref(cs), fake(1), C.byref(_routing()), C.byref(_weights()),
                                          None, fake(5), None, None) == E_DEVICE


@no_gpu
def test_int4_rejects_bad_groups():
    cs = _shape().c()
    for g in (0, 16, 48, 4096):
        w = CWeightsInt4(*([fake(50 + i) for i in range(6)] + [g] + [fake(60 + i) for i in range(3)]))
        assert pkg.lib().coli_moe_ffn_int4(C.byref(cs), fake(1), C.byref(_routing()), C.byref(w),
                                           None, fake(5), None, fake(4), 1 << 31, None) == E_SHAPE


@no_gpu
def test_valid_call_without_gpu_reports_device_error():
    # Only meaningful on a host with no GPU: there the last host check, the
    # device query, fails.  Never run it where a GPU could receive the fake
    # addresses.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake addresses must not reach it")
    assert _route(_shape()) == E_DEVICE
    assert _ffn(_shape()) == E_DEVICE
