"""Double-banked device expert cache ("feat(glm53): add device-resident HIP
backend for MI350P", section "Key changes": a double-banked device expert
cache with event-based publication): layers whose routed experts are copied
from pinned host memory into one of two device banks on a copy stream, while
the previous layer computes from the other bank, give bitwise the same
results as layers reading resident weights."""
import numpy as np
import pytest

import synth
from sparse_moe_ffn_coli_amd import (COLI_BF16, ColiError, Routing, Shape, Weights, WeightsInt4,
                                     coli_moe_bank_acquire, coli_moe_bank_fill,
                                     coli_moe_bank_release, coli_moe_ffn, coli_moe_ffn_int4,
                                     coli_moe_route, coli_moe_workspace_bytes)
from sparse_moe_ffn_coli_amd.layer import DeviceLayer, to_device

pytestmark = pytest.mark.gpu

ROUTED = {False: ("gate", "up", "down"), True: ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")}


def _pinned(a):
    import torch
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    p.copy_(t)
    return p


def _run_chain(cfgs, layers, x0, banked):
    """Chain of layers (y of one layer, rounded to bf16, feeds the next)."""
    import torch
    cfg = cfgs
    T, D, E, K, F = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"]
    int4 = cfg.get("int4", False)
    shape = Shape(T, D, E, K, F, COLI_BF16)
    names = ROUTED[int4]
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    ws = torch.empty(coli_moe_workspace_bytes(shape, int4), dtype=torch.uint8, device="cuda")
    routing = Routing.empty(T, E, K)
    dev = [{k: to_device(W[k]) for k in ("wr", "bias", "s_gate", "s_up", "s_down")} for W in layers]
    if banked:
        host = [[_pinned(W[k]) for k in names] for W in layers]
        banks = [[torch.empty_like(h, device="cuda") for h in host[0]] for _ in range(2)]
        ready = [torch.cuda.Event() for _ in range(2)]
        free = [torch.cuda.Event() for _ in range(2)]
        freed = [False, False]
        def fill(l):
            b = l % 2
            coli_moe_bank_fill(shape, host[l], banks[b], int4=int4, group=cfg.get("group", 32),
                               copy_stream=copy, wait_event=free[b] if freed[b] else None,
                               ready_event=ready[b])
        fill(0)
    else:
        resident = [{k: to_device(W[k]) for k in names} for W in layers]
    x = to_device(x0)
    outs = []
    for l, W in enumerate(layers):
        d = dev[l]
        if banked:
            if l + 1 < len(layers):
                fill(l + 1)                       # the next layer's experts, into the other bank
            coli_moe_bank_acquire(compute, ready[l % 2])
            routed = dict(zip(names, banks[l % 2]))
        else:
            routed = resident[l]
        y = torch.empty((T, D), dtype=torch.float32, device="cuda")
        yb = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
        coli_moe_route(shape, x, d["wr"], d["bias"], routing, ws)
        if int4:
            w = WeightsInt4(routed["gate_q"], routed["up_q"], routed["down_q"], routed["gate_s"],
                            routed["up_s"], routed["down_s"], cfg["group"], d["s_gate"], d["s_up"], d["s_down"])
            coli_moe_ffn_int4(shape, x, routing, w, y, y_bf16=yb, ws=ws)
        else:
            w = Weights(routed["gate"], routed["up"], routed["down"], d["s_gate"], d["s_up"], d["s_down"])
            coli_moe_ffn(shape, x, routing, w, y, y_bf16=yb, ws=ws)
        if banked:
            coli_moe_bank_release(compute, free[l % 2])
            freed[l % 2] = True
        outs.append(y)
        x = yb.view(torch.int16)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


@pytest.mark.parametrize("int4", [False, True])
def test_banked_layers_match_resident_weights(int4):
    cfg = dict(cid=301 + int(int4), T=96, D=256, E=40, K=8, F=192, dtype="bf16", bias="uniform",
               layers=4, int4=int4, group=32)
    layers = [synth.layer_weights(cfg, l) for l in range(4)]
    x0 = synth.x_rows(cfg)
    a = _run_chain(cfg, layers, x0, banked=False)
    b = _run_chain(cfg, layers, x0, banked=True)
    for l, (ya, yb) in enumerate(zip(a, b)):
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), f"layer {l} differs"
    print(f"int4={int4}: 4 banked layers bitwise equal to resident ones", flush=True)


def test_bank_fill_selected_experts():
    import torch
    cfg = dict(cid=303, T=8, D=128, E=24, K=8, F=64, dtype="bf16", bias="uniform", layers=1, int4=False)
    W = synth.layer_weights(cfg)
    shape = Shape(8, 128, 24, 8, 64, COLI_BF16)
    host = [_pinned(W[k]) for k in ROUTED[False]]
    bank = [torch.full(h.shape, 0x7777, dtype=torch.int16, device="cuda") for h in host]
    chosen = [0, 1, 2, 7, 9, 10, 23]             # three runs and two single experts
    done = torch.cuda.Event()
    coli_moe_bank_fill(shape, host, bank, experts=chosen, copy_stream=torch.cuda.Stream(), ready_event=done)
    done.synchronize()
    for h, b in zip(host, bank):
        bn, hn = b.cpu().numpy(), h.numpy()
        for e in range(24):
            if e in chosen:
                assert np.array_equal(bn[e], hn[e])
            else:
                assert (bn[e] == 0x7777).all()


def test_bank_fill_rejects_wrong_memory_and_lists():
    import torch
    shape = Shape(8, 128, 24, 8, 64, COLI_BF16)
    dev = [torch.empty((24, 64, 128), dtype=torch.int16, device="cuda") for _ in range(3)]
    dev[2] = torch.empty((24, 128, 64), dtype=torch.int16, device="cuda")
    pageable = [torch.empty(d.shape, dtype=torch.int16) for d in dev]
    pinned = [torch.empty(d.shape, dtype=torch.int16, pin_memory=True) for d in dev]
    with pytest.raises(ColiError) as e:
        coli_moe_bank_fill(shape, pageable, dev, copy_stream=torch.cuda.current_stream())
    assert e.value.code == 9
    with pytest.raises(ColiError) as e:
        coli_moe_bank_fill(shape, pinned, pinned, copy_stream=torch.cuda.current_stream())
    assert e.value.code in (8, 9)
    for bad in ([3, 3], [24], [-1]):
        with pytest.raises(ColiError) as e:
            coli_moe_bank_fill(shape, pinned, dev, experts=bad, copy_stream=torch.cuda.current_stream())
        assert e.value.code == 2
