"""Device-resident routed-MoE layer: owns the device tensors of one layer
(router, bias, routed and shared experts), the routing buffers and the
workspace, and calls the C ABI.  Allocation and argument passing only; all
arithmetic is in the library's kernels."""
from __future__ import annotations

import numpy as np

from . import (COLI_BF16, COLI_F32, Routing, Shape, Weights, WeightsInt4, coli_moe_ffn,
               coli_moe_ffn_int4, coli_moe_route, coli_moe_workspace_bytes)


def to_device(a, device="cuda"):
    """numpy -> torch on `device`; uint16 arrays are bf16/fp16 bit patterns and
    are moved as int16 (callers view them as the right floating type)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    """One MoE layer on the GPU.

    ``W`` holds numpy arrays as produced by ``synth.layer_weights`` (bf16 as
    uint16 bits, fp32 as float32, int4 as packed uint8 + fp16 bits).
    """

    def __init__(self, W: dict, T: int, D: int, E: int, K: int, F: int, dtype: int,
                 device="cuda", group: int = 32):
        import torch
        self.shape = Shape(T, D, E, K, F, dtype)
        self.device = device
        dev = lambda a: to_device(a, device)
        self.wr = dev(W["wr"])
        self.bias = dev(W["bias"])
        self.int4 = "gate_q" in W
        if self.int4:
            self.weights = WeightsInt4(dev(W["gate_q"]), dev(W["up_q"]), dev(W["down_q"]),
                                       dev(W["gate_s"]), dev(W["up_s"]), dev(W["down_s"]), group,
                                       dev(W["s_gate"]), dev(W["s_up"]), dev(W["s_down"]))
        else:
            self.weights = Weights(dev(W["gate"]), dev(W["up"]), dev(W["down"]),
                                   dev(W["s_gate"]), dev(W["s_up"]), dev(W["s_down"]))
        self.routing = Routing.empty(T, E, K, device)
        nbytes = coli_moe_workspace_bytes(self.shape, self.int4)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        self.y = torch.empty((T, D), dtype=torch.float32, device=device)

    def route(self, x, stream=None, events=None):
        coli_moe_route(self.shape, x, self.wr, self.bias, self.routing, self.ws, stream=stream,
                       events=events)

    def ffn(self, x, y=None, residual=None, y_bf16=None, stream=None, events=None):
        y = self.y if y is None else y
        if self.int4:
            coli_moe_ffn_int4(self.shape, x, self.routing, self.weights, y, residual=residual,
                              y_bf16=y_bf16, ws=self.ws, stream=stream, events=events)
        else:
            coli_moe_ffn(self.shape, x, self.routing, self.weights, y, residual=residual,
                         y_bf16=y_bf16, ws=self.ws, stream=stream, events=events)
        return y

    def __call__(self, x, y=None, residual=None, y_bf16=None, stream=None, route_events=None,
                 ffn_events=None):
        self.route(x, stream, route_events)
        return self.ffn(x, y, residual, y_bf16, stream, ffn_events)

    def routing_numpy(self) -> dict:
        r = self.routing
        return {k: getattr(r, k).cpu().numpy() for k in ("ids", "w", "count", "offset", "perm", "inv")}


__all__ = ["DeviceLayer", "to_device", "COLI_BF16", "COLI_F32"]
