"""coli_moe_ffn_noalloc (workspace from the library's per-GPU scratch array)
against coli_moe_ffn with a caller workspace: bitwise equal outputs on two
calls in a row, the second with a smaller batch.  (A shape too large for the
array is rejected on the host: tests/test_abi.py.)"""
import numpy as np
import pytest

import synth
from sparse_moe_ffn_coli_amd import COLI_BF16, coli_moe_ffn, coli_moe_ffn_noalloc
from sparse_moe_ffn_coli_amd.layer import DeviceLayer, to_device

pytestmark = pytest.mark.gpu


def _both(W, cfg, T):
    import torch
    D, E, K, F = cfg["D"], cfg["E"], cfg["K"], cfg["F"]
    layer = DeviceLayer(W, T, D, E, K, F, COLI_BF16)
    x = to_device(W["x"][:T])
    layer.route(x)
    res = torch.from_numpy(np.random.default_rng(T).standard_normal((T, D)).astype(np.float32)).cuda()
    outs = []
    for noalloc in (False, True):
        y = res.clone()
        yb = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
        if noalloc:
            coli_moe_ffn_noalloc(layer.shape, x, layer.routing, layer.weights, y, residual=y, y_bf16=yb)
        else:
            coli_moe_ffn(layer.shape, x, layer.routing, layer.weights, y, residual=y, y_bf16=yb, ws=layer.ws)
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), yb.view(torch.int16).cpu().numpy()))
    return outs


def test_noalloc_matches_workspace_entry_point():
    cfg = synth.CONFIGS["decode"]
    W = synth.workload("decode")
    for T in (64, 17):                            # the second call is smaller
        (y0, b0), (y1, b1) = _both(W, cfg, T)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"T={T}: y differs"
        assert np.array_equal(b0, b1), f"T={T}: y_bf16 differs"
        print(f"noalloc T={T}: bitwise equal to the workspace entry point", flush=True)
