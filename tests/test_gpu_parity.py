"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
inputs: small shapes that span several tiles with ragged tails, the full
workloads (every token), edge cases, and run-to-run bitwise determinism.
Tolerances are in gpu_helpers."""
import numpy as np
import pytest

import synth
from gpu_helpers import compare, custom_cfg, gpu_layer, make_inputs, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_moe_ffn_coli_amd as pkg
    pkg.lib()


def _report(label, err):
    print(f"{label}: ids/perm bit-exact, w_err={err['w_err']:.2e}, y_err={err['y_err']:.2e}",
          flush=True)


# ---------------------------------------------------------------------------
# small shapes: several tiles, ragged tails, full oracle
# ---------------------------------------------------------------------------
SMALL = [
    # cid, T, D, E, K, F, dtype, router bias -- rows per expert decide the tile engine
    (101, 200, 256, 40, 8, 192, "bf16", "uniform"),   # 40 rows/expert: 256-row tiles, ragged
    (102, 100, 128, 288, 8, 128, "bf16", "uniform"),  # ~3 rows/expert: 32-row tiles
    (103, 67, 192, 24, 8, 64, "f32", "uniform"),
    (104, 130, 64, 16, 8, 64, "bf16", "uniform"),     # minimum widths, heavy load per expert
    (105, 600, 256, 48, 8, 192, "bf16", "zipf"),      # skewed: full, partial and <= 32-row tiles
    # batches above 512 tokens take the LDS-staged router: ring depth 2 (E=500) and 3 (E=300),
    # four reduction splits of four 64-wide steps each, ragged token blocks and expert fragments
    (106, 700, 1024, 500, 8, 64, "bf16", "uniform"),
    (107, 1000, 1024, 300, 8, 64, "bf16", "zipf"),
    # row-light tiles (32 x 128) with a ragged last down tile (D = 192) and three h-column tiles
    (108, 150, 192, 288, 8, 192, "bf16", "uniform"),
    # the 256 x 256 engine's streaming-mode boundary: experts average 64 rows, so tiles of
    # just under and just over 64 rows; the shared expert's last tile has 64 rows, then 65
    (109, 320, 128, 40, 8, 64, "bf16", "uniform"),
    (110, 321, 128, 40, 8, 64, "bf16", "uniform"),
]


# small batches at reduction widths of 512, 1024 and 2048: experts with several
# row tiles, a shared expert whose last tile is ragged, K = 4, int4 experts with
# groups of 32 and 64
SMALL_BATCH = [
    # cid, T, D, E, K, F, int4, group
    (140, 50, 512, 40, 8, 192, False, 32),
    (141, 37, 1024, 64, 8, 128, True, 32),
    (142, 131, 2048, 288, 8, 256, False, 32),
    (143, 71, 2048, 96, 8, 64, True, 64),
    (144, 9, 512, 16, 4, 64, True, 32),
]


@pytest.mark.parametrize("cid,T,D,E,K,F,int4,group", SMALL_BATCH)
def test_small_batches(cid, T, D, E, K, F, int4, group):
    cfg = custom_cfg(cid, T, D, E, K, F, "bf16", int4=int4, group=group)
    W = make_inputs(cfg)
    _report(f"small batch cid={cid} int4={int4}", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label=f"cid={cid}"))


@pytest.mark.parametrize("cid,T,D,E,K,F,dt,bias", SMALL)
def test_small_shapes(cid, T, D, E, K, F, dt, bias):
    cfg = custom_cfg(cid, T, D, E, K, F, dt, bias=bias)
    W = make_inputs(cfg)
    got = run_gpu(W, cfg)
    ref = run_oracle(W, cfg)
    _report(f"small cid={cid} counts {sorted(ref['count'].tolist())[-3:]}..{sorted(ref['count'].tolist())[:3]}",
            compare(got, ref, cfg, label=f"cid={cid}"))


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------
def test_tiny_fp32():
    cfg = synth.CONFIGS["tiny"]
    W = synth.workload("tiny")
    _report("tiny", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label="tiny"))


def test_decode_bf16():
    cfg = synth.CONFIGS["decode"]
    W = synth.workload("decode")
    _report("decode", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label="decode"))


def test_prefill_bf16_every_token():
    cfg = synth.CONFIGS["prefill"]
    W = synth.workload("prefill")
    got = run_gpu(W, cfg)
    ref = run_oracle(W, cfg)
    assert (ref["count"] == 0).sum() > 0
    err = compare(got, ref, cfg, label="prefill")
    _report(f"prefill (all {cfg['T']} tokens, {(ref['count'] > 0).sum()} non-empty experts)", err)


# ---------------------------------------------------------------------------
# int4 routed experts (offset-binary nibbles, fp16 group scales)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cid,T,D,E,K,F,group", [
    (131, 100, 256, 40, 8, 192, 32),     # ~20 rows/expert: 32-row tiles, ragged columns
    (132, 300, 128, 20, 8, 128, 32),     # ~120 rows/expert: 64-row tiles
    (133, 57, 256, 24, 8, 128, 64),      # group of 64
])
def test_int4_small_shapes(cid, T, D, E, K, F, group):
    cfg = custom_cfg(cid, T, D, E, K, F, "bf16", int4=True, group=group)
    W = make_inputs(cfg)
    _report(f"int4 cid={cid}", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label=f"int4 cid={cid}"))


def test_int4_workload_every_token():
    cfg = synth.CONFIGS["int4"]
    W = synth.workload("int4")
    _report(f"int4 workload (all {cfg['T']} tokens)",
            compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label="int4"))


def test_int4_decode():
    # decode batch (T = 64) with int4 experts: every output token against the oracle
    cfg = synth.CONFIGS["int4_decode"]
    W = synth.workload("int4_decode")
    _report("int4 decode", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label="int4 decode"))


def test_int4_stacked_layer_shape_every_token():
    # one layer of the stacked decode shape (T = 256) with int4 experts; tokens and
    # router are the stacked workload's first layer, whose stored redraws keep the
    # 8th and 9th router probabilities apart
    cfg = dict(synth.CONFIGS["stacked"], layers=1, int4=True, group=32)
    W = synth.layer_weights(cfg, 0)
    W["x"] = synth.x_rows(cfg, synth.load_attempts("stacked"))
    _report("int4 stacked-layer shape (all 256 tokens)",
            compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label="int4 T=256"))


# batches of at most 128 tokens with group-32 scales and D a multiple of 256
# run the gate+up product on the narrow int4 engine: 8 token rows per pass, so
# experts with more rows take several passes over one tile (150: about 50 rows
# per expert; 151: D = 256, a single stage; 152: a single token; 153: the
# largest batch that takes this engine; 154: small scales; the small shapes
# 131, 134, 141 and 144 above take it too)
@pytest.mark.parametrize("cid,T,D,E,K,F", [
    (150, 100, 512, 16, 8, 256),
    (151, 64, 256, 288, 8, 256),
    (152, 1, 2048, 288, 8, 768),
    (153, 128, 1024, 64, 8, 512),
])
def test_int4_narrow_engine(cid, T, D, E, K, F):
    cfg = custom_cfg(cid, T, D, E, K, F, "bf16", int4=True, group=32)
    W = make_inputs(cfg)
    _report(f"int4 narrow cid={cid}", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label=f"int4 narrow cid={cid}"))


# bf16 routed batches on the row-light tiles (R <= 24 E): 160 about 21 rows per
# expert, 161 a single token at the workload widths, 162 K = 4, 163 128 tokens
# over 288 experts; 164 and 165 take the 32 x 256 gate+up tiles (at most 64
# tokens, at least 1024 tiles), 165 with F = 704, whose last column tile holds
# 64 of its 128 h columns
@pytest.mark.parametrize("cid,T,D,E,K,F", [
    (160, 128, 256, 48, 8, 256),
    (161, 1, 2048, 288, 8, 768),
    (162, 90, 512, 64, 4, 384),
    (163, 128, 1024, 288, 8, 512),
    (164, 32, 1024, 288, 8, 768),
    (165, 48, 256, 288, 8, 704),
])
def test_bf16_row_light_batches(cid, T, D, E, K, F):
    cfg = custom_cfg(cid, T, D, E, K, F, "bf16")
    W = make_inputs(cfg)
    _report(f"bf16 row-light cid={cid}", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label=f"cid={cid}"))


@pytest.mark.parametrize("cid,F", [(134, 128), (154, 256)])
def test_int4_small_scales(cid, F):
    # group scales in [2^-14, 2^-12), where a scale divided by 16 would be an fp16
    # subnormal: each weight must still be (nibble - 8) * scale rounded once.  The
    # tokens are scaled by 128 (exact in bf16) so the products keep their size, and
    # the shared expert is zero so that y is the routed experts' output alone.
    cfg = custom_cfg(cid, 90, 256, 24, 8, F, "bf16", int4=True, group=32)
    W = make_inputs(cfg)
    rng = np.random.default_rng(cid)
    for k in ("gate_s", "up_s", "down_s"):
        W[k] = rng.integers(0x0400, 0x0C00, size=W[k].shape, dtype=np.uint16)
    for k in ("s_gate", "s_up", "s_down"):
        W[k] = np.zeros_like(W[k])
    x32 = (W["x"].astype(np.uint32) << 16).view(np.float32) * np.float32(128.0)
    W["x"] = (x32.view(np.uint32) >> 16).astype(np.uint16)
    _report(f"int4 small scales F={F}", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label="int4 small scales"))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cid,T,D,E,K,F,dt", [
    (111, 1, 128, 288, 8, 64, "bf16"),       # a single token
    (112, 9, 64, 8, 8, 64, "bf16"),          # E = K: every expert chosen by every token
    (113, 33, 128, 50, 1, 64, "bf16"),       # K = 1
    (114, 70, 64, 1024, 8, 64, "bf16"),      # the largest supported E
    (115, 5, 64, 8, 8, 64, "f32"),
    # several 256-token permutation tiles with a ragged last one: E = 1000 fills
    # almost every thread's four experts, K = 6 leaves rows per tile uneven
    (116, 1500, 64, 1000, 8, 64, "bf16"),
    (117, 2100, 64, 288, 6, 64, "bf16"),
    # expert counts whose top-K slot count is rounded up to the next kernel size
    # (6 slots run as 8, 10 as 16): every slot's loads stay inside the logits and bias
    (118, 40, 64, 330, 8, 64, "bf16"),
    (119, 40, 64, 600, 8, 64, "bf16"),
    # fp32 above the fused top-K + permutation path: the fp32 router zeroes the
    # per-tile counts that the top-K kernel accumulates
    (120, 1100, 64, 40, 8, 64, "f32"),
    # the one-wave permutation of at most 64 tokens at the largest E it takes
    # (eight experts per lane), and one token past it (the 16-wave one)
    (121, 64, 128, 512, 8, 64, "bf16"),
    (122, 65, 128, 288, 8, 64, "bf16"),
])
def test_edge_shapes(cid, T, D, E, K, F, dt):
    cfg = custom_cfg(cid, T, D, E, K, F, dt)
    W = make_inputs(cfg)
    _report(f"edge cid={cid}", compare(run_gpu(W, cfg), run_oracle(W, cfg), cfg, label=f"cid={cid}"))


def test_zero_tokens():
    import torch
    cfg = custom_cfg(120, 0, 64, 16, 8, 64, "bf16")
    W = make_inputs(cfg)
    layer, x = gpu_layer(W, cfg)
    layer.routing.count.fill_(7)
    layer.routing.offset.fill_(7)
    layer(x)
    torch.cuda.synchronize()
    assert layer.routing.count.cpu().tolist() == [0] * 16
    assert layer.routing.offset.cpu().tolist() == [0] * 17


def test_residual_and_bf16_output():
    # y = residual + layer(x) written in place over the residual, and its bf16 copy:
    # y against the oracle given the same residual, y_bf16 against the oracle's
    # round-to-nearest-even of the GPU's fp32 y
    import oracle
    import torch
    cfg = custom_cfg(121, 80, 128, 32, 8, 64, "bf16")
    W = make_inputs(cfg)
    layer, x = gpu_layer(W, cfg)
    res = np.random.default_rng(121).standard_normal((cfg["T"], cfg["D"])).astype(np.float32) * 3
    y = torch.from_numpy(res.copy()).cuda()
    yb = torch.empty(y.shape, dtype=torch.bfloat16, device=y.device)
    layer(x, y=y, residual=y, y_bf16=yb)
    torch.cuda.synchronize()
    got = layer.routing_numpy()
    got["y"] = y.cpu().numpy().astype(np.float64)
    g, u, d = W["gate"], W["up"], W["down"]
    ref = oracle.moe_layer(W["x"], W["wr"], W["bias"], g, u, d, W["s_gate"], W["s_up"], W["s_down"],
                           cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"], residual=res.astype(np.float64))
    _report("residual in place", compare(got, ref, cfg, label="residual"))
    yf = y.cpu().numpy().reshape(-1)
    ybits = yb.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    want = np.array([oracle.bf16_from_double(float(v)) for v in yf], dtype=np.uint16)
    assert np.array_equal(ybits, want), "y_bf16 is not y rounded to nearest even"


# ---------------------------------------------------------------------------
# determinism: identical inputs give bitwise identical routing and outputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "int4", "int4_decode"])
def test_bitwise_determinism(name):
    import torch
    cfg = synth.CONFIGS[name]
    W = synth.workload(name)
    layer, x = gpu_layer(W, cfg)
    outs = []
    for _ in range(3):
        y = layer(x).clone()
        torch.cuda.synchronize()
        r = layer.routing_numpy()
        outs.append((y.cpu().numpy(), r))
    for y, r in outs[1:]:
        assert np.array_equal(y.view(np.uint32), outs[0][0].view(np.uint32))
        for k in r:
            assert np.array_equal(r[k], outs[0][1][k])
