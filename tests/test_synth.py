"""Checks of the seeded input generator (``synth``) and of the stored
per-token redraw table: determinism, row independence, storage rounding,
value distributions, the Zipf-shaped bias, and the 8th/9th router-gap rule
for every workload (measured with the oracle)."""
import hashlib
import json
import math

import numpy as np
import pytest

import oracle
import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_same_seed_same_bytes_and_streams_differ():
    cfg = synth.CONFIGS["tiny"]
    a = synth.layer_weights(cfg, 0)
    b = synth.layer_weights(cfg, 0)
    for k in a:
        assert _h(a[k]) == _h(b[k])
    assert _h(a["gate"]) != _h(a["up"])
    c = synth.layer_weights(cfg, 1)
    assert _h(a["gate"]) != _h(c["gate"])
    assert _h(synth.layer_weights(cfg, 0, seed=1)["gate"]) != _h(a["gate"])


def test_rows_regenerate_alone():
    cfg = synth.CONFIGS["decode"]
    k = synth.key(cfg, 0, synth.GATE)
    full = synth.normal(k, 50, 2048, 0.02, "bf16")
    part = synth.normal(k, 7, 2048, 0.02, "bf16", row0=31)
    assert np.array_equal(full[31:38], part)


def test_attempts_change_only_their_rows():
    cfg = synth.CONFIGS["decode"]
    att = np.zeros(cfg["T"], np.int32)
    x0 = synth.x_rows(cfg, att)
    att[5] = 3
    x1 = synth.x_rows(cfg, att)
    changed = np.nonzero(np.any(x0 != x1, axis=1))[0]
    assert changed.tolist() == [5]


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80), (1.0 + 2 ** -8, 0x3F80), (1.0 + 3 * 2 ** -8, 0x3F82),
    (1.0 + 2 ** -8 + 2 ** -40, 0x3F81), (-1.5, 0xBFC0), (3.14159265358979, 0x4049),
    (2.0 ** -133, 0x0001), (3 * 2.0 ** -134, 0x0002), (3.5e38, 0x7F80), (-0.0, 0x8000),
    ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80)])
def test_generator_bf16_rounding_points(value, bits):
    assert synth.bf16_bits(value) == bits


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3C00), (0.01, 0x211F), (0.005, 0x1D1F), (0.02, 0x251F), (65504.0, 0x7BFF),
    (65520.0, 0x7C00), (2.0 ** -24, 0x0001), (1.0 + 2 ** -11, 0x3C00),
    (1.0 + 3 * 2 ** -11, 0x3C02), (-2.0, 0xC000)])
def test_generator_fp16_rounding_points(value, bits):
    assert synth.fp16_bits(value) == bits


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_value_distributions():
    cfg = synth.CONFIGS["decode"]
    W = synth.layer_weights(dict(cfg, E=4))     # 4 experts are plenty for moments
    for name, fan in (("gate", 2048), ("up", 2048), ("down", 768), ("wr", 2048),
                      ("s_gate", 2048), ("s_down", 768)):
        v = _bf16_to_f64(W[name]).ravel()
        assert abs(v.mean()) < 5 * (1 / math.sqrt(fan)) / math.sqrt(v.size)
        assert v.std() * math.sqrt(fan) == pytest.approx(1.0, rel=5 / math.sqrt(2 * v.size))
        # roughly normal tails: ~0.27% beyond 3 sigma
        if v.size > 10 ** 6:
            frac3 = np.mean(np.abs(v) * math.sqrt(fan) > 3)
            assert 0.0024 < frac3 < 0.0030
    b = W["bias"]
    assert b.dtype == np.float32 and b.min() >= -0.1 and b.max() < 0.1
    x = _bf16_to_f64(synth.x_rows(cfg))
    assert x.std() == pytest.approx(1.0, rel=0.02)


def test_int4_generation():
    cfg = synth.CONFIGS["int4"]
    q, s = synth.int4_matrix(cfg, 0, synth.GATE_Q, synth.GATE_S, 4, 768, 2048)
    assert q.shape == (4, 768, 1024) and s.shape == (4, 768, 64)
    nib = np.concatenate([(q & 15).ravel(), (q >> 4).ravel()])
    counts = np.bincount(nib, minlength=16) / nib.size
    np.testing.assert_allclose(counts, 1 / 16, rtol=0.01)
    sv = s.view(np.float16).astype(np.float64)
    assert sv.min() >= 0.00499 and sv.max() <= 0.02001
    assert sv.mean() == pytest.approx(0.0125, rel=0.01)


def test_zipf_bias_is_minus_s_log_of_a_ranking():
    cfg = synth.CONFIGS["prefill"]
    b = synth.bias(cfg).astype(np.float64)
    ranks = np.exp(-b / synth.ZIPF_S)
    np.testing.assert_allclose(np.sort(ranks), np.arange(1, 289), rtol=1e-5)
    assert b.max() == 0.0


def _route(name):
    # only the router's inputs are needed: x, the router matrix and the bias
    cfg = synth.CONFIGS[name]
    D, E = cfg["D"], cfg["E"]
    x = synth.x_rows(cfg, synth.load_attempts(name))
    wr = synth.normal(synth.key(cfg, 0, synth.WR), E, D, 1.0 / math.sqrt(D), cfg["dtype"])
    assert np.array_equal(wr, synth.layer_weights(dict(cfg, E=E, F=32), 0)["wr"])
    z = oracle.router_logits(x, wr, synth.bias(cfg), cfg["T"], D, E)
    return cfg, z


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_stored_attempts_separate_8th_and_9th(name):
    with open(synth.GAP_ATTEMPTS_PATH) as f:
        table = json.load(f)
    assert name in table
    cfg, z = _route(name)
    gap = oracle.sigma_gap(z, cfg["K"])
    assert gap.min() > synth.GAP_MIN


def test_prefill_popularity_is_skewed_with_empty_experts():
    cfg, z = _route("prefill")
    ids, _ = oracle.select_topk(z, cfg["K"])
    count, *_ = oracle.permutation(ids, cfg["E"])
    assert (count == 0).sum() >= 1
    assert count.max() > 8 * count.mean()
