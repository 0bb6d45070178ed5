"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, a hand-computed point, an
invariant, a brute force on tiny inputs, or a special case that reduces to a
textbook computation done here with numpy matrix products.  The layer's
definition is taken from the pages:
  [glm5next] "Add GLM-5.3-Flash (glm5next) support with ROCmFP mix qtypes
             (105/106)": "Architecture" (clamped SwiGLU: gate limited above at
             10 then SiLU, up limited to [-10, 10]; 288 experts, top-8, one
             shared expert, sigmoid routing) and "MoE FFN" (router sigmoid of
             the gate projection plus bias, top-8, weight normalisation,
             gate/up/down expert products, shared expert added).
  [glm53-hip] "feat(glm53): add device-resident HIP backend for MI350P":
             "Key changes" (deterministic top-k; grouped int4 decoded as
             offset-binary nibble minus 8).
Values below were worked out by hand from the closed forms (sigmoid(1) =
1/(1+e^-1) etc.) and are written as literals.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import Mat

pytestmark = pytest.mark.usefixtures("oracle_lib")


# ---------------------------------------------------------------------------
# scalar functions
# ---------------------------------------------------------------------------

def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(math.log(3.0)) == pytest.approx(0.75, abs=1e-15)
    assert oracle.sigmoid(-math.log(3.0)) == pytest.approx(0.25, abs=1e-15)
    assert oracle.sigmoid(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    # extreme arguments neither overflow nor produce NaN
    assert oracle.sigmoid(800.0) == 1.0
    assert 0.0 <= oracle.sigmoid(-800.0) < 1e-300
    for z in (0.1, 1.7, 5.0, 33.0):
        assert oracle.sigmoid(z) + oracle.sigmoid(-z) == pytest.approx(1.0, abs=1e-15)


# (gate, up) -> clamped SwiGLU, by hand from silu(a) = a / (1 + e^-a)
SWIGLU_POINTS = [
    ((0.0, 5.0), 0.0),
    ((1.0, 1.0), 0.7310585786300049),            # sigmoid(1)
    ((-1.0, 1.0), -0.2689414213699951),          # -sigmoid(-1)
    ((10.0, 1.0), 9.999546021312977),            # 10*sigmoid(10)
    ((20.0, 1.0), 9.999546021312977),            # gate clamped to 10
    ((2.0, 20.0), 17.615941559557648),           # 2*sigmoid(2)*10, up clamped to 10
    ((2.0, -20.0), -17.615941559557648),         # up clamped to -10
    ((2.0, 10.0), 17.615941559557648),           # clamp bound is inclusive
    ((-20.0, 3.0), -1.2366921709141223e-07),     # -60*sigmoid(-20), no lower gate clamp
    ((-12.0, 1.0), -7.373009522657661e-05),      # would be -4.5398e-4 if gate were clamped at -10
    ((10.0, 10.0), 99.99546021312977),
    ((1e4, -1e4), -99.99546021312977),
]


@pytest.mark.parametrize("gu,expected", SWIGLU_POINTS)
def test_swiglu_hand_points(gu, expected):
    got = oracle.swiglu(*gu)
    if expected == 0.0:
        assert got == 0.0
    else:
        assert got == pytest.approx(expected, rel=1e-13)


def test_swiglu_large_negative_gate_is_negative_zero():
    v = oracle.swiglu(-1e4, 10.0)
    assert v == 0.0 and math.copysign(1.0, v) == -1.0
    assert not math.isnan(oracle.silu(-1e300))


# ---------------------------------------------------------------------------
# encodings
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x0001, 2.0 ** -133),
    (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127), (0x8000, -0.0)])
def test_bf16_decode_points(bits, value):
    assert oracle.bf16_to_double(bits) == value


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0x211F, 0.01000213623046875), (0x0001, 2.0 ** -24),
    (0x03FF, 1023 * 2.0 ** -24), (0x7BFF, 65504.0), (0xC000, -2.0),
    (0x3555, 0.333251953125)])
def test_fp16_decode_points(bits, value):
    assert oracle.fp16_to_double(bits) == value


def test_fp16_decode_inf():
    assert oracle.fp16_to_double(0x7C00) == math.inf
    assert oracle.fp16_to_double(0xFC00) == -math.inf


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),               # exact tie -> even mantissa (0)
    (1.0 + 3 * 2 ** -8, 0x3F82),           # exact tie -> even mantissa (2)
    (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),    # just above the tie: up (no double rounding via fp32)
    (1.0 + 2 ** -8 - 2 ** -40, 0x3F80),
    (-1.5, 0xBFC0),
    (3.14159265358979, 0x4049),
    (2.0 ** -133, 0x0001),
    (3 * 2.0 ** -134, 0x0002),             # subnormal tie -> even
    (3.5e38, 0x7F80),                      # overflow -> inf
    (-0.0, 0x8000),
])
def test_bf16_rounding_points(value, bits):
    assert oracle.bf16_from_double(value) == bits


S001 = 0x211F   # fp16 nearest to 0.01 = 0.01000213623046875


@pytest.mark.parametrize("nib,value", [
    (0, -0.08001708984375), (7, -0.01000213623046875), (8, 0.0),
    (15, 0.07001495361328125), (1, -0.07001495361328125)])
def test_int4_decode_points(nib, value):
    # one row of K=32 elements, one group, all nibbles = nib
    q = np.full((1, 16), nib | (nib << 4), np.uint8)
    s = np.array([[S001]], np.uint16)
    m = Mat.int4(q, s, 32)
    for k in (0, 1, 17, 31):
        assert oracle.mat_elem(m, 0, 1, 32, 0, k) == value


def test_int4_nibble_order_and_sign_convention():
    # byte 0x80: even k holds the low nibble (0 -> -8s), odd k the high (8 -> 0)
    # byte 0x0F: even k -> 15 -> +7s, odd k -> 0 -> -8s  (offset-binary, not two's complement)
    q = np.zeros((1, 16), np.uint8)
    q[0, 0] = 0x80
    q[0, 1] = 0x0F
    s = np.array([[S001]], np.uint16)
    m = Mat.int4(q, s, 32)
    assert oracle.mat_elem(m, 0, 1, 32, 0, 0) == -0.08001708984375
    assert oracle.mat_elem(m, 0, 1, 32, 0, 1) == 0.0
    assert oracle.mat_elem(m, 0, 1, 32, 0, 2) == 0.07001495361328125
    assert oracle.mat_elem(m, 0, 1, 32, 0, 3) == -0.08001708984375


def test_int4_group_scale_indexing():
    # two rows, K=64, two groups per row: each element's scale is its own group's
    q = np.full((2, 32), 0x99, np.uint8)          # nibble 9 -> +1 * scale
    s = np.array([[0x3C00, 0x4000], [0x4200, 0x4400]], np.uint16)   # 1, 2, 3, 4
    m = Mat.int4(q, s, 32)
    assert oracle.mat_elem(m, 0, 2, 64, 0, 31) == 1.0
    assert oracle.mat_elem(m, 0, 2, 64, 0, 32) == 2.0
    assert oracle.mat_elem(m, 0, 2, 64, 1, 0) == 3.0
    assert oracle.mat_elem(m, 0, 2, 64, 1, 63) == 4.0


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def test_router_logits_hand_example():
    x = np.array([[1.0, 2.0]], np.float32)
    wr = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]], np.float32)
    b = np.array([0.5, 0.0, -1.0], np.float32)
    z = oracle.router_logits(x, wr, b, 1, 2, 3)
    assert z.tolist() == [[1.5, 2.0, 2.0]]


def test_router_logits_match_matrix_product():
    rng = np.random.default_rng(1)
    T, D, E = 7, 96, 33
    x = rng.standard_normal((T, D)).astype(np.float32)
    wr = rng.standard_normal((E, D)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    z = oracle.router_logits(x, wr, b, T, D, E)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T + b.astype(np.float64)
    np.testing.assert_allclose(z, ref, rtol=0, atol=1e-12)


def _brute_topk(zrow, K):
    order = sorted(range(len(zrow)), key=lambda e: (-zrow[e], e))
    return sorted(order[:K])


def test_select_matches_full_sort():
    rng = np.random.default_rng(2)
    T, E, K = 64, 40, 8
    z = rng.standard_normal((T, E))
    # inject exact ties in some rows
    z[3, :] = 0.25
    z[5, ::3] = z[5, 0]
    z[9, 10:20] = 7.0
    ids, w = oracle.select_topk(z, K)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(z[t].tolist(), K)
        assert list(ids[t]) == sorted(ids[t])                 # ascending canonical order
        assert len(set(ids[t].tolist())) == K


def test_select_ties_go_to_lowest_index():
    z = np.zeros((1, 20))
    z[0, [4, 9, 13, 17]] = 1.0       # four strictly-better experts
    ids, _ = oracle.select_topk(z, 8)
    assert ids[0].tolist() == [0, 1, 2, 3, 4, 9, 13, 17]


def test_select_weights_closed_form():
    # E = K = 8: all experts chosen.  sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4,
    # sigmoid(0) = 1/2; sum = 3/4 + 1/4 + 6/2 = 4.
    z = np.zeros((1, 8))
    z[0, 2] = math.log(3.0)
    z[0, 5] = -math.log(3.0)
    ids, w = oracle.select_topk(z, 8)
    assert ids[0].tolist() == list(range(8))
    exp = [0.125, 0.125, 0.1875, 0.125, 0.125, 0.0625, 0.125, 0.125]
    np.testing.assert_allclose(w[0], exp, rtol=0, atol=1e-15)


def test_select_equal_logits_give_equal_weights():
    ids, w = oracle.select_topk(np.full((2, 288), -3.0), 8)
    assert ids.tolist() == [list(range(8))] * 2
    np.testing.assert_allclose(w, 0.125, rtol=0, atol=1e-16)
    _, w0 = oracle.select_topk(np.zeros((1, 288)), 8)   # 8 * sigmoid(0) = 4 exactly
    assert np.all(w0 == 0.125)


def test_weights_sum_to_one_and_follow_logit_order():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((100, 288)) * 4
    ids, w = oracle.select_topk(z, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(w > 0)
    for t in range(100):
        zt = z[t, ids[t]]
        # larger logit -> larger weight (sigmoid is increasing)
        assert np.all(np.argsort(zt, kind="stable") == np.argsort(w[t], kind="stable"))


def test_zero_input_selects_largest_biases():
    rng = np.random.default_rng(4)
    E, D = 288, 64
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    wr = rng.standard_normal((E, D)).astype(np.float32)
    x = np.zeros((2, D), np.float32)
    z = oracle.router_logits(x, wr, b, 2, D, E)
    ids, _ = oracle.select_topk(z, 8)
    assert ids[0].tolist() == sorted(np.argsort(-b.astype(np.float64), kind="stable")[:8].tolist())


# ---------------------------------------------------------------------------
# permutation
# ---------------------------------------------------------------------------

def _random_ids(rng, T, E, K):
    return np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]).astype(np.int32)


def test_permutation_matches_stable_sort():
    rng = np.random.default_rng(5)
    T, E, K = 37, 23, 8
    ids = _random_ids(rng, T, E, K)
    count, offset, perm, inv = oracle.permutation(ids, E)
    pairs = sorted(((int(ids[t, j]), t, j) for t in range(T) for j in range(K)))
    assert perm.tolist() == [t * K + j for (_, t, j) in pairs]
    assert count.tolist() == [sum(1 for p in pairs if p[0] == e) for e in range(E)]
    assert offset[0] == 0 and offset[E] == T * K
    assert np.all(np.diff(offset) == count)
    assert np.all(inv[perm] == np.arange(T * K))
    for e in range(E):
        rows = perm[offset[e]:offset[e + 1]]
        assert np.all(ids.reshape(-1)[rows] == e)


def test_permutation_empty_experts_and_zero_tokens():
    ids = np.array([[0, 5, 7], [0, 5, 6]], np.int32)
    count, offset, perm, inv = oracle.permutation(ids, 9)
    assert count.tolist() == [2, 0, 0, 0, 0, 2, 1, 1, 0]
    assert offset.tolist() == [0, 2, 2, 2, 2, 2, 4, 5, 6, 6]
    assert perm.tolist() == [0, 3, 1, 4, 5, 2]
    c0, o0, p0, i0 = oracle.permutation(np.zeros((0, 8), np.int32), 9)
    assert c0.tolist() == [0] * 9 and o0.tolist() == [0] * 10 and len(p0) == 0


# ---------------------------------------------------------------------------
# expert FFN and combine
# ---------------------------------------------------------------------------

def _rand_layer(rng, T, D, E, F, dtype=np.float32, scale=1.0):
    g = lambda *s, fan: (rng.standard_normal(s) * scale / math.sqrt(fan)).astype(dtype)
    return dict(
        x=rng.standard_normal((T, D)).astype(dtype),
        wr=g(E, D, fan=D), bias=rng.uniform(-0.1, 0.1, E).astype(np.float32),
        gate=g(E, F, D, fan=D), up=g(E, F, D, fan=D), down=g(E, D, F, fan=F),
        s_gate=g(F, D, fan=D), s_up=g(F, D, fan=D), s_down=g(D, F, fan=F))


def _layer(L, T, D, E, K, F, **kw):
    return oracle.moe_layer(L["x"], L["wr"], L["bias"], L["gate"], L["up"], L["down"],
                            L["s_gate"], L["s_up"], L["s_down"], T, D, E, K, F, **kw)


_swiglu_vec = np.vectorize(oracle.swiglu)   # activation pinned by the hand points above


def _textbook_ffn(x, wg, wu, wd):
    """Dense SwiGLU FFN with numpy matrix products (rows of x)."""
    x = x.astype(np.float64)
    g = x @ wg.astype(np.float64).T
    u = x @ wu.astype(np.float64).T
    return _swiglu_vec(g, u) @ wd.astype(np.float64).T


def test_single_expert_reduces_to_textbook_swiglu_ffn():
    # E = K = 1: the routed weight is exactly 1, so y = S(x) + E_0(x).  D != F
    # catches a transposed down projection.
    rng = np.random.default_rng(6)
    T, D, E, K, F = 5, 48, 1, 1, 20
    L = _rand_layer(rng, T, D, E, F, scale=3.0)
    out = _layer(L, T, D, E, K, F)
    assert np.all(out["w"] == 1.0)
    ref = (_textbook_ffn(L["x"], L["s_gate"], L["s_up"], L["s_down"]) +
           _textbook_ffn(L["x"], L["gate"][0], L["up"][0], L["down"][0]))
    np.testing.assert_allclose(out["y"], ref, rtol=0, atol=1e-11 * np.abs(ref).max())


def test_identical_experts_sum_to_one_expert():
    rng = np.random.default_rng(7)
    T, D, E, K, F = 6, 32, 16, 8, 24
    L = _rand_layer(rng, T, D, E, F)
    for name in ("gate", "up", "down"):
        L[name] = np.broadcast_to(L[name][:1], L[name].shape).copy()
    out = _layer(L, T, D, E, K, F)
    ref = (_textbook_ffn(L["x"], L["gate"][0], L["up"][0], L["down"][0]) +
           _textbook_ffn(L["x"], L["s_gate"], L["s_up"], L["s_down"]))
    np.testing.assert_allclose(out["y"], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # and with the shared expert equal to them too: y = 2 * E(x)
    L["s_gate"], L["s_up"], L["s_down"] = L["gate"][0], L["up"][0], L["down"][0]
    out2 = _layer(L, T, D, E, K, F)
    np.testing.assert_allclose(out2["y"], 2 * _textbook_ffn(L["x"], L["gate"][0], L["up"][0],
                                                            L["down"][0]),
                               rtol=0, atol=1e-12 * np.abs(ref).max())


def test_sparse_path_equals_dense_brute_force():
    # every expert computed for every token with numpy, combined through a mask
    # built from a full sort of the logits
    rng = np.random.default_rng(8)
    T, D, E, K, F = 9, 40, 12, 3, 16
    L = _rand_layer(rng, T, D, E, F, scale=2.0)
    out = _layer(L, T, D, E, K, F)
    x64 = L["x"].astype(np.float64)
    z = x64 @ L["wr"].astype(np.float64).T + L["bias"].astype(np.float64)
    y = _textbook_ffn(L["x"], L["s_gate"], L["s_up"], L["s_down"])
    for t in range(T):
        chosen = _brute_topk(z[t].tolist(), K)
        p = np.array([1.0 / (1.0 + math.exp(-z[t, e])) for e in chosen])
        for e, pe in zip(chosen, p / p.sum()):
            y[t] += pe * _textbook_ffn(L["x"][t:t + 1], L["gate"][e], L["up"][e], L["down"][e])[0]
    np.testing.assert_allclose(out["y"], y, rtol=0, atol=1e-12 * np.abs(y).max())


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(9)
    T, D, E, K, F = 3, 32, 20, 8, 16
    L = _rand_layer(rng, T, D, E, F)
    L["x"] = np.zeros_like(L["x"])
    out = _layer(L, T, D, E, K, F)
    assert np.all(out["y"] == 0.0)


def test_clamps_fire_inside_the_layer():
    # huge weights drive gate and up far past the limits: each hidden unit is
    # then +-100*sigmoid(10) or ~0, never larger
    rng = np.random.default_rng(10)
    D, F = 16, 8
    xr = rng.standard_normal(D)
    wg = (rng.standard_normal((1, F, D)) * 100).astype(np.float32)
    wu = (rng.standard_normal((1, F, D)) * 100).astype(np.float32)
    h = oracle.expert_hidden(xr, wg, wu, 0, D, F, 1)
    g = wg[0].astype(np.float64) @ xr
    u = wu[0].astype(np.float64) @ xr
    assert np.all(np.abs(h) <= 10 * oracle.silu(10.0) + 1e-12)
    big = (g > 10) & (np.abs(u) > 10)
    assert big.any()
    np.testing.assert_allclose(h[big], np.sign(u[big]) * 99.99546021312977, rtol=1e-13)


def test_token_order_equivariance():
    rng = np.random.default_rng(11)
    T, D, E, K, F = 12, 32, 30, 8, 16
    L = _rand_layer(rng, T, D, E, F)
    out = _layer(L, T, D, E, K, F)
    p = rng.permutation(T)
    L2 = dict(L, x=L["x"][p].copy())
    out2 = _layer(L2, T, D, E, K, F)
    assert np.array_equal(out2["ids"], out["ids"][p])
    assert np.array_equal(out2["w"], out["w"][p])
    assert np.array_equal(out2["y"], out["y"][p])


def test_token_subset_and_residual():
    rng = np.random.default_rng(12)
    T, D, E, K, F = 10, 32, 30, 8, 16
    L = _rand_layer(rng, T, D, E, F)
    full = _layer(L, T, D, E, K, F)
    res = rng.standard_normal((T, D))
    sub = _layer(L, T, D, E, K, F, residual=res, tokens=[7, 2, 2])
    np.testing.assert_array_equal(sub["y"], full["y"][[7, 2, 2]] + res[[7, 2, 2]])


def test_bf16_operands_widen_exactly():
    # the bf16 path equals the fp32 path run on the same (exactly widened) values
    rng = np.random.default_rng(13)
    T, D, E, K, F = 4, 32, 20, 8, 16
    L = _rand_layer(rng, T, D, E, F)
    bits = {k: (v.view(np.uint32) >> 16).astype(np.uint16) for k, v in L.items() if k != "bias"}
    widened = {k: (b.astype(np.uint32) << 16).view(np.float32) for k, b in bits.items()}
    a = _layer(dict(bits, bias=L["bias"]), T, D, E, K, F)
    b = _layer(dict(widened, bias=L["bias"]), T, D, E, K, F)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["ids"], b["ids"])


def _pack_int4(nib):
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def _fp16_bits_value(bits):
    return bits.view(np.float16).astype(np.float64)


def test_int4_layer_equals_layer_on_decoded_weights():
    rng = np.random.default_rng(14)
    T, D, E, K, F, G = 6, 64, 12, 4, 32, 32
    L = _rand_layer(rng, T, D, E, F)
    mats = {}
    dec = {}
    for name, (rows, kdim) in dict(gate=(F, D), up=(F, D), down=(D, F)).items():
        nib = rng.integers(0, 16, (E, rows, kdim)).astype(np.uint8)
        sc = rng.uniform(0.005, 0.02, (E, rows, kdim // G)).astype(np.float16).view(np.uint16)
        mats[name] = Mat.int4(_pack_int4(nib), sc, G)
        # decode here, independently of the oracle: (nibble - 8) * scale, exact in fp32
        dec[name] = ((nib.astype(np.float64) - 8.0) *
                     np.repeat(_fp16_bits_value(sc), G, axis=-1)).astype(np.float32)
    a = oracle.moe_layer(L["x"], L["wr"], L["bias"], mats["gate"], mats["up"], mats["down"],
                         L["s_gate"], L["s_up"], L["s_down"], T, D, E, K, F)
    b = oracle.moe_layer(L["x"], L["wr"], L["bias"], dec["gate"], dec["up"], dec["down"],
                         L["s_gate"], L["s_up"], L["s_down"], T, D, E, K, F)
    assert np.array_equal(a["y"], b["y"])


def test_residual_layer_chain_step():
    rng = np.random.default_rng(15)
    n, D, E, K, F = 4, 32, 20, 8, 16
    L = _rand_layer(rng, n, D, E, F)
    x = rng.standard_normal((n, D)) * 3
    xin, ids, w, z, y, xn = oracle.residual_layer(x, L["wr"], L["bias"], L["gate"], L["up"],
                                                  L["down"], L["s_gate"], L["s_up"],
                                                  L["s_down"], D, E, K, F)
    assert np.array_equal(xin, np.vectorize(oracle.bf16_from_double)(x).astype(np.uint16))
    ref = _layer(dict(L, x=xin), n, D, E, K, F)
    assert np.array_equal(ref["y"], y) and np.array_equal(ref["ids"], ids)
    assert np.array_equal(xn, x + y)


def test_sigma_gap_helper():
    z = np.array([[5.0, 4.0, 3.0, 0.0, 0.0, 0.0, 0.0, 0.0, -1.0, -2.0]])
    # 8th largest = 0 (index 7), 9th = -1
    assert oracle.sigma_gap(z, 8)[0] == pytest.approx(0.5 - 0.2689414213699951, abs=1e-15)


# ---------------------------------------------------------------------------
# dense FFN layers ([glm5next] "Architecture": layers 0-2 run a dense FFN with
# no experts; the clamped SwiGLU holds for the model's FFNs)
# ---------------------------------------------------------------------------

def test_dense_ffn_hand_points():
    # D = 2, F = 1: g = x0, u = x1, y = (1, 3) * silu(min(g, 10)) * clamp(u)
    gate = np.array([[1.0, 0.0]], np.float32)
    up = np.array([[0.0, 1.0]], np.float32)
    down = np.array([[1.0], [3.0]], np.float32)
    x = np.array([[1.0, 2.0], [20.0, 20.0], [-1.0, -30.0]], np.float32)
    y = oracle.dense_ffn(x, gate, up, down, 3, 2, 1)
    h = [2 * 0.7310585786300049,          # silu(1) * 2
         99.99546021312977,               # silu(10) * 10: both clamps
         -0.2689414213699951 * -10.0]     # silu(-1) * (-10): up clamped below
    np.testing.assert_allclose(y, [[v, 3 * v] for v in h], rtol=1e-14)
    res = np.array([[0.5, -0.5], [1.0, 2.0], [0.0, 0.0]])
    y2 = oracle.dense_ffn(x, gate, up, down, 3, 2, 1, residual=res)
    np.testing.assert_allclose(y2, y + res, rtol=1e-15)


def test_dense_ffn_matches_textbook_swiglu_ffn():
    # bf16 operands with D != F (a transposed down projection would not fit),
    # inputs scaled so both clamps fire
    rng = np.random.default_rng(7)
    T, D, F = 6, 48, 80

    def bf16(a):
        b = np.array([oracle.bf16_from_double(float(v)) for v in a.reshape(-1)], np.uint16)
        return b.reshape(a.shape)

    def wide(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    x, g, u, d = (bf16(rng.standard_normal(s) * sc) for s, sc in
                  (((T, D), 6.0), ((F, D), 0.5), ((F, D), 0.5), ((D, F), 0.2)))
    y = oracle.dense_ffn(Mat.bf16(x), Mat.bf16(g), Mat.bf16(u), Mat.bf16(d), T, D, F)
    gg = wide(x) @ wide(g).T
    uu = wide(x) @ wide(u).T
    assert (gg > 10).any() and (np.abs(uu) > 10).any()
    gc = np.minimum(gg, 10.0)
    hh = gc / (1.0 + np.exp(-gc)) * np.clip(uu, -10.0, 10.0)
    np.testing.assert_allclose(y, hh @ wide(d).T, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------------
# index selection ([glm5next] "MLA/DSA": top-k of the indexer scores with
# k = 2048; the last kpool positions always selected)
# ---------------------------------------------------------------------------

def test_index_topk_hand_example():
    s = np.array([[3, 1, 3, 2, 5, 0, 1, 1, 2, 4]], np.float32)
    # 5 at 4, 4 at 9, then 3 at 0 and 2 tie: the lower position wins
    assert oracle.index_topk(s, 3).tolist() == [[0, 4, 9]]
    # tail 2 keeps positions 8 and 9, the one free slot goes to the 5 at position 4
    assert oracle.index_topk(s, 3, tail=2).tolist() == [[4, 8, 9]]
    # the first 6 positions only: 5 at 4, 3 at 0 and 2
    assert oracle.index_topk(s, 3, lens=[6]).tolist() == [[0, 2, 4]]
    # k = 4 with the tail at positions 4, 5 of the first 6: then 3, 3 at 0 and 2
    assert oracle.index_topk(s, 4, tail=2, lens=[6]).tolist() == [[0, 2, 4, 5]]


def test_index_topk_short_rows_take_everything():
    s = np.arange(12, dtype=np.float32).reshape(2, 6)[:, ::-1].copy()
    out = oracle.index_topk(s, 8, lens=[6, 0])
    assert out[0].tolist() == [0, 1, 2, 3, 4, 5, -1, -1]
    assert out[1].tolist() == [-1] * 8
    assert oracle.index_topk(s, 6).tolist() == [list(range(6))] * 2


def test_index_topk_signed_zero_and_infinities_order():
    s = np.array([[0.0, -0.0, -np.inf, 1e-45, -1e-45, np.inf, -0.0]], np.float32)
    # inf; the smallest positive subnormal; then +0 and -0 tie: positions 0 and 1
    assert oracle.index_topk(s, 4).tolist() == [[0, 1, 3, 5]]
    assert oracle.index_topk(s, 6).tolist() == [[0, 1, 3, 4, 5, 6]]


def test_index_topk_matches_lexsort_brute_force():
    rng = np.random.default_rng(11)
    for trial in range(40):
        rows, L = 3, int(rng.integers(1, 60))
        s = rng.integers(0, 5, size=(rows, L)).astype(np.float32)   # many ties
        k = int(rng.integers(1, 40))
        tail = int(rng.integers(0, 6))
        lens = rng.integers(0, L + 3, size=rows).astype(np.int32)
        got = oracle.index_topk(s, k, tail=tail, lens=lens)
        for r in range(rows):
            n = min(int(lens[r]), L)
            pos = np.arange(n)
            if n <= k:
                want = list(range(n)) + [-1] * (k - n)
            else:
                is_tail = pos >= n - min(tail, k)
                order = np.lexsort((pos, -s[r, :n], ~is_tail))
                want = sorted(order[:k].tolist())
            assert got[r].tolist() == want, (trial, r)


def test_index_topk_invariants_at_scale():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((4, 5000)).astype(np.float32)
    k, tail = 2048, 4
    out = oracle.index_topk(s, k, tail=tail)
    for r in range(4):
        sel = out[r]
        assert len(set(sel.tolist())) == k and np.all(np.diff(sel) > 0)
        assert set(range(5000 - tail, 5000)) <= set(sel.tolist())
        rest = np.setdiff1d(np.arange(5000 - tail), sel)
        chosen = np.setdiff1d(sel, np.arange(5000 - tail, 5000))
        assert s[r, chosen].min() >= s[r, rest].max()
