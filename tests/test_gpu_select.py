"""Index selection of the sparse attention's IndexPool (top-k of the
indexer scores with the last kpool positions always kept: "Add GLM-5.3-Flash
(glm5next) support with ROCmFP mix qtypes (105/106)", section "MLA/DSA")
through the C ABI against the oracle: the selected positions are unique, so
they must match bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from sparse_moe_ffn_coli_amd import coli_index_topk

pytestmark = pytest.mark.gpu


def _gpu(scores, k, tail=0, lens=None):
    # rows are stored with a stride rounded up to 4 floats (the padding holds
    # +inf, which must never be selected: only the first L columns are read)
    import torch
    rows, L = scores.shape
    ld = (L + 3) // 4 * 4
    buf = np.full((rows, ld), np.inf, np.float32)
    buf[:, :L] = scores
    s = torch.from_numpy(buf).cuda()
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    ln = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    coli_index_topk(s, k, idx, tail=tail, lens=ln, L=L, ld=ld)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _check(scores, k, tail=0, lens=None, label=""):
    got = _gpu(scores, k, tail, lens)
    ref = oracle.index_topk(scores, k, tail=tail, lens=lens)
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert len(bad) == 0, f"{label}: rows {bad[:8]} differ"
    print(f"{label}: {scores.shape[0]} rows bit-exact", flush=True)


@pytest.mark.parametrize("rows,L,k,tail,ties", [
    (5, 100, 16, 0, True),          # many equal scores: lowest positions win
    (7, 257, 64, 4, True),          # ragged length (not a multiple of 4), tail kept
    (3, 8192, 2048, 4, False),      # the largest row of the small LDS cache
    (3, 8195, 2048, 4, False),      # just past it: the large cache
    (2, 32768, 2048, 4, True),      # the largest cached row
    (2, 40000, 2048, 4, False),     # uncached: passes re-read the scores
    (4, 5000, 4096, 3, False),      # the largest k
    (4, 3000, 1, 0, True),          # k = 1
    (4, 3000, 2, 5, False),         # tail longer than k: the last k positions
])
def test_index_topk_shapes(rows, L, k, tail, ties):
    rng = np.random.default_rng(rows * 1000 + L)
    s = (rng.integers(0, 7, size=(rows, L)) if ties else rng.standard_normal((rows, L))).astype(np.float32)
    _check(s, k, tail, label=f"rows={rows} L={L} k={k} tail={tail}")


def test_index_topk_lengths_and_short_rows():
    rng = np.random.default_rng(3)
    L, k = 6000, 2048
    s = rng.standard_normal((8, L)).astype(np.float32)
    lens = np.array([0, 1, 2047, 2048, 2049, 5999, 6000, 9000], np.int32)
    _check(s, k, 4, lens, label="lens")


def test_index_topk_signed_zero_and_infinities():
    s = np.zeros((3, 300), np.float32)
    s[0, ::2] = -0.0
    s[1, :] = -np.inf
    s[1, 7] = np.inf
    s[2, :] = np.float32(1e-45)
    s[2, 50:60] = -np.float32(1e-45)
    _check(s, 37, 0, label="signed zeros / infinities / subnormals")


@pytest.mark.parametrize("name", ["index_topk", "index_topk_decode"])
def test_index_topk_workloads_every_row(name):
    cfg = synth.INDEX_CONFIGS[name]
    s, lens = synth.index_scores(cfg)
    _check(s, cfg["k"], cfg["tail"], lens, label=name)


# Launches with more rows than CUs run the register-key kernel: the same
# cases at 260-300 rows.
@pytest.mark.parametrize("rows,L,k,tail,ties", [
    (300, 100, 16, 0, True),
    (260, 257, 64, 4, True),
    (257, 32768, 2048, 4, True),
    (260, 32765, 2048, 4, False),
    (260, 5000, 4096, 3, False),
    (260, 3000, 1, 0, True),
    (260, 3000, 2, 5, False),
    (260, 7, 3, 1, False),
])
def test_index_topk_many_rows(rows, L, k, tail, ties):
    rng = np.random.default_rng(rows * 7 + L)
    s = (rng.integers(0, 7, size=(rows, L)) if ties else rng.standard_normal((rows, L))).astype(np.float32)
    _check(s, k, tail, label=f"rows={rows} L={L} k={k} tail={tail}")


def test_index_topk_many_rows_lengths():
    # lengths from empty to past the cached limit in one launch
    rng = np.random.default_rng(11)
    rows, L, k = 300, 40000, 2048
    s = rng.standard_normal((rows, L)).astype(np.float32)
    lens = rng.integers(0, L + 1, size=rows).astype(np.int32)
    lens[:12] = [0, 1, 3, 2047, 2048, 2049, 2050, 2051, 32767, 32768, 32769, 40000]
    _check(s, k, 4, lens, label="many rows, mixed lengths")


def test_index_topk_many_rows_special_values():
    rows, L = 270, 300
    s = np.zeros((rows, L), np.float32)
    s[0::3, ::2] = -0.0
    s[1::3, :] = -np.inf
    s[1::3, 7] = np.inf
    s[2::3, :] = np.float32(1e-45)
    s[2::3, 50:60] = -np.float32(1e-45)
    _check(s, 37, 0, label="many rows: signed zeros / infinities / subnormals")
