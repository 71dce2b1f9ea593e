"""Pins for the oracle's indexer scores and Top-K / pool selection.

Scoring follows the CSA2 roles paragraph of the MarkTechPost retelling (Full
layers score the context, Reindex layers rescore the candidate pool);
selection follows the HN summary's key points (shared Top-K indices, a
shallow-layer candidate pool).  Pins: an exact-rational brute force, two
independent exact routes (int64 and float64 GEMM), Python's sorted() as the
brute-force selection, and the invariants the pages imply.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F, indexer as I, topk as T


def _fp8(rng, shape, scale=1.0):
    return torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_scores_exact_vs_rational_brute_force():
    rng = np.random.default_rng(0)
    q = _fp8(rng, 64)
    k = _fp8(rng, (40, 64), scale=3.0)
    k[0] = 0x7E                                   # +448 everywhere
    k[1] = 0x01                                   # smallest subnormal everywhere
    qv = [Fraction(float(v)) for v in F.e4m3_decode(q)]
    got = I.scores_exact(q, k)
    for j in range(k.shape[0]):
        want = sum(qv[d] * Fraction(float(F.e4m3_decode(k[j, d:d + 1])[0])) for d in range(64))
        assert Fraction(int(got[j])) * Fraction(1, 2 ** 18) == want


def test_int64_and_float64_routes_agree_exactly():
    rng = np.random.default_rng(1)
    q = _fp8(rng, (7, 64))
    k = _fp8(rng, (3000, 64), scale=50.0)
    a = I.scores_exact(q, k).astype(np.float64) * I.SCORE_UNIT
    b = I.scores_f64(q, k)
    assert np.array_equal(a, b)


def test_score_special_cases():
    # key equal to the query: the score is the sum of squares
    rng = np.random.default_rng(2)
    q = _fp8(rng, 64)
    v = F.e4m3_decode(q)
    assert I.full_scores(q, q[None, :])[0] == np.sum(v * v)
    # one-hot query picks out one channel of each key
    q1 = np.zeros(64, dtype=np.uint8); q1[5] = 0x38    # 1.0 at channel 5
    k = _fp8(rng, (10, 64))
    assert np.array_equal(I.full_scores(q1, k), F.e4m3_decode(k[:, 5]))


def test_causal_limit_masks_later_positions():
    rng = np.random.default_rng(3)
    q, k = _fp8(rng, 64), _fp8(rng, (50, 64))
    s = I.full_scores(q, k, limit=20)
    assert np.all(np.isneginf(s[21:])) and np.all(np.isfinite(s[:21]))
    assert np.array_equal(s[:21], I.full_scores(q, k)[:21])


def test_reindex_equals_full_on_pool_positions():
    rng = np.random.default_rng(4)
    q, k = _fp8(rng, 64), _fp8(rng, (300, 64))
    pool = np.array([3, 7, 100, 299, -1, -1])
    s = I.reindex_scores(q, k, pool)
    full = I.full_scores(q, k)
    assert np.array_equal(s[:4], full[[3, 7, 100, 299]])
    assert np.all(np.isneginf(s[4:]))


def _brute_topk(scores, k, pos=None):
    n = len(scores)
    pos = list(range(n)) if pos is None else list(pos)
    cand = [i for i in range(n) if np.isfinite(scores[i]) and pos[i] >= 0]
    cand.sort(key=lambda i: (-scores[i], pos[i]))
    out = sorted(pos[i] for i in cand[:k])
    return out + [-1] * (k - len(out))


@pytest.mark.parametrize("seed", range(6))
def test_topk_vs_sorted_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    s = rng.integers(-5, 6, n).astype(np.float64)        # many ties
    s[rng.random(n) < 0.1] = -np.inf
    for k in (1, 3, n // 2 + 1, n, n + 7):
        assert T.topk(s, k).tolist() == _brute_topk(s, k)


def test_topk_int_scores_and_index_map():
    rng = np.random.default_rng(7)
    pos = np.sort(rng.choice(10000, 300, replace=False))
    pos[-20:] = -1
    s = rng.integers(0, 30, 300).astype(np.float64)
    s[pos < 0] = -np.inf
    got = T.topk(s, 50, index_map=pos)
    assert got.tolist() == _brute_topk(s, 50, pos)
    assert np.all(np.diff(got[got >= 0]) > 0)


def test_topk_with_scores_reports_selected_values():
    s = np.array([3.0, 1.0, 7.0, -np.inf, 7.0])
    idx, vals = T.topk_with_scores(s, 4)
    assert idx.tolist() == [0, 1, 2, 4]
    assert vals.tolist() == [3.0, 1.0, 7.0, 7.0]
    idx, vals = T.topk_with_scores(s, 6)
    assert idx.tolist() == [0, 1, 2, 4, -1, -1] and np.isnan(vals[-1])


def test_top_k_of_pool_equals_top_k_of_all():
    rng = np.random.default_rng(8)
    q, k = _fp8(rng, 64), _fp8(rng, (50000, 64))
    s = I.full_scores(q, k)
    pool = T.candidate_pool(s, 16384)
    assert pool.shape == (16384,) and np.all(np.diff(pool) > 0)
    pool_scores = s[pool]
    a = T.topk(pool_scores, 2048, index_map=pool)
    b = T.topk(s, 2048)
    assert np.array_equal(a, b)


def test_pool_smaller_context_pads():
    s = np.array([1.0, 5.0, 2.0])
    assert T.candidate_pool(s, 8).tolist() == [0, 1, 2, -1, -1, -1, -1, -1]
