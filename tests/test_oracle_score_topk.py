"""Pins of the oracle's indexer score and Top-K (CPU only).

Index score: brute-force integer dots on tiny inputs (every E4M3 value is an
integer multiple of 2^-9), an exact-rational weighted head sum, one-hot head
weights that isolate the ReLU of one head, and the +0 convention.
Top-K: a brute-force repeated-argmax selection, constructed ties, K >= n,
n_valid, and invariance under pool permutation.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import csa2 as O
from oracle import formats as F


def _rand_e4m3(rng, shape):
    b = rng.integers(0, 256, size=shape, dtype=np.uint16).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x7E          # no NaN codes (precondition)
    return b


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_index_dots_exact_vs_integer_bruteforce(seed):
    rng = np.random.default_rng(seed)
    key = _rand_e4m3(rng, (7, 8, 64))
    key[0] = 0x7E                          # +448 everywhere: largest magnitudes
    key[1] = 0x01                          # smallest subnormal
    q = _rand_e4m3(rng, (8, 64))
    exact = O.index_dots_bruteforce(key, q)            # int64, true dot * 2^18
    got = np.einsum("nhi,hi->nh", F.e4m3_value(key), F.e4m3_value(q))
    assert np.array_equal(got * 2.0 ** 18, exact.astype(np.float64))
    # the full score against an exact rational evaluation
    w = rng.random(8, dtype=np.float32)
    s = O.index_scores(key, q, w)
    for j in range(7):
        ex = sum(Fraction(float(w[h])) * max(Fraction(int(exact[j, h]), 1 << 18), Fraction(0))
                 for h in range(8))
        terms = sum(abs(float(w[h])) * abs(exact[j, h]) * 2.0 ** -18 for h in range(8))
        assert abs(Fraction(s[j]) - ex) <= Fraction(16 * 2.0 ** -53) * Fraction(terms)


def test_index_score_relu_per_head_and_positive_zero():
    # one-hot head weights isolate ReLU(dot_h); negative dots give +0.0
    rng = np.random.default_rng(3)
    key = _rand_e4m3(rng, (32, 8, 64))
    q = _rand_e4m3(rng, (8, 64))
    dots = O.index_dots_bruteforce(key, q) * 2.0 ** -18
    assert (dots < 0).any() and (dots > 0).any()
    for h in range(8):
        w = np.zeros(8, np.float32)
        w[h] = 1.0
        s = O.index_scores(key, q, w)
        assert np.array_equal(s, np.maximum(dots[:, h], 0.0))
        assert not np.signbit(s).any()
    # a ReLU applied after the head sum instead of per head would differ here
    w = np.ones(8, np.float32)
    s = O.index_scores(key, q, w)
    assert np.array_equal(s, np.maximum(dots, 0).sum(1))
    assert not np.array_equal(s, np.maximum(dots.sum(1), 0))


def test_index_scores_rows_subset_and_chunking():
    rng = np.random.default_rng(4)
    key = _rand_e4m3(rng, (300, 8, 64))
    q = _rand_e4m3(rng, (8, 64))
    w = rng.random(8, dtype=np.float32)
    full = O.index_scores(key, q, w, chunk=17)
    assert np.array_equal(full, O.index_scores(key, q, w))
    rows = np.array([299, 5, 5, 0, 123])
    assert np.array_equal(O.index_scores(key, q, w, rows=rows), full[rows])


@pytest.mark.parametrize("n,K", [(1, 1), (7, 3), (7, 7), (7, 10), (40, 5), (64, 64), (64, 1)])
def test_topk_vs_bruteforce_with_ties(n, K):
    rng = np.random.default_rng(n * 100 + K)
    s = rng.integers(0, 6, size=n).astype(np.float64)   # many exact ties, zeros
    got, _ = O.topk(s, K)
    assert np.array_equal(got, O.topk_bruteforce(s, K))
    # selected positions ascending, padding at the end
    v = got[got >= 0]
    assert np.all(np.diff(v) > 0) and np.all(got[len(v):] == -1)
    assert len(v) == min(n, K)


def test_topk_tie_goes_to_lower_index():
    s = np.array([1.0, 5.0, 3.0, 5.0, 5.0, 0.0])
    assert O.topk(s, 1)[0].tolist() == [1]
    assert O.topk(s, 2)[0].tolist() == [1, 3]
    assert O.topk(s, 4)[0].tolist() == [1, 2, 3, 4]
    assert O.topk(np.zeros(5), 2)[0].tolist() == [0, 1]
    # -0.0 and +0.0 compare equal: index decides
    assert O.topk(np.array([-0.0, 0.0, -0.0]), 2)[0].tolist() == [0, 1]


def test_topk_n_valid_and_gap():
    s = np.array([9.0, 1.0, 8.0, 7.0, 100.0])
    idx, gap = O.topk(s, 2, n_valid=4)
    assert idx.tolist() == [0, 2]
    assert gap == pytest.approx((8.0 - 7.0) / 8.0)
    idx, gap = O.topk(s, 3, n_valid=2)
    assert idx.tolist() == [0, 1, -1] and gap is None
    idx, gap = O.topk(s, 2, n_valid=0)
    assert idx.tolist() == [-1, -1]


def test_topk_permutation_invariance():
    rng = np.random.default_rng(9)
    s = rng.standard_normal(500) ** 2          # continuous: no ties straddle K
    perm = rng.permutation(500)                # new position p holds old entry perm[p]
    a, _ = O.topk(s, 37)
    b, _ = O.topk(s[perm], 37)
    assert sorted(perm[b].tolist()) == a.tolist()


def test_map_positions():
    cand = np.array([3, 10, 11, 40])
    assert O.map_positions(np.array([0, 2, 3, -1]), cand).tolist() == [3, 11, 40, -1]
