"""Pins of the oracle's product-key selection against things other than itself.

The method (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)", section
"Meccanismo Core", item 2) selects the top-K of the N = n^2 summed scores
x1[a] + x2[b] through topk(x1 (+) x2) = topk(topk(x1) (+) topk(x2)).  These
tests check the oracle's two-stage result against a brute-force ranking of
all N binary32 sums, against the special case K = n where stage 1 keeps
everything, against exact ties on integer-valued scores, and the softmax
weights against closed forms.
"""
import math

import numpy as np
import pytest

import oracle


def brute_topk(x1, x2, K):
    """All N binary32 sums ranked by (sum desc, flat index asc)."""
    n = x1.shape[0]
    s = (x1[:, None] + x2[None, :]).astype(np.float32).reshape(-1)
    f = np.arange(n * n)
    order = np.lexsort((f, -s))
    return order[:K].astype(np.int32), s[order[:K]]


def test_brute_force_random_normal():
    rng = np.random.default_rng(1)
    mism = 0
    for trial in range(400):
        n = int(rng.choice([8, 16, 32, 64]))
        K = int(rng.integers(1, n + 1)) if trial % 3 else min(n, 64)
        x1 = rng.standard_normal(n).astype(np.float32)
        x2 = rng.standard_normal(n).astype(np.float32)
        idx, sc, w = oracle.select(x1, x2, K)
        bidx, bsc = brute_topk(x1, x2, K)
        if not np.array_equal(idx, bidx):
            # Only possible where binary32 rounding merges distinct sums:
            # the scores must then still agree element by element.
            assert np.array_equal(sc, bsc), (n, K)
            mism += 1
        np.testing.assert_array_equal(sc, bsc)
    assert mism == 0


def test_rounding_tie_follows_two_stage_contract():
    # x1[1] = 1 + 2^-23: both 1 + 2 and (1 + 2^-23) + 2 round to 3.0.
    # Brute force ranks f = 0 first (lower flat index); the two-stage method
    # sees only a = 1 in stage 1 and therefore returns f = 1*2 + 0 = 2.
    x1 = np.array([1.0, 1.0 + 2.0 ** -23], np.float32)
    x2 = np.array([2.0, -5.0], np.float32)
    idx, sc, w = oracle.select(x1, x2, 1)
    bidx, bsc = brute_topk(x1, x2, 1)
    assert bidx[0] == 0 and idx[0] == 2
    assert sc[0] == bsc[0] == np.float32(3.0)
    # With K = 2 both rows survive stage 1, so the tied sums (both 3.0 in
    # binary32, though not in exact arithmetic) are ordered by flat index.
    idx2, sc2, _ = oracle.select(x1, x2, 2)
    assert idx2.tolist() == [0, 2] and sc2.tolist() == [3.0, 3.0]


def test_k_equals_n_is_full_sort():
    rng = np.random.default_rng(2)
    for n in (4, 8, 16, 32):
        for _ in range(30):
            x1 = rng.standard_normal(n).astype(np.float32)
            x2 = rng.standard_normal(n).astype(np.float32)
            idx, sc, _ = oracle.select(x1, x2, n)
            bidx, bsc = brute_topk(x1, x2, n)
            np.testing.assert_array_equal(idx, bidx)
            np.testing.assert_array_equal(sc, bsc)


def test_integer_scores_exact_ties():
    # Small integers: every sum is exact, so ties are real ties and the
    # lower flat index must win, exactly as in the brute-force ranking.
    rng = np.random.default_rng(3)
    for trial in range(2000):
        n = int(rng.choice([4, 8, 16]))
        K = int(rng.integers(1, n + 1))
        x1 = rng.integers(-2, 3, n).astype(np.float32)
        x2 = rng.integers(-2, 3, n).astype(np.float32)
        idx, sc, _ = oracle.select(x1, x2, K)
        bidx, bsc = brute_topk(x1, x2, K)
        np.testing.assert_array_equal(idx, bidx, err_msg=f"trial {trial}")


def test_negative_zero_equals_positive_zero():
    x1 = np.array([-0.0, 0.0, -1.0, -2.0], np.float32)
    x2 = np.array([0.0, -0.0, -3.0, -4.0], np.float32)
    idx, sc, _ = oracle.select(x1, x2, 4)
    bidx, _ = brute_topk(x1, x2, 4)
    np.testing.assert_array_equal(idx, bidx)
    assert list(idx[:4]) == [0, 1, 4, 5]


def test_indices_distinct_and_in_range():
    rng = np.random.default_rng(4)
    n, K, units = 64, 64, 200
    x1 = rng.standard_normal((units, n)).astype(np.float32)
    x2 = rng.standard_normal((units, n)).astype(np.float32)
    idx, sc, w = oracle.select(x1, x2, K)
    assert idx.min() >= 0 and idx.max() < n * n
    for u in range(units):
        assert len(set(idx[u].tolist())) == K
        # output order: score non-increasing, lower index first on ties
        assert np.all(np.diff(sc[u]) <= 0)


def test_weights_closed_forms():
    rng = np.random.default_rng(5)
    n = 32
    x1 = rng.standard_normal((100, n)).astype(np.float32)
    x2 = rng.standard_normal((100, n)).astype(np.float32)
    # K = 1: the single weight is exactly one.
    _, _, w1 = oracle.select(x1, x2, 1)
    assert np.all(w1 == 1.0)
    # K = 2: logistic function of the score gap.
    _, sc, w2 = oracle.select(x1, x2, 2)
    d = sc[:, 0].astype(np.float64) - sc[:, 1].astype(np.float64)
    np.testing.assert_allclose(w2[:, 0], 1.0 / (1.0 + np.exp(-d)), rtol=0, atol=1e-15)
    # Any K: sums to one, non-increasing.
    _, sc, w = oracle.select(x1, x2, 24)
    np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=-1) <= 0)
    # ratio of weights equals exp of score difference
    r = w[:, 0] / w[:, 5]
    np.testing.assert_allclose(r, np.exp(sc[:, 0].astype(np.float64) - sc[:, 5]), rtol=1e-12)


def test_hand_worked_example():
    # x1 = [0.5, 2], x2 = [1, -1], K = 2.  Stage 1: A = (1, 0), B = (0, 1).
    # Candidates: f=2 -> 3.0, f=3 -> 1.0, f=0 -> 1.5, f=1 -> -0.5.
    # Top two: f=2 (3.0) then f=0 (1.5); weights 1/(1+e^-1.5), e^-1.5/(1+e^-1.5).
    x1 = np.array([0.5, 2.0], np.float32)
    x2 = np.array([1.0, -1.0], np.float32)
    idx, sc, w = oracle.select(x1, x2, 2)
    assert idx.tolist() == [2, 0]
    assert sc.tolist() == [3.0, 1.5]
    e = math.exp(-1.5)
    assert w[0] == pytest.approx(1 / (1 + e), abs=1e-16)
    assert w[1] == pytest.approx(e / (1 + e), abs=1e-16)


def test_rejects_bad_input():
    x = np.zeros(8, np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.select(x, x, 9)
    y = x.copy()
    y[3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.select(y, x, 2)
    y[3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.select(x, y, 2)


def test_threaded_select_matches_serial():
    rng = np.random.default_rng(6)
    x1 = rng.standard_normal((500, 128)).astype(np.float32)
    x2 = rng.standard_normal((500, 128)).astype(np.float32)
    a = oracle.select(x1, x2, 16)
    b = oracle.select(x1, x2, 16, threads=4)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
