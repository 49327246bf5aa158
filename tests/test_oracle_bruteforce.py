"""Brute-force pins of the oracle's selection on tiny rows.

Two definitions that do not use the oracle's sort:

* subset enumeration: among all m-subsets whose every score ranks at or above
  every unselected score, the one whose sorted position tuple is
  lexicographically smallest (that is the lowest-position tie-break);
* the rank formula: position i is selected iff
  #{j : s_j > s_i} + #{j < i : s_j == s_i} < k.

Scores are ranked here by a hand-written table over a small alphabet, so the
pins do not reuse the key transform either.
"""
import itertools

import numpy as np
import pytest

# alphabet in strictly increasing rank order (+0.0 ranks above -0.0)
ALPHABET = np.array([float("-inf"), -1.0, -0.0, 0.0, 1.4e-45, 1.0, float("inf")],
                    dtype=np.float32)


def _all_rows(n):
    idx = np.array(list(itertools.product(range(len(ALPHABET)), repeat=n)), dtype=np.int64)
    return idx  # ranks; scores = ALPHABET[idx]


def _subset_reference(ranks: np.ndarray, k: int) -> np.ndarray:
    """[R, m] lexicographically smallest valid position tuple per row."""
    R, n = ranks.shape
    m = min(k, n)
    if m == 0:
        return np.zeros((R, 0), dtype=np.int64)
    # candidate tuples in lexicographic order
    tuples = list(itertools.combinations(range(n), m))
    chosen = np.full(R, -1, dtype=np.int64)
    for t_i, t in enumerate(tuples):
        mask = np.zeros(n, dtype=bool)
        mask[list(t)] = True
        if m == n:
            valid = np.ones(R, dtype=bool)
        else:
            valid = ranks[:, mask].min(axis=1) >= ranks[:, ~mask].max(axis=1)
        take = valid & (chosen < 0)
        chosen[take] = t_i
    assert (chosen >= 0).all()
    return np.array(tuples, dtype=np.int64)[chosen]


def _rank_reference(ranks: np.ndarray, k: int) -> np.ndarray:
    R, n = ranks.shape
    gt = (ranks[:, None, :] > ranks[:, :, None]).sum(axis=2)
    lower = np.tril(np.ones((n, n), dtype=bool), k=-1)  # [i, j] true for j < i
    eq = ((ranks[:, None, :] == ranks[:, :, None]) & lower[None]).sum(axis=2)
    return (gt + eq) < k


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4, 5, 6])
def test_all_rows_over_alphabet(oracle_mod, n):
    ranks = _all_rows(n) if n > 0 else np.zeros((1, 0), dtype=np.int64)
    scores = ALPHABET[ranks].reshape(ranks.shape[0], n)
    for k in range(1, n + 2):
        got = oracle_mod.topk_raw(scores, k)
        m = min(k, n)
        assert (got[:, m:] == -1).all()
        got_sorted = np.sort(got[:, :m], axis=1)
        want = _subset_reference(ranks, k)
        np.testing.assert_array_equal(got_sorted, want)
        sel = _rank_reference(ranks, k)
        got_mask = np.zeros_like(sel)
        np.put_along_axis(got_mask, got[:, :m].astype(np.int64), True, axis=1)
        np.testing.assert_array_equal(got_mask, sel)


@pytest.mark.parametrize("seed", range(6))
def test_random_rows_rank_formula(oracle_mod, seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 300))
    R = 16
    # few distinct values so that ties are frequent
    pool = rng.standard_normal(int(rng.integers(1, 12))).astype(np.float32)
    ranks = rng.integers(0, pool.shape[0], size=(R, n))
    order = np.argsort(pool)
    rank_of = np.empty_like(order)
    rank_of[order] = np.arange(order.shape[0])
    scores = pool[ranks]
    for k in (1, max(1, n // 3), n, n + 5):
        got = oracle_mod.topk_raw(scores, k)
        sel = _rank_reference(rank_of[ranks], k)
        m = min(k, n)
        got_mask = np.zeros_like(sel)
        np.put_along_axis(got_mask, got[:, :m].astype(np.int64), True, axis=1)
        np.testing.assert_array_equal(got_mask, sel)
        assert (got[:, m:] == -1).all()
