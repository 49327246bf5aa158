"""Closed-form pins of the oracle: hand rows from tests/golden, rows whose
answer is known without sorting, and the three output maps.

Output maps: sglang PR #36004 digest, "Implementation breakdown" item 4 and the
test excerpt (identity page table => emitted paged slot == token position,
output pre-filled with -1); PR #37591 digest, the CoopParams excerpt (ragged
rows addressed by row_starts / lengths).
"""
import json
import os

import numpy as np
import pytest

from tests.checkers import check_row, split_output

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_rows.json")


def _load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_golden_hand_rows(oracle_mod, case):
    bits = np.array([int(b, 16) for b in case["bits"]], dtype=np.uint32).reshape(1, -1)
    k = case["k"]
    got = oracle_mod.topk_raw(bits, k)[0]
    valid, npad = split_output(got)
    assert sorted(valid.tolist()) == case["expect"]
    assert npad == k - len(case["expect"])


@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (100, 100), (100, 7), (3000, 1024), (50, 2048)])
def test_all_equal_takes_lowest_positions(oracle_mod, n, k):
    row = np.full((2, n), -2.75, dtype=np.float32)
    got = oracle_mod.topk_raw(row, k)
    m = min(k, n)
    for b in range(2):
        assert sorted(got[b, :m].tolist()) == list(range(m))
        assert (got[b, m:] == -1).all()


@pytest.mark.parametrize("n,k", [(10, 3), (4096, 1024), (5000, 2048)])
def test_monotone_rows(oracle_mod, n, k):
    inc = np.linspace(-5, 5, n, dtype=np.float64).astype(np.float32)
    assert np.unique(inc).shape[0] == n
    m = min(k, n)
    got = oracle_mod.topk_raw(inc[None, :], k)[0]
    assert sorted(got[:m].tolist()) == list(range(n - m, n))
    got = oracle_mod.topk_raw(inc[::-1].copy()[None, :], k)[0]
    assert sorted(got[:m].tolist()) == list(range(m))


def test_planted_maxima(oracle_mod):
    rng = np.random.default_rng(7)
    B, L, k = 6, 20000, 1024
    x = rng.standard_normal((B, L)).astype(np.float32)
    planted = []
    for b in range(B):
        pos = rng.choice(L, size=k, replace=False)
        x[b, pos] = (100.0 + rng.random(k)).astype(np.float32)
        planted.append(np.sort(pos))
    got = oracle_mod.topk_raw(x, k)
    for b in range(B):
        np.testing.assert_array_equal(np.sort(got[b]), planted[b])


def test_lengths_clamp_and_poisoned_tail(oracle_mod):
    rng = np.random.default_rng(3)
    B, L, k = 6, 3000, 1024
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.array([0, 1, 1023, 1024, 1025, 2999], dtype=np.int32)
    poisoned = x.copy()
    for b in range(B):
        poisoned[b, lens[b]:] = np.inf
    a = oracle_mod.topk_raw(x, k, lens)
    b_ = oracle_mod.topk_raw(poisoned, k, lens)
    np.testing.assert_array_equal(a, b_)
    for b in range(B):
        valid, npad = split_output(a[b])
        check_row(x[b, :lens[b]], k, valid, npad)
    # lengths outside [0, L] clamp
    c = oracle_mod.topk_raw(x, k, np.array([-5, L + 9, L, 0, L, L], dtype=np.int32))
    assert (c[0] == -1).all() and (c[3] == -1).all()
    np.testing.assert_array_equal(c[1], oracle_mod.topk_raw(x[1:2], k)[0])


def test_paged_identity_equals_raw(oracle_mod):
    rng = np.random.default_rng(11)
    B, L, ps, k = 3, 8192, 64, 1024
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.array([8192, 5000, 100], dtype=np.int32)
    pt = np.broadcast_to(np.arange(L // ps, dtype=np.int32), (B, L // ps)).copy()
    np.testing.assert_array_equal(oracle_mod.topk_paged(x, lens, pt, ps, k),
                                  oracle_mod.topk_raw(x, k, lens))


@pytest.mark.parametrize("ps", [1, 16, 64, 100])
def test_paged_permuted_table_closed_form(oracle_mod, ps):
    rng = np.random.default_rng(ps)
    B, L, k = 4, 6400, 700
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.array([6400, 6399, 1, 3333], dtype=np.int32)
    npages = (L + ps - 1) // ps
    pt = np.stack([rng.permutation(npages) + 7 for _ in range(B)]).astype(np.int32)
    raw = oracle_mod.topk_raw(x, k, lens)
    paged = oracle_mod.topk_paged(x, lens, pt, ps, k)
    for b in range(B):
        r = raw[b]
        want = np.where(r >= 0, pt[b, np.maximum(r, 0) // ps] * ps + np.maximum(r, 0) % ps, -1)
        np.testing.assert_array_equal(paged[b], want)


def test_ragged_matches_rows(oracle_mod):
    rng = np.random.default_rng(5)
    lengths = np.array([0, 7, 3000, 1024, 5000], dtype=np.int32)
    starts = np.zeros_like(lengths)
    starts[1:] = np.cumsum(lengths[:-1])
    packed = rng.standard_normal(int(lengths.sum()) + 13).astype(np.float32)
    k = 1024
    got = oracle_mod.topk_ragged(packed, starts, lengths, k)
    for b in range(lengths.shape[0]):
        row = packed[starts[b]:starts[b] + lengths[b]][None, :]
        raw = oracle_mod.topk_raw(row, k)[0] if lengths[b] else np.full(k, -1, np.int32)
        want = np.where(raw >= 0, raw + starts[b], -1)
        np.testing.assert_array_equal(got[b], want)


def test_threads_do_not_change_result(oracle_mod):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((37, 4000)).astype(np.float32)
    x[:, ::3] = 0.5  # many ties
    np.testing.assert_array_equal(oracle_mod.topk_raw(x, 1024, threads=1),
                                  oracle_mod.topk_raw(x, 1024, threads=8))
