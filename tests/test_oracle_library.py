"""Library pins of the oracle on the five named workloads, and fault injection.

* NumPy's stable ``argsort`` of the negated scores yields (value descending,
  position ascending); on rows with no NaN and no signed zero that is exactly
  the oracle's order, so the first m positions must match element by element.
* ``torch.topk`` is the ground truth of the pages' own test (sglang PR #36004
  digest, test excerpt); with ties the index set may differ, so the pages
  compare value multisets (PR #37591 digest, "Implementation breakdown" item 3)
  -- and so do we.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.checkers import check_row, split_output


def _rows(w):
    """Yield (row values of the valid prefix, row offset) per row of a workload."""
    rl = w.row_lengths
    for b in range(w.B):
        if w.api == "ragged":
            s = int(w.row_starts[b])
            yield w.scores[s:s + rl[b]], s
        else:
            yield w.scores[b, :rl[b]], 0


def _raw_oracle(oracle_mod, w, threads=8):
    if w.api == "ragged":
        out = oracle_mod.topk_ragged(w.scores, w.row_starts, w.lengths, w.k, threads=threads)
        return np.where(out >= 0, out - w.row_starts[:, None], -1)
    return oracle_mod.topk_raw(w.scores, w.k, w.lens, threads=threads)


@pytest.fixture(scope="module", params=workloads.NAMES)
def wl(request):
    return workloads.make(request.param, seed=42)


def test_numpy_stable_argsort(oracle_mod, wl):
    got = _raw_oracle(oracle_mod, wl)
    for b, (vals, _) in enumerate(_rows(wl)):
        assert not np.isnan(vals).any() and not (vals == 0).any()
        m = min(wl.k, vals.shape[0])
        want = np.argsort(-vals, kind="stable")[:m]
        np.testing.assert_array_equal(got[b, :m], want)
        assert (got[b, m:] == -1).all()


def test_torch_topk_value_multiset(oracle_mod, wl):
    got = _raw_oracle(oracle_mod, wl)
    for b, (vals, _) in enumerate(_rows(wl)):
        m = min(wl.k, vals.shape[0])
        ref = torch.topk(torch.from_numpy(vals.copy()), m, sorted=False).values.numpy()
        mine = vals[got[b, :m]]
        np.testing.assert_array_equal(np.sort(mine.view(np.uint32)), np.sort(ref.view(np.uint32)))


def test_invariants(oracle_mod, wl):
    got = _raw_oracle(oracle_mod, wl)
    for b, (vals, _) in enumerate(_rows(wl)):
        valid, npad = split_output(got[b])
        check_row(vals, wl.k, valid, npad)


def test_mapped_apis_agree_with_raw(oracle_mod, wl):
    raw = _raw_oracle(oracle_mod, wl)
    if wl.api == "paged":
        out = oracle_mod.topk_paged(wl.scores, wl.lens, wl.page_table, wl.page_size, wl.k,
                                    threads=8)
        ps = wl.page_size
        r = np.maximum(raw, 0)
        want = np.where(raw >= 0, np.take_along_axis(wl.page_table, r // ps, axis=1) * ps + r % ps, -1)
        np.testing.assert_array_equal(out, want)
    elif wl.api == "ragged":
        out = oracle_mod.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, threads=8)
        np.testing.assert_array_equal(out, np.where(raw >= 0, raw + wl.row_starts[:, None], -1))


def test_concentrated_workload_shape():
    """C4 stresses one coarse bucket: most scores are 1 + j 2^-23, j = 0 .. 8."""
    w = workloads.make("C4", seed=42)
    bits = w.scores.view(np.uint32)
    cluster = (bits >= 0x3F800000) & (bits <= 0x3F800008)
    frac = cluster.mean()
    assert 0.88 <= frac < 0.90
    assert (w.scores.view(np.uint32) >> 16 == 0x3F80).mean() > 0.88


def test_fault_injection_is_caught(oracle_mod):
    w = workloads.make("C2", seed=43)
    got = _raw_oracle(oracle_mod, w)
    vals = w.scores[0]
    valid, npad = split_output(got[0])
    check_row(vals, w.k, valid, npad)
    # swap the weakest selected position for the best unselected one
    bad = valid.copy()
    unsel = np.setdiff1d(np.arange(vals.shape[0]), valid)
    bad[np.argmin(vals[bad])] = unsel[np.argmax(vals[unsel])]
    with pytest.raises(AssertionError):
        check_row(vals, w.k, bad, npad)
    # a duplicated position
    dup = valid.copy()
    dup[1] = dup[0]
    with pytest.raises(AssertionError):
        check_row(vals, w.k, dup, npad)
    # a lost entry turned into padding
    with pytest.raises(AssertionError):
        check_row(vals, w.k, valid[:-1], npad + 1)
    # ties at the threshold broken the wrong way
    row = np.array([1.0, 0.5, 0.5, 0.5], dtype=np.float32)
    check_row(row, 2, np.array([0, 1]), 0)
    with pytest.raises(AssertionError):
        check_row(row, 2, np.array([0, 3]), 0)
