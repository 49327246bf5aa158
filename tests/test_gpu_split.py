"""GPU parity of the row-split path (several workgroups per row).

The path is forced with ETS_ROW_SPLIT (read by the library at every call);
its results must equal the oracle's and the one-workgroup path's.
"""
import contextlib
import os

import numpy as np
import pytest

import workloads
from workloads import Workload
from tests.gpu_helpers import assert_parity, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def split(g):
    old = os.environ.get("ETS_ROW_SPLIT")
    os.environ["ETS_ROW_SPLIT"] = str(g)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("ETS_ROW_SPLIT", None)
        else:
            os.environ["ETS_ROW_SPLIT"] = old


def _raw(name, x, k, lens=None):
    B, L = x.shape
    return Workload(name, "raw", k, B, x, L=L, lens=None if lens is None else lens.astype(np.int32))


@pytest.mark.parametrize("g", [2, 3, 8, 17])
@pytest.mark.parametrize("name", ["C2", "C3"])
def test_forced_split_matches_single(name, g):
    w = workloads.make(name, seed=45)
    w.B = 16
    w.scores = np.ascontiguousarray(w.scores[:16])
    w.lens = w.lens[:16]
    w.page_table = w.page_table[:16]
    with split(0):
        single = run_gpu(w)
    with split(g):
        got = run_gpu(w)
    want = run_oracle(w)
    assert_parity(w, single, want)
    assert_parity(w, got, want)


@pytest.mark.parametrize("g", [4, 16])
def test_forced_split_concentrated(g):
    rng = np.random.Generator(np.random.PCG64(11))
    x = np.stack([workloads.concentrated_row(rng, 32768) for _ in range(4)])
    lens = np.array([32768, 20000, 4097, 2050], dtype=np.int32)
    for k in (1024, 2048):
        w = _raw("conc-split", x, k, lens)
        with split(g):
            assert_parity(w, run_gpu(w), run_oracle(w))


def test_split_long_rows_default_heuristic():
    rng = np.random.default_rng(21)
    L = 100000
    x = rng.standard_normal((3, L)).astype(np.float32)
    lens = np.array([L, 70001, 1500], dtype=np.int32)
    for k in (1, 1024, 2048):
        w = _raw("long", x, k, lens)
        assert_parity(w, run_gpu(w), run_oracle(w))


def test_split_all_equal_and_ties():
    L = 70000
    x = np.full((2, L), 2.5, dtype=np.float32)
    x[1, ::7] = 3.0  # 10000 winners above a sea of ties
    for k in (1, 2048):
        w = _raw("equal-split", x, k)
        assert_parity(w, run_gpu(w), run_oracle(w))


def test_split_concentrated_long_rows():
    rng = np.random.Generator(np.random.PCG64(12))
    x = np.stack([workloads.concentrated_row(rng, 65536) for _ in range(2)])
    w = _raw("conc-long", x, 2048)
    assert_parity(w, run_gpu(w), run_oracle(w))


def test_split_paged_long_rows():
    rng = np.random.default_rng(31)
    B, L, ps, k = 3, 65536, 64, 1024
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.array([65536, 40000, 33000], dtype=np.int32)
    pt = np.stack([rng.permutation(L // ps) for _ in range(B)]).astype(np.int32)
    w = Workload("paged-split", "paged", k, B, x, L=L, lens=lens, page_table=pt, page_size=ps)
    assert_parity(w, run_gpu(w), run_oracle(w))


def test_ragged_row_longer_than_hint():
    """The last chunk of a row runs to the row's end, whatever the hint said."""
    import torch
    import exact_top_selection_amd as ets
    from tests.gpu_helpers import dev
    rng = np.random.default_rng(41)
    lengths = np.array([50000, 90000, 3000, 1024], dtype=np.int32)
    starts = np.zeros_like(lengths)
    starts[1:] = np.cumsum(lengths[:-1])
    packed = (rng.standard_normal(int(lengths.sum())) * 1e-3 + 1.0).astype(np.float32)
    w = Workload("ragged-hint", "ragged", 2048, 4, packed, row_starts=starts, lengths=lengths)
    d = dev()
    for hint in (40000, 60000):
        out = ets.topk_ragged(torch.from_numpy(packed).to(d), torch.from_numpy(starts).to(d),
                              torch.from_numpy(lengths).to(d), 2048, max_len=hint)
        torch.cuda.synchronize()
        assert_parity(w, out.cpu().numpy(), run_oracle(w))
