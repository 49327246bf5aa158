"""The measurement floors: the read-only launch must read exactly the spans a
selection launch reads (each workgroup reports its span's largest key), and
the empty launch must run."""
import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import workloads
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _keys(x: np.ndarray) -> np.ndarray:
    u = x.view(np.uint32).astype(np.uint64)
    return np.where(u >> 31 == 1, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.uint64)


def _expected(rows, G):
    """Largest key of chunk g of each row, chunks cut as the row groups cut them."""
    want = []
    for r in rows:
        n = r.size
        chunk = ((n + G - 1) // G + 3) & ~3
        for g in range(G):
            s = min(g * chunk, n)
            e = n if g == G - 1 else min(s + chunk, n)
            want.append(int(_keys(r[s:e]).max()) if e > s else 0)
    return np.array(want, dtype=np.uint64)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C5"])
def test_floor_read_reports_each_span_max(name):
    w = workloads.make(name, seed=7)
    d = dev()
    limits = ets.device_limits()
    if w.api == "ragged":
        G = max(1, ets.row_split(w.B, w.max_len, *limits))
        s = torch.from_numpy(w.scores).to(d)
        got = ets.floor_read(s, torch.from_numpy(w.lengths).to(d),
                             torch.from_numpy(w.row_starts).to(d), w.max_len)
        rows = [w.scores[a:a + n] for a, n in zip(w.row_starts, w.lengths)]
    else:
        G = max(1, ets.row_split(w.B, w.L, *limits))
        lens = None if w.lens is None else torch.from_numpy(w.lens).to(d)
        got = ets.floor_read(torch.from_numpy(w.scores).to(d), lens)
        n = w.lens if w.lens is not None else np.full(w.B, w.L)
        rows = [w.scores[b, :n[b]] for b in range(w.B)]
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32).astype(np.uint64)
    np.testing.assert_array_equal(got, _expected(rows, G))


def test_floor_read_unaligned_and_short_rows():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3001)).astype(np.float32)
    lens = np.array([0, 1, 3001, 1500, 7], dtype=np.int32)
    d = dev()
    got = ets.floor_read(torch.from_numpy(x).to(d), torch.from_numpy(lens).to(d))
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32).astype(np.uint64)
    np.testing.assert_array_equal(got, _expected([x[b, :lens[b]] for b in range(5)], 1))


def test_floor_launch_runs():
    d = dev()
    for B, L in ((1, 2048), (64, 32768), (4, 262144)):
        ets.floor_launch(B, L, d)
    torch.cuda.synchronize()
