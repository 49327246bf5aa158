"""GPU parity: the HIP path against the CPU oracle, element by element.

Bar: bit-exact sorted index sets per row (including the count of -1 padding)
and equal value multisets by bit pattern.  Inputs are seeded and synthetic.
"""
import json
import os

import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import workloads
from workloads import Workload
from tests.gpu_helpers import POISON, assert_parity, dev, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_rows.json")


def _dense(name, api, scores, k, lens=None, ps=64, pt=None):
    B, L = scores.shape
    if api == "paged":
        if lens is None:
            lens = np.full(B, L, dtype=np.int32)
        if pt is None:
            npg = (L + ps - 1) // ps
            pt = np.broadcast_to(np.arange(npg, dtype=np.int32), (B, npg)).copy()
        return Workload(name, "paged", k, B, scores, L=L, lens=lens.astype(np.int32),
                        page_table=pt.astype(np.int32), page_size=ps)
    return Workload(name, "raw", k, B, scores, L=L,
                    lens=None if lens is None else lens.astype(np.int32))


@pytest.mark.parametrize("seed", [42, 43, 44, 45])
@pytest.mark.parametrize("name", workloads.NAMES)
def test_named_workloads(name, seed):
    w = workloads.make(name, seed=seed)
    print("case", name, "seed", seed, flush=True)
    got = run_gpu(w)
    assert_parity(w, got, run_oracle(w))


def test_named_workloads_deterministic():
    """The selected sets never change between runs; with one workgroup per row
    the slot order does not either (split rows place chunks as they finish)."""
    old = os.environ.get("ETS_ROW_SPLIT")
    try:
        for name in ("C3", "C4"):
            w = workloads.make(name, seed=44)
            os.environ.pop("ETS_ROW_SPLIT", None)
            a = run_gpu(w)
            b = run_gpu(w, out_fill=-5)
            np.testing.assert_array_equal(np.sort(a, axis=1), np.sort(b, axis=1))
            os.environ["ETS_ROW_SPLIT"] = "0"
            a = run_gpu(w)
            b = run_gpu(w, out_fill=-5)
            np.testing.assert_array_equal(a, b)
    finally:
        if old is None:
            os.environ.pop("ETS_ROW_SPLIT", None)
        else:
            os.environ["ETS_ROW_SPLIT"] = old


@pytest.mark.parametrize("k", [1, 7, 1024, 2048])
def test_short_and_boundary_lengths(k):
    rng = np.random.default_rng(k)
    L = 2 * k + 64
    lens = np.array([0, 1, 2, 3, 5, max(k - 1, 0), k, k + 1, 2 * k, L], dtype=np.int32)
    x = rng.standard_normal((lens.shape[0], L)).astype(np.float32)
    w = _dense("short", "raw", x, k, lens)
    assert_parity(w, run_gpu(w), run_oracle(w))
    # an infinite tail beyond each row's length must be ignored
    poisoned = x.copy()
    for b, n in enumerate(lens):
        poisoned[b, n:] = np.inf
    got = run_gpu(w, scores=poisoned)
    assert_parity(w, got, run_oracle(w), check_values=False)


def test_golden_hand_rows():
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        bits = np.array([int(b, 16) for b in case["bits"]], dtype=np.uint32)
        n = bits.shape[0]
        L = max(n, 4)
        row = np.zeros((1, L), dtype=np.uint32)
        row[0, :n] = bits
        w = _dense(case["name"], "raw", row.view(np.float32), case["k"],
                   np.array([n], dtype=np.int32))
        got = run_gpu(w)[0]
        assert sorted(got[got != -1].tolist()) == case["expect"], case["name"]
        assert int((got == -1).sum()) == case["k"] - len(case["expect"]), case["name"]


@pytest.mark.parametrize("k", [1, 1024, 2048])
@pytest.mark.parametrize("L", [2048, 32768])
def test_all_equal_rows(k, L):
    x = np.full((3, L), 0.75, dtype=np.float32)
    x[1] = -0.0
    x[2] = np.float32(1.0e-40)  # subnormal
    w = _dense("equal", "raw", x, k)
    assert_parity(w, run_gpu(w), run_oracle(w))


def test_all_subnormal_and_signed_zero_rows():
    rng = np.random.default_rng(5)
    L = 20000
    sub = rng.integers(1, 1 << 23, size=(2, L), dtype=np.uint32)
    sub[1] |= np.uint32(0x80000000)
    zeros = np.where(rng.random((1, L)) < 0.5, np.uint32(0), np.uint32(0x80000000)).astype(np.uint32)
    x = np.concatenate([sub, zeros]).view(np.float32)
    for k in (1024, 2048):
        w = _dense("subnormal", "raw", x, k)
        assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("pool", [1, 2, 3, 17, 300])
def test_heavy_ties(pool):
    rng = np.random.default_rng(pool)
    vals = rng.standard_normal(pool).astype(np.float32)
    x = vals[rng.integers(0, pool, size=(6, 32768))]
    lens = np.array([32768, 30000, 4097, 2049, 1025, 20000], dtype=np.int32)
    for k in (1024, 2048):
        w = _dense("ties", "raw", x, k, lens)
        assert_parity(w, run_gpu(w), run_oracle(w))


def test_ties_at_the_lowest_key():
    """Ties on key 0 (bit pattern 0xFFFFFFFF), the key the padding slots also
    hold: rows whose length is not a multiple of 4 must still take the
    lowest real positions."""
    rng = np.random.default_rng(8)
    L = 32768
    bits = np.full((4, L), 0xFFFFFFFF, dtype=np.uint32)
    bits[1, rng.integers(0, L, size=700)] = np.float32(2.0).view(np.uint32)
    bits[2, ::3] = np.float32(-1.0).view(np.uint32)
    x = bits.view(np.float32)
    lens = np.array([32767, 30001, 4097, 2050], dtype=np.int32)
    for k in (1, 1024, 2048):
        w = _dense("key0-ties", "raw", x, k, lens)
        assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("copies", [1, 2, 64, 127, 128, 129, 200, 255, 256, 257, 300])
def test_threshold_key_with_copies(copies):
    """The k-th largest score repeated `copies` times at random positions, with
    k - copies // 2 larger scores: the kernel takes the lowest-position half of
    the copies.  On one workgroup, copies of at most 256 are ranked directly
    (entries ordered by key, then position; 8 lanes per entry up to 128, 4
    above), more are resolved by position; row groups rank at most 128.
    Rows that fit one workgroup and rows split over a row group."""
    rng = np.random.default_rng(1000 + copies)
    for L, lens in ((32768, [32768, 20000, 8192]), (70001, [70001, 40000])):
        B = len(lens)
        x = (rng.standard_normal((B, L)) - 4.0).astype(np.float32)  # below the copies
        for k in (1024, 2048):
            y = x.copy()
            for b, n in enumerate(lens):
                pos = rng.permutation(n)
                above = k - copies // 2
                y[b, pos[:above]] = (rng.random(above) + 2.0).astype(np.float32)
                y[b, pos[above:above + copies]] = np.float32(1.5)
            w = _dense("copies", "raw", y, k, np.array(lens, dtype=np.int32))
            assert_parity(w, run_gpu(w), run_oracle(w))


def test_largest_scores_away_from_the_first_waves():
    """A row whose largest scores all sit where the last waves of a 1024-lane
    workgroup read (positions 2048..4095 of every 4096) and whose first
    waves hold only small ones: the first round's bounds come from the
    first waves, so the threshold lies in the bin that holds every key above
    their range."""
    rng = np.random.default_rng(12)
    L = 32768
    x = (rng.standard_normal((4, L)) * 1e-3).astype(np.float32)
    late = (np.arange(L) % 4096) >= 2048
    x[0, late] += 100.0
    x[1, late] = rng.standard_normal(int(late.sum())).astype(np.float32) + 50.0
    x[2, late & (np.arange(L) % 3 == 0)] = 7.0   # ties above the first waves' range
    x[3] = -x[3]
    x[3, late] -= 1.0                              # the late half lowest instead
    lens = np.array([32768, 30000, 20000, 16384], dtype=np.int32)
    for k in (1, 1024, 2048):
        w = _dense("late-max", "raw", x, k, lens)
        assert_parity(w, run_gpu(w), run_oracle(w))


def test_concentrated_rows_small_batch():
    rng = np.random.Generator(np.random.PCG64(9))
    x = np.stack([workloads.concentrated_row(rng, 32768) for _ in range(6)])
    lens = np.array([32768, 32768, 20000, 5000, 3000, 2049], dtype=np.int32)
    for k in (1024, 2048):
        w = _dense("concentrated", "raw", x, k, lens)
        assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("L", [32769, 70001, 100000])
def test_rows_longer_than_one_tile(L):
    rng = np.random.default_rng(L)
    x = rng.standard_normal((3, L)).astype(np.float32)
    lens = np.array([L, L - 1, 40000], dtype=np.int32)
    for k in (1024, 2048):
        w = _dense("long", "raw", x, k, lens)
        assert_parity(w, run_gpu(w), run_oracle(w))
    rng2 = np.random.Generator(np.random.PCG64(L))
    y = np.stack([workloads.concentrated_row(rng2, L) for _ in range(2)])
    w = _dense("long-concentrated", "raw", y, 2048)
    assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("L", [8191, 4099])
def test_unaligned_rows(L):
    """Odd row capacity: the scalar-load layout."""
    rng = np.random.default_rng(L)
    x = rng.standard_normal((4, L)).astype(np.float32)
    lens = np.array([L, L - 3, 1500, 1024], dtype=np.int32)
    w = _dense("unaligned", "raw", x, 1024, lens)
    assert_parity(w, run_gpu(w), run_oracle(w))
    # a row-stride view that is not a multiple of four
    big = rng.standard_normal((4, L + 1)).astype(np.float32)
    t = torch.from_numpy(big).to(dev())[:, :L]
    out = ets.topk_raw(t, 1024, torch.from_numpy(lens).to(dev()))
    w2 = _dense("strided", "raw", np.ascontiguousarray(big[:, :L]), 1024, lens)
    assert_parity(w2, out.cpu().numpy(), run_oracle(w2))


@pytest.mark.parametrize("ps", [1, 16, 48, 64, 100])
def test_paged_page_sizes(ps):
    rng = np.random.default_rng(ps)
    B, L = 5, 9600
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.array([9600, 9599, 5000, 1025, 7], dtype=np.int32)
    npg = (L + ps - 1) // ps
    pt = np.stack([rng.permutation(npg) + 3 for _ in range(B)]).astype(np.int32)
    w = _dense("paged", "paged", x, 1024, lens, ps=ps, pt=pt)
    assert_parity(w, run_gpu(w), run_oracle(w))


def test_ragged_small_and_odd():
    rng = np.random.default_rng(77)
    lengths = np.array([0, 1, 1023, 1024, 1025, 5001, 32768, 40000, 3], dtype=np.int32)
    starts = np.zeros_like(lengths)
    starts[1:] = np.cumsum(lengths[:-1])
    packed = rng.standard_normal(int(lengths.sum())).astype(np.float32)
    for k in (1, 1024, 2048):
        w = Workload("ragged", "ragged", k, lengths.shape[0], packed, row_starts=starts,
                     lengths=lengths)
        assert_parity(w, run_gpu(w), run_oracle(w))


def test_empty_batch_and_output_stride():
    d = dev()
    s = torch.empty((0, 128), dtype=torch.float32, device=d)
    out = ets.topk_raw(s, 16)
    assert out.shape == (0, 16)
    # output rows wider than k: only the first k slots are written
    x = np.random.default_rng(1).standard_normal((3, 5000)).astype(np.float32)
    wide = torch.full((3, 1500), 99, dtype=torch.int32, device=d)
    ets.topk_raw(torch.from_numpy(x).to(d), 1024, out=wide[:, :1024])
    torch.cuda.synchronize(d)
    wn = wide.cpu().numpy()
    assert (wn[:, 1024:] == 99).all()
    w = _dense("stride", "raw", x, 1024)
    assert_parity(w, wn[:, :1024], run_oracle(w))


def test_invalid_arguments_raise():
    d = dev()
    s = torch.zeros((2, 64), dtype=torch.float32, device=d)
    with pytest.raises(ets.EtsError):
        ets.topk_raw(s, 0)
    with pytest.raises(ets.EtsError):
        ets.topk_raw(s, 4096)
    with pytest.raises(TypeError):
        ets.topk_raw(s.double(), 8)


# Row capacities at and around each resident tile size (2048 and 4096 scores
# on 256 / 512 lanes, 8192 / 16384 / 32768 on 1024 lanes).
@pytest.mark.parametrize("L", [1100, 2048, 2049, 4096, 4097, 8192, 8193, 16384, 16385, 32768])
def test_every_tile_size(L):
    rng = np.random.default_rng(L)
    print("case tile L", L, flush=True)
    x = rng.standard_normal((4, L)).astype(np.float32)
    lens = np.array([L, L - 1, (L + 1) // 2, 1030], dtype=np.int32)
    for k in (1, 1024):
        w = _dense("tile", "raw", x, k, lens)
        assert_parity(w, run_gpu(w), run_oracle(w))
    pt = np.stack([rng.permutation((L + 63) // 64) for _ in range(4)]).astype(np.int32)
    w = _dense("tile-paged", "paged", x, 1024, lens, pt=pt)
    assert_parity(w, run_gpu(w), run_oracle(w))
    crng = np.random.Generator(np.random.PCG64(L))
    y = np.stack([workloads.concentrated_row(crng, L) for _ in range(2)])
    w = _dense("tile-concentrated", "raw", y, min(2048, L - 1))
    assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("hint", [1500, 3000, 6000])
def test_ragged_hint_below_row_length(hint):
    """Rows longer than the length hint take the streamed passes of the
    hinted tile size."""
    rng = np.random.default_rng(hint)
    lengths = np.array([hint, 3 * hint + 5, 20000, 1025, 0], dtype=np.int32)
    starts = np.zeros_like(lengths)
    starts[1:] = np.cumsum(lengths[:-1])
    packed = rng.standard_normal(int(lengths.sum())).astype(np.float32)
    d = dev()
    for k in (1, 1024):
        w = Workload("ragged-short-hint", "ragged", k, lengths.shape[0], packed,
                     row_starts=starts, lengths=lengths)
        out = ets.topk_ragged(torch.from_numpy(packed).to(d), torch.from_numpy(starts).to(d),
                              torch.from_numpy(lengths).to(d), k, max_len=hint)
        torch.cuda.synchronize()
        assert_parity(w, out.cpu().numpy(), run_oracle(w))


@pytest.mark.parametrize("overlap", [False, True])
def test_variable_windows(overlap):
    """Per-row windows inside dense rows through the ragged call: row b reads
    [row_starts[b], row_starts[b] + lengths[b]) of the flat score buffer and
    its indices are absolute.  Overlapping windows (sliding windows over one
    sequence, as in decode) read shared scores; long windows take the row-group
    path."""
    rng = np.random.default_rng(2024 + overlap)
    if overlap:
        B = 4
        lengths = np.array([70001, 120000, 262144, 99999], dtype=np.int32)
        starts = (np.arange(B, dtype=np.int64) * 3001 + 7).astype(np.int32)
        total = int((starts.astype(np.int64) + lengths).max())
        flat = rng.standard_normal(total).astype(np.float32)
    else:
        B, L = 6, 40000
        offs = rng.integers(0, L, B)
        offs[0] = 0
        lengths = np.array([rng.integers(0, L - o + 1) for o in offs], dtype=np.int32)
        lengths[1] = L - offs[1]
        starts = (np.arange(B) * L + offs).astype(np.int32)
        flat = rng.standard_normal(B * L).astype(np.float32)
    d = dev()
    for k in (1, 1024, 2048):
        print("case windows overlap", overlap, "k", k, flush=True)
        w = Workload("windows", "ragged", k, B, flat, row_starts=starts, lengths=lengths)
        out = ets.topk_ragged(torch.from_numpy(flat).to(d), torch.from_numpy(starts).to(d),
                              torch.from_numpy(lengths).to(d), k, max_len=int(lengths.max()))
        torch.cuda.synchronize()
        assert_parity(w, out.cpu().numpy(), run_oracle(w))


@pytest.mark.parametrize("api", ["raw", "paged"])
def test_dense_length_clamp_readings(api):
    """Dense lengths outside [0, L] are clamped on both sides: a negative
    length selects nothing (all -1), a length above L reads the whole row."""
    rng = np.random.default_rng(606)
    B, L, k = 6, 4096, 1024
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.array([-1, -5000, L + 1, 2 ** 31 - 1, 0, 2000], dtype=np.int32)
    pt = np.stack([rng.permutation(L // 64) for _ in range(B)]).astype(np.int32)
    w = _dense("clamp", api, x, k, lens=lens, pt=pt if api == "paged" else None)
    got = run_gpu(w)
    want = run_oracle(w)
    assert (want[0] == -1).all() and (want[1] == -1).all()
    assert_parity(w, got, want)


def test_ragged_negative_lengths():
    """A negative ragged length counts as 0: the row is all padding."""
    rng = np.random.default_rng(607)
    lengths = np.array([3000, -1, 5000, -70000, 0, 1500], dtype=np.int32)
    n = np.maximum(lengths, 0)
    starts = np.zeros_like(lengths)
    starts[1:] = np.cumsum(n[:-1])
    packed = rng.standard_normal(int(n.sum()) + 8).astype(np.float32)
    for k in (1, 1024):
        w = Workload("ragged-neg", "ragged", k, lengths.size, packed, row_starts=starts,
                     lengths=lengths)
        got = run_gpu(w)
        want = run_oracle(w)
        assert (want[1] == -1).all() and (want[3] == -1).all()
        assert_parity(w, got, want)


@pytest.mark.parametrize("name", ["C3", "C5"])
def test_twenty_calls_select_the_same_sets(name):
    """The same input 20 times on one stream: every call selects the same sets
    (a split row may order its slots differently), and they are the oracle's."""
    w = workloads.make(name, seed=46)
    d = dev()
    s = torch.from_numpy(w.scores).to(d)
    out = torch.empty((w.B, w.k), dtype=torch.int32, device=d)
    if w.api == "paged":
        lens = torch.from_numpy(w.lens).to(d)
        pt = torch.from_numpy(w.page_table).to(d)
        ws = ets.new_workspace(w.B, w.L, w.k, d)
        call = lambda: ets.topk_paged(s, lens, pt, out, w.page_size, workspace=ws)
    else:
        st = torch.from_numpy(w.row_starts).to(d)
        ln = torch.from_numpy(w.lengths).to(d)
        ws = ets.new_workspace(w.B, w.max_len, w.k, d)
        call = lambda: ets.topk_ragged(s, st, ln, w.k, max_len=w.max_len, out=out, workspace=ws)
    first = None
    for i in range(20):
        out.fill_(-3)
        call()
        got = np.sort(out.cpu().numpy(), axis=1)
        if ws is not None:
            assert ets.workspace_error(ws) == 0
        if first is None:
            first = got
            assert_parity(w, out.cpu().numpy(), run_oracle(w))
        else:
            bad = np.nonzero((got != first).any(axis=1))[0]
            assert bad.size == 0, "call %d: %d rows differ from the first call" % (i, bad.size)


def _ordered_rows(rng, kind, B, L):
    x = rng.standard_normal((B, L)).astype(np.float32)
    if kind == "ascending":
        x = np.sort(x, axis=1)
    elif kind == "descending":
        x = -np.sort(x, axis=1)
    elif kind == "late-max":
        # the float4 groups of the first 8 waves of a 1024-lane workgroup
        # (positions 4 (v T + t), t < 512) hold small scores only, so the
        # bounds taken from those waves are far below the threshold
        idx = np.arange(L)
        first = ((idx // 4) % 1024) < 512
        x[:, first] = x[:, first] * 0.25 - 3.0
    elif kind == "ties":
        x = rng.integers(-40, 40, size=(B, L)).astype(np.float32) / 8
    return x


@pytest.mark.parametrize("kind", ["normal", "ascending", "descending", "late-max", "ties"])
@pytest.mark.parametrize("L", [16384, 32768])
def test_long_rows_by_score_order(kind, L):
    """Long rows whose scores are sorted either way, whose largest scores all
    sit away from the waves whose loads land first, or that hold few distinct
    values, at lengths from just above 8k to the full tile."""
    kinds = ["normal", "ascending", "descending", "late-max", "ties"]
    rng = np.random.default_rng(1000 * kinds.index(kind) + L)
    B = 8
    x = _ordered_rows(rng, kind, B, L)
    lens = np.array([L, L - 1, L - 3, 3 * L // 4 + 1, L // 2, L // 2 - 5, 8193, 8192],
                    dtype=np.int32)
    for k in (1, 2, 64, 500, 1024):
        for api in ("raw", "paged"):
            print("case ordered", kind, "L", L, "k", k, api, flush=True)
            w = _dense("ordered", api, x, k, lens=lens,
                       pt=np.stack([rng.permutation(L // 64) for _ in range(B)]) if api == "paged" else None)
            assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("k", [1, 64, 256, 512, 1024, 2048])
def test_k_sweep_on_c3(k):
    """Runtime k over its range on the C3 shape (paged, B = 64, seq_lens up
    to 32768), the k sweep of the measurement."""
    base = workloads.make("C3", seed=47)
    w = Workload("C3-k%d" % k, "paged", k, base.B, base.scores, L=base.L, lens=base.lens,
                 page_table=base.page_table, page_size=base.page_size)
    print("case C3 k", k, flush=True)
    assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("B", [1, 8, 256, 512])
def test_decode_batches(B):
    """Full 32768-score paged rows at the decode batch sizes of the latency
    sweep, up to twice the compute-unit count."""
    rng = np.random.Generator(np.random.PCG64(900 + B))
    L, k, ps = 32768, 1024, 64
    x = workloads.normal_dense(rng, B, L)
    pt = np.stack([rng.permutation(L // ps) for _ in range(B)]).astype(np.int32)
    w = Workload("decode", "paged", k, B, x, L=L, lens=np.full(B, L, dtype=np.int32),
                 page_table=pt, page_size=ps)
    print("case decode B", B, flush=True)
    assert_parity(w, run_gpu(w), run_oracle(w))


def _window_oracle(x, lens, wins, pt, ps, k):
    """Each row's window [w_b, n_b) selected by the oracle's ragged call on the
    rows' flat buffer (row b's window starts at b * L + w_b), then mapped to
    paged slots of the row positions."""
    import oracle
    B, L = x.shape
    n = np.clip(lens.astype(np.int64), 0, L)
    w = np.clip(wins.astype(np.int64), 0, n)
    starts = (np.arange(B) * L + w).astype(np.int32)
    flat = oracle.topk_ragged(np.ascontiguousarray(x.reshape(-1)), starts, (n - w).astype(np.int32), k)
    out = np.full((B, k), -1, np.int32)
    for b in range(B):
        v = flat[b][flat[b] != -1].astype(np.int64) - b * L
        out[b, :v.size] = pt[b, v // ps] * ps + v % ps
    return out


def _run_window(x, lens, wins, pt, ps, k):
    d = dev()
    out = torch.full((x.shape[0], k), POISON, dtype=torch.int32, device=d)
    ets.topk_paged(torch.from_numpy(x).to(d), torch.from_numpy(lens).to(d),
                   torch.from_numpy(pt).to(d), out, ps, window_starts=torch.from_numpy(wins).to(d))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("ps", [64, 48])
@pytest.mark.parametrize("L", [32768, 70000])
def test_paged_windows(L, ps):
    """A window per row on the paged call (ets_topk_paged_window): row b selects
    among [window_starts[b], seq_lens[b]), both clamped, and emits paged slots
    of row positions; rows that fit one workgroup (L = 32768) and rows split
    over row groups (L = 70000)."""
    rng = np.random.default_rng(3000 + L + ps)
    lens = np.array([L, L, L - 7, 20001, 5000, 2049, 1500, L, L], dtype=np.int32)
    wins = np.array([0, 1, 63, 64 * 7, 1000, 2048, 2000, L - 1, -3], dtype=np.int32)
    B = lens.size
    x = rng.standard_normal((B, L)).astype(np.float32)
    npg = -(-L // ps)
    pt = np.stack([rng.permutation(npg) for _ in range(B)]).astype(np.int32)
    for k in (1, 1024, 2048):
        print("case windows L", L, "ps", ps, "k", k, flush=True)
        got = _run_window(x, lens, wins, pt, ps, k)
        want = _window_oracle(x, lens, wins, pt, ps, k)
        gs, ws_ = np.sort(got, axis=1), np.sort(want, axis=1)
        bad = np.nonzero((gs != ws_).any(axis=1))[0]
        assert bad.size == 0, "rows %s differ" % bad.tolist()


def test_paged_windows_on_page_boundaries():
    """Windows that start on a page boundary equal the plain paged call on the
    rows shifted by the window, with the page table shifted by its pages: the
    oracle's own paged map, no formula in the test."""
    import oracle
    rng = np.random.default_rng(3100)
    B, L, ps, k = 5, 32768, 64, 1024
    lens = np.array([L, 30000, 12345, 4096, L], dtype=np.int32)
    wins = np.array([0, 64, 640, 4096, 64 * 500], dtype=np.int32)
    x = rng.standard_normal((B, L)).astype(np.float32)
    pt = np.stack([rng.permutation(L // ps) for _ in range(B)]).astype(np.int32)
    got = _run_window(x, lens, wins, pt, ps, k)
    xs = np.zeros_like(x)
    pts = np.zeros_like(pt)
    for b in range(B):
        xs[b, :L - wins[b]] = x[b, wins[b]:]
        pts[b, :pt.shape[1] - wins[b] // ps] = pt[b, wins[b] // ps:]
    want = oracle.topk_paged(xs, (lens - wins).astype(np.int32), pts, ps, k)
    np.testing.assert_array_equal(np.sort(got, axis=1), np.sort(want, axis=1))
