"""GPU parity of the row-group path (several workgroups per row, one launch).

The path is chosen by the library's heuristic or forced with ETS_ROW_SPLIT
(read at every call); its results must equal the oracle's and the
one-workgroup path's.  The workspace's counters and tables must come back
zero after every call.
"""
import contextlib
import ctypes
import os

import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import oracle
import workloads
from workloads import Workload
from tests.gpu_helpers import WS_HDR, WS_ROW, assert_parity, dev, run_gpu, run_oracle, workspace_dirty

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def split(g, min_chunk=4):
    """Forces g workgroups per row.  min_chunk (ETS_MIN_CHUNK, default 4)
    sets the fewest scores per member chunk: 4 divides even short rows
    among all g members, which the geometry tests below rely on; None keeps
    the library's default (4096)."""
    saved = {v: os.environ.get(v) for v in ("ETS_ROW_SPLIT", "ETS_MIN_CHUNK")}
    os.environ["ETS_ROW_SPLIT"] = str(g)
    if min_chunk is None:
        os.environ.pop("ETS_MIN_CHUNK", None)
    else:
        os.environ["ETS_MIN_CHUNK"] = str(min_chunk)
    try:
        yield
    finally:
        for v, old in saved.items():
            if old is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = old


def _raw(name, x, k, lens=None):
    B, L = x.shape
    return Workload(name, "raw", k, B, x, L=L, lens=None if lens is None else lens.astype(np.int32))


def _assert_clean(ws):
    """The error word is zero, and so is the rest of the workspace: counters,
    histogram tables and tie lists."""
    torch.cuda.synchronize()
    e = ets.workspace_error(ws)
    assert e == 0, "a call stopped waiting for its row group (error word %d)" % e
    nz = workspace_dirty(ws)
    assert nz == 0, "%d workspace words left non-zero" % nz


def _cached_workspaces():
    return [w for w in ets._ws_cache.values()]


@pytest.fixture(autouse=True)
def _error_words_stay_zero():
    """After every test: no call on the implicit workspaces stopped waiting for
    its row group (the error word, read and cleared through the C ABI)."""
    for ws in _cached_workspaces():
        ets.workspace_error(ws)
    yield
    for ws in _cached_workspaces():
        e = ets.workspace_error(ws)
        assert e == 0, "a call stopped waiting for its row group (error word %d)" % e


_G64 = pytest.param(64, marks=pytest.mark.skip(
    reason="64 members per row exceed one XCD's 32 row-group slots on MI355X: a ticketed "
           "grid can then stall until the bounded waits expire (seen on a 4096-workgroup "
           "grid; tests/test_dispatch_model.py models it); the library rejects G above "
           "the device's cap"))


@pytest.mark.parametrize("g", [2, 3, 8, 17, 32, _G64])
@pytest.mark.parametrize("name", ["C2", "C3"])
def test_forced_split_matches_single(name, g):
    w = workloads.make(name, seed=45)
    w.B = 16
    w.scores = np.ascontiguousarray(w.scores[:16])
    w.lens = w.lens[:16]
    w.page_table = w.page_table[:16]
    print("case", name, "G", g, flush=True)
    with split(0):
        single = run_gpu(w)
    with split(g):
        got = run_gpu(w)
    want = run_oracle(w)
    assert_parity(w, single, want)
    assert_parity(w, got, want)
    for ws in _cached_workspaces():
        _assert_clean(ws)


@pytest.mark.parametrize("g", [2, 4, 16])
def test_forced_split_concentrated(g):
    """88% of a row in one 12-bit bucket: the tie list overflows and the group
    narrows the bucket by further rounds, down to positions among equal keys."""
    rng = np.random.Generator(np.random.PCG64(11))
    x = np.stack([workloads.concentrated_row(rng, 32768) for _ in range(4)])
    lens = np.array([32768, 20000, 4097, 2050], dtype=np.int32)
    for k in (1, 1024, 2048):
        w = _raw("conc-split", x, k, lens)
        print("case concentrated G", g, "k", k, flush=True)
        with split(g):
            assert_parity(w, run_gpu(w), run_oracle(w))
    for ws in _cached_workspaces():
        _assert_clean(ws)


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


@pytest.mark.parametrize("g", [2, 8])
def test_split_special_values(g):
    """Signed zeros, subnormals, infinities and NaNs ranked by key in the group path."""
    rng = np.random.default_rng(77)
    L = 16384
    bits = rng.integers(0, 2 ** 32, size=(4, L), dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F800000, 0xFF800000,
                         0x7FC00000, 0xFFC00000, 0x3F800000], dtype=np.uint32)
    bits[1] = specials[rng.integers(0, specials.size, size=L)]
    bits[2, :] = 0x80000000          # all -0.0 ...
    bits[2, ::97] = 0x00000000       # ... with some +0.0 above them
    bits[3] = rng.integers(1, 1 << 23, size=L).astype(np.uint32)  # positive subnormals
    x = bits.view(np.float32)
    for k in (1, 1000, 2048):
        w = _raw("special-split", x, k)
        with split(g):
            assert_parity(w, run_gpu(w), run_oracle(w))


def test_split_short_rows_and_empty_chunks():
    """Rows at and just above k, where most chunks of a 17-way split are empty."""
    rng = np.random.default_rng(5)
    k = 1024
    L = 8192
    lens = np.array([0, 1, k - 1, k, k + 1, k + 3, 2 * k, 4100, L], dtype=np.int32)
    x = rng.standard_normal((lens.size, L)).astype(np.float32)
    w = _raw("short-split", x, k, lens)
    for g in (2, 17, 32):
        with split(g):
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


def test_split_paged_odd_page_size():
    """A page size that is not a power of two reads page ids from global memory."""
    rng = np.random.default_rng(32)
    B, L, ps, k = 6, 12000, 48, 1024
    npg = (L + ps - 1) // ps
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = rng.integers(1000, L + 1, size=B).astype(np.int32)
    pt = np.stack([rng.permutation(npg) for _ in range(B)]).astype(np.int32)
    w = Workload("paged-odd", "paged", k, B, x, L=L, lens=lens, page_table=pt, page_size=ps)
    for g in (3, 8):
        with split(g):
            assert_parity(w, run_gpu(w), run_oracle(w))


def test_ragged_row_longer_than_hint():
    """A chunk longer than one tile (the row outgrew the hint) is streamed."""
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


def _edge_rows(rng, lengths, first_lead, kinds):
    """A packed buffer of ragged rows: row b starts (first_lead + b) % 4
    scores past a 16-byte boundary, rows are separated by 4 to 7 scores of
    +1e30 that belong to no row (larger than any row score: a neighbour's
    score read as the row's would be selected), and the last row ends the
    buffer 1 to 3 scores past a 16-byte boundary (one score shorter than
    asked where it would end on one).  kinds[b]: "normal" N(0,1); "pad-key" mostly the bit pattern
    0xFFFFFFFF (key 0, the padding's key) with fewer other scores than k
    asks, so the threshold is key 0 and ties go by position; "equal" all 1.0."""
    parts, starts, lens = [], [], []
    pos = 0
    for b, n in enumerate(lengths):
        lead = (first_lead + b) % 4
        gap = (lead - pos) % 4 + (4 if b else 0)
        if b == len(lengths) - 1 and (pos + gap + n) % 4 == 0:
            n -= 1
        parts.append(np.full(gap, 1e30, dtype=np.float32))
        pos += gap
        starts.append(pos)
        lens.append(n)
        if kinds[b] == "normal":
            row = rng.standard_normal(n).astype(np.float32)
        elif kinds[b] == "equal":
            row = np.ones(n, dtype=np.float32)
        else:
            row = np.full(n, 0xFFFFFFFF, dtype=np.uint32).view(np.float32)
            few = rng.choice(n, size=min(n, 40), replace=False)
            row[few] = rng.standard_normal(few.size).astype(np.float32)
        parts.append(row)
        pos += n
    packed = np.ascontiguousarray(np.concatenate(parts))
    return packed, np.array(starts, dtype=np.int32), np.array(lens, dtype=np.int32)


@pytest.mark.parametrize("first_lead", [0, 1, 2, 3])
def test_ragged_row_edges(first_lead):
    """Packed ragged rows on the row-group path, starting at every offset
    from a 16-byte boundary: nothing outside a row is ever selected, whatever
    its neighbours hold, also where the threshold is the padding slots' own
    key (0) and ties go by position."""
    rng = np.random.default_rng(500 + first_lead)
    lengths = [5003, 4098, 7001, 3073, 6150]
    kinds = ["normal", "pad-key", "equal", "pad-key", "normal"]
    packed, starts, lens = _edge_rows(rng, lengths, first_lead, kinds)
    assert ((starts % 4) == (first_lead + np.arange(5)) % 4).all()
    assert starts[-1] + lens[-1] == packed.size and packed.size % 4 != 0
    d = dev()
    for k in (64, 1000, 2048):
        w = Workload("ragged-edges", "ragged", k, 5, packed, row_starts=starts, lengths=lens)
        want = run_oracle(w)
        for g in (2, 3, 8):
            with split(g):
                print("first_lead", first_lead, "k", k, "G", g, flush=True)
                assert_parity(w, run_gpu(w), want)


@pytest.mark.parametrize("k", [64, 2048])
def test_default_min_chunk_leaves_members_empty(k):
    """With the library's fewest scores per chunk (4096), a 16-way split of
    rows shorter than 16 * 4096 gives each row ceil(n / 4096) non-empty
    members and leaves the rest empty; rows longer than that are divided
    evenly.  Both must match the oracle."""
    rng = np.random.default_rng(77 + k)
    L = 81920
    lens = np.array([k + 1, 4095, 4096, 4097, 12289, 40964, 65536, 65537, L], dtype=np.int32)
    x = rng.standard_normal((lens.size, L)).astype(np.float32)
    x[3, 4096] = 1e9  # the only score of the second member of a 4097-score row
    w = _raw("min-chunk", x, k, lens)
    want = run_oracle(w)
    for g in (2, 16, 20):
        with split(g, min_chunk=None):
            assert_parity(w, run_gpu(w), want)


def test_spread_lengths_at_the_default_split():
    """Long raw rows whose lengths spread far below the longest (the host
    sees only the longest): the default split and chunking against the
    oracle."""
    rng = np.random.Generator(np.random.PCG64(1008))
    B, L, k = 4, 262144, 2048
    x = workloads.normal_dense(rng, B, L)
    lens = rng.integers(L // 8, L, size=B, endpoint=True).astype(np.int32)
    lens[0] = L // 8
    w = _raw("spread", x, k, lens)
    assert_parity(w, run_gpu(w), run_oracle(w))


def test_one_workspace_across_shapes_and_apis():
    """Every call returns its workspace's counters and tables to zero, so one
    buffer serves calls of any shape and map in turn."""
    d = dev()
    ws = ets.new_workspace(128, 262144, 2048, d)  # the largest batch below
    _assert_clean(ws)
    cases = [workloads.make(n, seed=60 + i) for i, n in enumerate(["C3", "C5", "C2", "C4", "C3"])]
    for w in cases:
        s = torch.from_numpy(w.scores).to(d)
        out = torch.full((w.B, w.k), 3, dtype=torch.int32, device=d)
        if w.api == "paged":
            ets.topk_paged(s, torch.from_numpy(w.lens).to(d), torch.from_numpy(w.page_table).to(d),
                           out, w.page_size, workspace=ws)
        elif w.api == "raw":
            ets.topk_raw(s, w.k, None if w.lens is None else torch.from_numpy(w.lens).to(d),
                         out=out, workspace=ws)
        else:
            ets.topk_ragged(s, torch.from_numpy(w.row_starts).to(d),
                            torch.from_numpy(w.lengths).to(d), w.k, max_len=w.max_len, out=out,
                            workspace=ws)
        print("case", w.name, flush=True)
        _assert_clean(ws)
        assert_parity(w, out.cpu().numpy(), run_oracle(w))


def test_workspace_init_zero_fills():
    d = dev()
    ws = torch.full((4 * (WS_HDR + 2 * WS_ROW),), 0xAB, dtype=torch.uint8, device=d)
    ets.workspace_init(ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws).item() == 0


def test_split_call_rejects_small_workspace():
    lib = ets._load()
    d = dev()
    B, L, k = 4, 65536, 64
    need = ets.workspace_size(B, L, k)
    assert need > 0
    x = torch.zeros((B, L), dtype=torch.float32, device=d)
    out = torch.empty((B, k), dtype=torch.int32, device=d)
    ws = torch.zeros(need, dtype=torch.uint8, device=d)
    st = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), L, B, L, None, k, out.data_ptr(), k)
    assert lib.ets_topk_raw(*args, ws.data_ptr(), need - 1, st) == 3
    assert lib.ets_topk_raw(*args, None, 0, st) == 3
    assert lib.ets_topk_raw(*args, ws.data_ptr() + 4, need - 4, st) == 3  # misaligned
    assert lib.ets_topk_raw(*args, ws.data_ptr(), need, st) == 0
    _assert_clean(ws)


def test_workspace_size_formula():
    # header + per-row record, three 4096-bin tables and the 4096-entry tie list
    env = os.environ.pop("ETS_ROW_SPLIT", None)
    try:
        for B in (1, 4, 64):
            assert ets.workspace_size(B, 262144, 2048) == 4 * (WS_HDR + B * WS_ROW)
        assert ets.workspace_size(4096, 4096, 1024) == 0
    finally:
        if env is not None:
            os.environ["ETS_ROW_SPLIT"] = env


def test_large_row_group_grids():
    """64 rows of 32 members (2048 workgroups, more than the device holds at
    once: eight index grids of 8 rows, since 32 members exceed one shader
    engine's slots) and rows of over a million scores on the default split:
    every bounded wait ends in time (error word zero) over repeated calls, and
    the output matches the oracle."""
    d = dev()
    k = 2048
    for B, L, g in ((64, 131072, 32), (2, 1500000, None)):
        print("case large grid B", B, "L", L, "G", g, flush=True)
        x = np.random.default_rng(B + L).standard_normal((B, L)).astype(np.float32)
        s = torch.from_numpy(x).to(d)
        out = torch.empty((B, k), dtype=torch.int32, device=d)
        with (split(g) if g is not None else contextlib.nullcontext()):
            ws = ets.new_workspace(B, L, k, d)
            for _ in range(4):
                ets.topk_raw(s, k, None, out=out, workspace=ws)
                e = ets.workspace_error(ws)
                assert e == 0, "a call stopped waiting for its row group (error word %d)" % e
        w = _raw("large-grid", x, k)
        assert_parity(w, out.cpu().numpy(), run_oracle(w))
        _assert_clean(ws)


@pytest.mark.parametrize("B,L,k,g,window", [
    (134, 55023, 4, 32, True),    # the random call whose ticketed grid ran into a bounded wait
    (64, 131072, 2048, 16, False),
    (40, 262144, 1024, 9, False),
    (70, 40000, 100, 12, True),
])
def test_groups_above_one_engine_on_grids_beyond_the_device(B, L, k, g, window):
    """G above one shader engine's row-group slots on a batch whose grid does
    not fit the device at once: the library runs it as several index grids
    (as many whole rows per XCD as fit), never as a ticketed grid, and every
    call matches the oracle with the error word zero and the workspace clean."""
    d = dev()
    cu, nx, occ = ets.device_limits()
    assert ets.ticket_cap(cu, nx, occ) < g <= ets.group_cap(cu, nx, occ)
    rng = np.random.default_rng(B * L + g)
    x = rng.standard_normal((B, L)).astype(np.float32)
    lens = rng.integers(L // 2, L + 1, size=B).astype(np.int32)
    ps = 64
    P = -(-L // ps)
    pt = np.stack([rng.permutation(P) for _ in range(B)]).astype(np.int32)
    wins = rng.integers(0, L // 4, size=B).astype(np.int32) if window else None
    print("case B", B, "L", L, "k", k, "G", g, "window", window, flush=True)
    with split(g):
        ws = ets.new_workspace(B, L, k, d)
        out = torch.full((B, k), -7, dtype=torch.int32, device=d)
        for _ in range(2):
            ets.topk_paged(torch.from_numpy(x).to(d), torch.from_numpy(lens).to(d), torch.from_numpy(pt).to(d),
                           out, ps, workspace=ws,
                           window_starts=None if wins is None else torch.from_numpy(wins).to(d))
            _assert_clean(ws)
    got = out.cpu().numpy()
    n = np.clip(lens.astype(np.int64), 0, L)
    lo = np.zeros(B, np.int64) if wins is None else np.clip(wins.astype(np.int64), 0, n)
    starts = (np.arange(B) * L + lo).astype(np.int32)
    flat = oracle.topk_ragged(np.ascontiguousarray(x.reshape(-1)), starts, (n - lo).astype(np.int32), k,
                              threads=8)
    want = np.full((B, k), -1, np.int32)
    for b in range(B):
        v = flat[b][flat[b] != -1].astype(np.int64) - b * L
        want[b, :v.size] = pt[b, v // ps] * ps + v % ps
    np.testing.assert_array_equal(np.sort(got, axis=1), np.sort(want, axis=1))


def _banded(rng, B, L):
    """Each row: four bands of scores at well-separated centres, each band a
    few ULPs wide, so that whole bands tie bit for bit."""
    centres = np.array([-3.0, 0.5, 2.0, 7.0], dtype=np.float32)
    band = rng.integers(0, 4, size=(B, L))
    ulps = rng.integers(0, 4, size=(B, L)).astype(np.int32)
    x = centres[band]
    return (x.view(np.int32) + ulps).view(np.float32)


def _narrow(rng, B, L):
    """Each row inside [1, 1 + 2^-13): at most 1024 distinct scores."""
    return (np.float32(1.0).view(np.int32) + rng.integers(0, 1024, size=(B, L)).astype(np.int32)).view(np.float32)


@pytest.mark.parametrize("kind", ["banded", "narrow"])
@pytest.mark.parametrize("g", [0, 4, 16])
def test_banded_and_narrow_rows(kind, g):
    """Few distinct scores per row: the threshold falls inside a band of
    equal keys, resolved by position among equal keys on one workgroup
    (G = 0) and across a row group."""
    rng = np.random.default_rng(500 + g)
    L = 65536
    x = (_banded if kind == "banded" else _narrow)(rng, 3, L)
    lens = np.array([L, 40001, 20000], dtype=np.int32)
    for k in (1, 1024, 2048):
        print("case", kind, "G", g, "k", k, flush=True)
        w = _raw(kind, x, k, lens)
        with split(g):
            assert_parity(w, run_gpu(w), run_oracle(w))
    for ws in _cached_workspaces():
        _assert_clean(ws)


def test_split_override_above_cap_is_rejected():
    """ETS_ROW_SPLIT above the device's row-group cap is an argument error,
    reported before anything is enqueued, never a silent clamp."""
    cu, xcd, occ = ets.device_limits()
    cap = ets.group_cap(cu, xcd, occ)
    assert cap >= 2
    d = dev()
    x = torch.zeros((2, 65536), dtype=torch.float32, device=d)
    with split(cap + 1):
        assert ets.row_split(2, 65536, cu, xcd, occ) == -1
        with pytest.raises(ets.EtsError) as e:
            ets.topk_raw(x, 64)
        assert e.value.status == 1
        with pytest.raises(ets.EtsError):
            ets.workspace_size(2, 65536, 64)
    with split(cap):
        out = ets.topk_raw(x, 64)
        torch.cuda.synchronize()
        assert out.shape == (2, 64)


@pytest.mark.parametrize("B,L,k", [(128, 262144, 2048), (192, 131072, 1024), (192, 65536, 1024),
                                   (256, 262144, 2048)])
def test_default_heuristic_large_batches(B, L, k):
    """The heuristic's choices for long rows at large batches: chunks of 32768
    scores held in registers on a ticketed grid (B = 128 and 256, L = 262144:
    G = 8; B = 192, L = 131072: G = 4; B = 192, L = 65536: G = 2), also where
    the rows alone would fill the compute units."""
    limits = ets.device_limits()
    print("case default B", B, "L", L, "G", ets.row_split(B, L, *limits), flush=True)
    rng = np.random.Generator(np.random.PCG64(B * 7 + L))
    x = workloads.normal_dense(rng, B, L)
    lens = rng.integers(L // 2, L, size=B, endpoint=True).astype(np.int32)
    w = _raw("default-large", x, k, lens)
    d = dev()
    ws = ets.new_workspace(B, L, k, d)
    out = torch.full((B, k), 5, dtype=torch.int32, device=d)
    ets.topk_raw(torch.from_numpy(x).to(d), k, torch.from_numpy(lens).to(d), out=out, workspace=ws)
    if ws is not None:
        assert ets.workspace_error(ws) == 0
    assert_parity(w, out.cpu().numpy(), run_oracle(w))
    if ws is not None:
        _assert_clean(ws)


@pytest.mark.parametrize("api", ["raw", "paged"])
@pytest.mark.parametrize("g,L", [(3, 65536), (2, 60000), (5, 131072)])
def test_forced_split_resident_chunks_above_16384(api, g, L):
    """Chunks of 16385 to 32768 scores: each member holds 32 keys per lane."""
    rng = np.random.Generator(np.random.PCG64(g * 100 + L % 97))
    B, k, ps = 4, 1024, 64
    x = workloads.normal_dense(rng, B, L)
    lens = np.array([L, L - 1, L // 2 + 3, 33000], dtype=np.int32)
    if api == "raw":
        w = _raw("chunks-big", x, k, lens)
    else:
        pt = np.stack([rng.permutation(-(-L // ps)) for _ in range(B)]).astype(np.int32)
        w = Workload("chunks-big-paged", "paged", k, B, x, L=L, lens=lens, page_table=pt,
                     page_size=ps)
    print("case", api, "G", g, "L", L, flush=True)
    with split(g):
        assert_parity(w, run_gpu(w), run_oracle(w))


@pytest.mark.parametrize("g", [4, 5])
def test_split_k2_one_score_tail_chunk(g):
    """k = 2 with a member whose chunk holds one score (a 49-score row at G = 4:
    chunks of 16, 16, 16 and 1): such a chunk offers no lower bound."""
    rng = np.random.default_rng(9)
    L = 52
    lens = np.array([49, 45, 33, 52, 3, 17], dtype=np.int32)
    x = rng.standard_normal((lens.size, L)).astype(np.float32)
    x[1, 44] = 50.0  # the only score of its member's chunk is the row's largest
    for k in (1, 2, 3):
        w = _raw("tail-one", x, k, lens)
        with split(g):
            assert_parity(w, run_gpu(w), run_oracle(w))


def test_workspace_error_word_is_copied_and_cleared():
    """ets_workspace_error copies the word into a caller buffer on the stream
    and clears it; a call that needed no workspace reports 0."""
    d = dev()
    ws = ets.new_workspace(4, 262144, 2048, d)
    flag = torch.full((1,), -1, dtype=torch.int32, device=d)
    ets.workspace_error_async(ws, flag)
    torch.cuda.synchronize()
    assert flag.item() == 0
    ws.view(torch.int32)[32] = 7  # planted from the host
    ets.workspace_error_async(ws, flag)
    torch.cuda.synchronize()
    assert flag.item() == 7
    assert int(ws.view(torch.int32)[32].item()) == 0
    ets.workspace_error_async(None, flag)
    torch.cuda.synchronize()
    assert flag.item() == 0


def test_stale_ticket_sets_the_error_word():
    """A ticketed grid on a workspace whose ticket counter is not zero (a
    planted stale value): every workgroup finds no row, ends at once and the
    error word says so; the last one re-arms the counter, so the next call on
    the same workspace is exact again."""
    d = dev()
    limits = ets.device_limits()
    cu, nx, occ = limits
    B, L, k = 96, 131072, 2048
    G = ets.row_split(B, L, *limits)
    assert 2 <= G <= ets.ticket_cap(*limits) and nx * G * -(-B // nx) > cu * occ, "needs a ticketed grid"
    x = workloads.normal_dense(np.random.Generator(np.random.PCG64(3)), B, L)
    s = torch.from_numpy(x).to(d)
    ws = ets.new_workspace(B, L, k, d)
    ws.view(torch.int32)[0] = 1 << 30  # stale ticket
    out = torch.full((B, k), 7, dtype=torch.int32, device=d)
    ets.topk_raw(s, k, out=out, workspace=ws)
    assert ets.workspace_error(ws) == 2
    assert int(torch.count_nonzero(out != 7).item()) == 0  # nothing was selected
    _assert_clean(ws)
    ets.topk_raw(s, k, out=out, workspace=ws)
    assert ets.workspace_error(ws) == 0
    assert_parity(_raw("after-stale", x, k), out.cpu().numpy(), run_oracle(_raw("after-stale", x, k)))
