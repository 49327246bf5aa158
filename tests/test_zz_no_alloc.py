"""The paged entry point that allocates nothing (ets_topk_paged_noalloc),
called through the C ABI and compared with ets_topk_paged (same arguments,
its own workspace): bit-exact sorted index sets per row, including the -1
count, on two calls in a row (the second smaller) that split their rows over
row groups and so use the static scratch, then on a shape that needs none,
and a shape beyond the scratch is rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import workloads
from tests.gpu_helpers import run_oracle
from workloads import Workload

pytestmark = pytest.mark.gpu

ETS_ERR_SCRATCH = 6
SCRATCH_BYTES = 4 << 20


def _case(seed, B, L, k, ps=64):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = workloads.normal_dense(rng, B, L)
    lens = rng.integers(L // 3, L, size=B, endpoint=True).astype(np.int32)
    pt = np.stack([rng.permutation(-(-L // ps)) for _ in range(B)]).astype(np.int32)
    return Workload("noalloc", "paged", k, B, x, L=L, lens=lens, page_table=pt, page_size=ps)


def _both(lib, w, d):
    """(noalloc output, error flag, existing entry point's output), both poisoned first."""
    s = torch.from_numpy(w.scores).to(d)
    lens = torch.from_numpy(w.lens).to(d)
    pt = torch.from_numpy(w.page_table).to(d)
    a = torch.full((w.B, w.k), 0x5A5A, dtype=torch.int32, device=d)
    b = torch.full((w.B, w.k), 0x3C3C, dtype=torch.int32, device=d)
    flag = torch.full((1,), -1, dtype=torch.int32, device=d)
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.ets_topk_paged_noalloc(s.data_ptr(), w.L, w.B, w.L, lens.data_ptr(), pt.data_ptr(),
                                    pt.shape[1], w.page_size, w.k, a.data_ptr(), w.k,
                                    flag.data_ptr(), stream)
    assert st == 0, st
    need = ets.workspace_size(w.B, w.L, w.k)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=d)
    st = lib.ets_topk_paged(s.data_ptr(), w.L, w.B, w.L, lens.data_ptr(), pt.data_ptr(),
                            pt.shape[1], w.page_size, w.k, b.data_ptr(), w.k,
                            ws.data_ptr() if need else None, need, stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return a.cpu().numpy(), int(flag.item()), b.cpu().numpy()


def _same_sets(got, want):
    gs, ws = np.sort(got, axis=1), np.sort(want, axis=1)
    bad = np.nonzero((gs != ws).any(axis=1))[0]
    assert bad.size == 0, "%d rows differ, first %d" % (bad.size, bad[0])


def test_noalloc_matches_the_workspace_call():
    lib = ets._load()
    d = torch.device("cuda:0")
    limits = ets.device_limits()
    cases = [_case(71, 8, 131072, 2048), _case(72, 3, 70000, 1024)]
    for w in cases:
        G = ets.row_split(w.B, w.L, *limits)
        print("case noalloc B", w.B, "L", w.L, "G", G, flush=True)
        assert G > 0, "the case must use the scratch"
        assert ets.workspace_size(w.B, w.L, w.k) <= SCRATCH_BYTES
        got, err, want = _both(lib, w, d)
        assert err == 0
        _same_sets(got, want)
        _same_sets(got, run_oracle(w))
    # one workgroup per row: no scratch needed, any batch
    w = workloads.make("C3", seed=73)
    got, err, want = _both(lib, w, d)
    assert err == 0
    _same_sets(got, want)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    lib = ets._load()
    d = torch.device("cuda:0")
    limits = ets.device_limits()
    B, L, k = 64, 262144, 2048
    assert ets.row_split(B, L, *limits) > 0 and ets.workspace_size(B, L, k) > SCRATCH_BYTES
    x = torch.zeros((1,), dtype=torch.float32, device=d)  # never read: rejected first
    lens = torch.zeros((B,), dtype=torch.int32, device=d)
    out = torch.full((B, k), 9, dtype=torch.int32, device=d)
    st = lib.ets_topk_paged_noalloc(x.data_ptr(), L, B, L, lens.data_ptr(), lens.data_ptr(),
                                    L // 64, 64, k, out.data_ptr(), k, None,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == ETS_ERR_SCRATCH
    assert b"scratch" in lib.ets_status_string(ETS_ERR_SCRATCH)
    torch.cuda.synchronize()
    assert int((out != 9).sum().item()) == 0


def test_noalloc_graph_replays_match_the_oracle():
    """Split calls captured in a HIP graph use the static scratch on every
    replay: four replays, each after an eager call of another shape on the
    same stream (which leaves the scratch zero in between), all equal the
    oracle, with the error flag at zero."""
    d = torch.device("cuda:0")
    limits = ets.device_limits()
    w = _case(81, 4, 70000, 1024)
    other = _case(82, 3, 131072, 2048)
    for c in (w, other):
        assert ets.row_split(c.B, c.L, *limits) > 0
    want = run_oracle(w)
    want_other = run_oracle(other)
    s = torch.from_numpy(w.scores).to(d)
    lens = torch.from_numpy(w.lens).to(d)
    pt = torch.from_numpy(w.page_table).to(d)
    out = torch.full((w.B, w.k), 7, dtype=torch.int32, device=d)
    flag = torch.full((1,), -1, dtype=torch.int32, device=d)
    s2 = torch.from_numpy(other.scores).to(d)
    lens2 = torch.from_numpy(other.lens).to(d)
    pt2 = torch.from_numpy(other.page_table).to(d)
    out2 = torch.full((other.B, other.k), 7, dtype=torch.int32, device=d)
    flag2 = torch.full((1,), -1, dtype=torch.int32, device=d)
    # one eager call first, so that the scratch has been zero-filled outside capture
    ets.topk_paged_noalloc(s, lens, pt, out, w.page_size, error_flag=flag)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            ets.topk_paged_noalloc(s, lens, pt, out, w.page_size, error_flag=flag)
    torch.cuda.synchronize()
    for rep in range(4):
        print("noalloc graph replay", rep, flush=True)
        out.fill_(7)
        flag.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        _same_sets(out.cpu().numpy(), want)
        out2.fill_(7)
        ets.topk_paged_noalloc(s2, lens2, pt2, out2, other.page_size, error_flag=flag2)
        torch.cuda.synchronize()
        assert int(flag2.item()) == 0
        _same_sets(out2.cpu().numpy(), want_other)
