"""The library's launches inside a captured HIP graph: every replay must select
the oracle's sets, with eager work and synchronisations between replays, and
leave its workspace ready for the next replay.  One of the captured calls
splits its rows over row groups (a caller workspace)."""
import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import workloads
from tests.gpu_helpers import assert_parity, run_oracle, workspace_dirty

pytestmark = pytest.mark.gpu


def test_graph_replays_match_the_oracle():
    d = torch.device("cuda:0")
    w3 = workloads.make("C3", seed=50)
    w4 = workloads.make("C4", seed=51)
    w5 = workloads.make("C5", seed=52)
    s3 = torch.from_numpy(w3.scores).to(d)
    l3 = torch.from_numpy(w3.lens).to(d)
    p3 = torch.from_numpy(w3.page_table).to(d)
    s4 = torch.from_numpy(w4.scores).to(d)
    s5 = torch.from_numpy(w5.scores).to(d)
    st5 = torch.from_numpy(w5.row_starts).to(d)
    ln5 = torch.from_numpy(w5.lengths).to(d)
    want3, want4, want5 = run_oracle(w3), run_oracle(w4), run_oracle(w5)

    g3 = torch.full((w3.B, w3.k), -7, dtype=torch.int32, device=d)
    g4 = torch.full((w4.B, w4.k), -7, dtype=torch.int32, device=d)
    g5 = torch.full((w5.B, w5.k), -7, dtype=torch.int32, device=d)
    # zero-filled workspaces made before capture; each call leaves them zero
    ws3 = ets.new_workspace(w3.B, w3.L, w3.k, d)
    ws4 = ets.new_workspace(w4.B, w4.L, w4.k, d)
    ws5 = ets.new_workspace(w5.B, w5.max_len, w5.k, d)
    assert ws5 is not None, "C5 runs on row groups"
    flag = torch.zeros(1, dtype=torch.int32, device=d)
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            ets.topk_paged(s3, l3, p3, g3, w3.page_size, workspace=ws3)
            ets.topk_raw(s4, w4.k, out=g4, workspace=ws4)
            ets.topk_ragged(s5, st5, ln5, w5.k, max_len=w5.max_len, out=g5, workspace=ws5)
            ets.workspace_error_async(ws5, flag)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        g3.fill_(-9)
        g4.fill_(-9)
        g5.fill_(-9)
        flag.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        print("replay", rep, flush=True)
        assert flag.item() == 0, "replay %d: a row group stopped waiting" % rep
        assert_parity(w3, g3.cpu().numpy(), want3)
        assert_parity(w4, g4.cpu().numpy(), want4)
        assert_parity(w5, g5.cpu().numpy(), want5)
        for ws in (ws3, ws4, ws5):
            if ws is not None:
                # counters and histogram tables back at zero
                assert workspace_dirty(ws) == 0
        # eager work between replays, on other data
        tmp = torch.empty_like(g3)
        ets.topk_paged(s3.flip(1).contiguous(), l3, p3, tmp, w3.page_size)
        tmp5 = ets.topk_ragged(s5.flip(0).contiguous(), st5, ln5, w5.k, max_len=w5.max_len,
                               workspace=ws5)
        torch.cuda.synchronize()
        del tmp, tmp5


def test_graph_replays_of_batches_beyond_the_device():
    """Inside one captured graph: a batch whose grid exceeds the device with G
    above one shader engine's slots (B = 40, G = 16: three index grids of 16,
    16 and 8 rows) and a ticketed batch (B = 96, L = 131072: the default G =
    4, a grid of 384 workgroups).  Every replay matches the oracle, with the
    error word zero and both workspaces clean."""
    import os
    from workloads import Workload
    d = torch.device("cuda:0")
    rng = np.random.Generator(np.random.PCG64(60))
    w1 = Workload("graph-grids", "raw", 1024, 40, workloads.normal_dense(rng, 40, 100000), L=100000)
    w2 = Workload("graph-ticket", "raw", 2048, 96, workloads.normal_dense(rng, 96, 131072), L=131072)
    cu, nx, occ = ets.device_limits()
    g2 = ets.row_split(w2.B, w2.L, cu, nx, occ)
    # a ticketed grid: beyond the device's slots, G within one engine's
    assert 2 <= g2 <= ets.ticket_cap(cu, nx, occ) and nx * g2 * -(-w2.B // nx) > cu * occ
    s1, s2 = torch.from_numpy(w1.scores).to(d), torch.from_numpy(w2.scores).to(d)
    want1, want2 = run_oracle(w1), run_oracle(w2)
    g1 = torch.full((w1.B, w1.k), -7, dtype=torch.int32, device=d)
    g2 = torch.full((w2.B, w2.k), -7, dtype=torch.int32, device=d)
    saved = os.environ.pop("ETS_ROW_SPLIT", None)
    try:
        os.environ["ETS_ROW_SPLIT"] = "16"
        ws1 = ets.new_workspace(w1.B, w1.L, w1.k, d)
        os.environ.pop("ETS_ROW_SPLIT")
        ws2 = ets.new_workspace(w2.B, w2.L, w2.k, d)
        assert ws1 is not None and ws2 is not None
        f1 = torch.zeros(1, dtype=torch.int32, device=d)
        f2 = torch.zeros(1, dtype=torch.int32, device=d)
        graph = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                os.environ["ETS_ROW_SPLIT"] = "16"
                ets.topk_raw(s1, w1.k, out=g1, workspace=ws1)
                os.environ.pop("ETS_ROW_SPLIT")
                ets.topk_raw(s2, w2.k, out=g2, workspace=ws2)
                ets.workspace_error_async(ws1, f1)
                ets.workspace_error_async(ws2, f2)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("ETS_ROW_SPLIT", None)
        if saved is not None:
            os.environ["ETS_ROW_SPLIT"] = saved
    for rep in range(3):
        g1.fill_(-9)
        g2.fill_(-9)
        f1.fill_(-1)
        f2.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        print("replay", rep, flush=True)
        assert f1.item() == 0 and f2.item() == 0, "replay %d: a row group stopped waiting" % rep
        assert_parity(w1, g1.cpu().numpy(), want1)
        assert_parity(w2, g2.cpu().numpy(), want2)
        assert workspace_dirty(ws1) == 0 and workspace_dirty(ws2) == 0
        # eager work between replays, on other data
        tmp = ets.topk_raw(s2.flip(1).contiguous(), w2.k, workspace=ws2)
        torch.cuda.synchronize()
        del tmp


def test_capture_refuses_an_implicit_workspace():
    """A call that needs a workspace must be given one while a graph is being
    captured: the shared implicit buffer may be replaced (and freed) later."""
    d = torch.device("cuda:0")
    w5 = workloads.make("C5", seed=53)
    s5 = torch.from_numpy(w5.scores).to(d)
    st5 = torch.from_numpy(w5.row_starts).to(d)
    ln5 = torch.from_numpy(w5.lengths).to(d)
    out = torch.empty((w5.B, w5.k), dtype=torch.int32, device=d)
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    raised = False
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            try:
                ets.topk_ragged(s5, st5, ln5, w5.k, max_len=w5.max_len, out=out)
            except ValueError:
                raised = True
    torch.cuda.synchronize()
    assert raised
