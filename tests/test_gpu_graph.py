"""The library's launches inside a captured HIP graph: every replay must select
the eager result's sets, with eager work and synchronisations between
replays, and leave its workspace ready for the next replay."""
import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import workloads
from tests.gpu_helpers import workspace_dirty

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    d = torch.device("cuda:0")
    w3 = workloads.make("C3", seed=50)
    w4 = workloads.make("C4", seed=51)
    s3 = torch.from_numpy(w3.scores).to(d)
    l3 = torch.from_numpy(w3.lens).to(d)
    p3 = torch.from_numpy(w3.page_table).to(d)
    s4 = torch.from_numpy(w4.scores).to(d)
    eager3 = torch.empty((w3.B, w3.k), dtype=torch.int32, device=d)
    eager4 = torch.empty((w4.B, w4.k), dtype=torch.int32, device=d)
    ets.topk_paged(s3, l3, p3, eager3, w3.page_size)
    ets.topk_raw(s4, w4.k, out=eager4)
    torch.cuda.synchronize()

    g3 = torch.full_like(eager3, -7)
    g4 = torch.full_like(eager4, -7)
    # zero-filled workspaces made before capture; each call leaves them zero
    ws3 = ets.new_workspace(w3.B, w3.L, w3.k, d)
    ws4 = ets.new_workspace(w4.B, w4.L, w4.k, d)
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            ets.topk_paged(s3, l3, p3, g3, w3.page_size, workspace=ws3)
            ets.topk_raw(s4, w4.k, out=g4, workspace=ws4)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        g3.fill_(-9)
        g4.fill_(-9)
        graph.replay()
        torch.cuda.synchronize()
        # split rows may place their chunks in another order: compare sets
        assert torch.equal(g3.sort(dim=1).values, eager3.sort(dim=1).values), \
            "paged replay %d differs" % rep
        assert torch.equal(g4.sort(dim=1).values, eager4.sort(dim=1).values), \
            "raw replay %d differs" % rep
        for ws in (ws3, ws4):
            if ws is not None:
                # error word, counters and histogram tables back at zero
                assert ets.workspace_error(ws) == 0
                assert workspace_dirty(ws) == 0
        # eager work between replays, on other data
        tmp = torch.empty_like(eager3)
        ets.topk_paged(s3.flip(1).contiguous(), l3, p3, tmp, w3.page_size)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(np.sort(g4.cpu().numpy(), axis=1),
                                  np.sort(eager4.cpu().numpy(), axis=1))
