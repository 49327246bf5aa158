"""The library's launches inside a captured HIP graph: every replay must equal
the eager result, with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import workloads

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
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            ets.topk_paged(s3, l3, p3, g3, w3.page_size)
            ets.topk_raw(s4, w4.k, out=g4)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        g3.fill_(-9)
        g4.fill_(-9)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g3, eager3), "paged replay %d differs" % rep
        assert torch.equal(g4, eager4), "raw replay %d differs" % rep
        # eager work between replays, on other data
        tmp = torch.empty_like(eager3)
        ets.topk_paged(s3.flip(1).contiguous(), l3, p3, tmp, w3.page_size)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(g4.cpu().numpy(), eager4.cpu().numpy())
