"""The dispatch that the row-group launch plan relies on, checked on the
device with a test-only probe kernel (tests/native/dispatch_probe.hip):

  * workgroup i of a launch runs on XCD i % X (the index grids place a row's
    members on one XCD by it);
  * each XCD deals its workgroups, in index order, to its shader engines in a
    fixed rotation, and waits for a slot on the engine whose turn it is (so a
    ticketed grid keeps G within one engine's row-group slots);
  * each engine has cu_count / X / 4 compute units, as ets_ticket_cap assumes.

Workgroups on engine 0 hold 200 us, the others 5 us, one workgroup per
compute unit; every hold is bounded by a clock and no workgroup waits for
another."""
import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
from tests import dispatch_probe

pytestmark = pytest.mark.gpu

ENGINES = 4  # per XCD on gfx950, the count ets_ticket_cap divides by


def test_dispatch_matches_the_launch_plans_premises():
    cu, nx, occ = ets.device_limits()
    lib = dispatch_probe.load()
    d = torch.device("cuda:0")
    n = 8 * cu  # eight workgroups per compute unit: each XCD deals 8 rounds to each engine
    rec = torch.zeros((n, 4), dtype=torch.int64, device=d)
    print("case dispatch probe, workgroups", n, flush=True)
    st = lib.ets_test_dispatch_probe(rec.data_ptr(), n, 20000, 500, torch.cuda.current_stream(d).cuda_stream)
    assert st == 0, "launch failed (%d)" % st
    torch.cuda.synchronize(d)
    r = rec.cpu().numpy().view(np.uint64)
    xcc = (r[:, 0] & 0xF).astype(np.int64)
    hw = r[:, 1]
    engine = ((hw >> np.uint64(13)) & np.uint64(3)).astype(np.int64)
    unit = ((hw >> np.uint64(8)) & np.uint64(0x1F)).astype(np.int64)  # SH_ID and CU_ID
    t0 = r[:, 2].astype(np.int64)
    start = t0 - t0.min()

    assert (xcc == np.arange(n) % nx).all(), "workgroup i does not run on XCD i % X"
    for x in range(nx):
        idx = np.arange(x, n, nx)  # XCD x's workgroups in dealing order
        seq = engine[idx]
        rot = seq[:ENGINES]
        assert sorted(rot.tolist()) == list(range(ENGINES)), (x, rot)
        assert (seq == np.tile(rot, len(seq) // ENGINES)).all(), "not a fixed rotation on XCD %d" % x
        for e in range(ENGINES):
            assert len(set(unit[idx][seq == e].tolist())) == cu // nx // ENGINES, (x, e)
        # in order: the other engines' last workgroups start only as engine 0's
        # last ones do, although theirs hold 5 us and engine 0's 200 us
        last = [start[idx][seq == e].max() for e in range(ENGINES)]
        assert min(last[1:]) >= 0.8 * last[0], (x, last)
    assert ets.ticket_cap(cu, nx, occ) == (cu // nx // ENGINES) * occ
