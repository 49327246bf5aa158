"""A host-only model of how the row-group kernel's workgroups reach the device,
to check the progress argument behind the library's cap on workgroups per row.

The model follows the hardware behaviour the kernel relies on:
  * workgroup i is bound to XCD i % X; each XCD starts its own workgroups in
    index order whenever one of its S slots (compute units times row-group
    workgroups per compute unit) is free;
  * a started workgroup takes the next ticket (start order, ticketed grids;
    ticket // G is its row group), or, on grids that fit the device at once,
    its index names its row: the G workgroups of XCD x's s-th block of G are
    row x + X * (s // G), the grid padded to X * G * ceil(B / X) workgroups
    (padding finishes at once);
  * a member works, then waits until every member of its group has reached
    the exchange, works again and frees its slot.
XCDs run at different speeds, so near the end of a grid the slower XCDs are
the only ones still starting workgroups.  A run stalls when nothing is left
to happen but workgroups are still queued or waiting.
"""
import heapq
from collections import deque

import numpy as np
import pytest


def index_row(wg, G, n_xcd):
    """(row, member) of workgroup wg on a grid grouped by index, one XCD per
    row, as the kernel assigns them."""
    x, s = wg % n_xcd, wg // n_xcd
    return x + n_xcd * (s // G), s % G


def simulate(n_wg, G, n_xcd, slots, speed, ticket=True, work=(1.0, 1.0), rows=None):
    """Returns the number of workgroups that finished (n_wg = no stall).
    ticket=False: grouped by index; with rows=B, one XCD per row on the
    padded grid n_wg = X * G * ceil(B / X), else row wg // G."""
    queues = [deque(range(x, n_wg, n_xcd)) for x in range(n_xcd)]
    free = [slots] * n_xcd
    events = []
    seq = 0
    state = {"ticket": 0}
    group_of = {}
    arrived = {}
    finished = 0

    def push(t, kind, wg):
        nonlocal seq
        heapq.heappush(events, (t, seq, kind, wg))
        seq += 1

    def start_ready(now):
        for x in range(n_xcd):
            while free[x] > 0 and queues[x]:
                wg = queues[x].popleft()
                free[x] -= 1
                if ticket:
                    tk = state["ticket"]
                    state["ticket"] += 1
                    group_of[wg] = tk // G
                elif rows is not None:
                    b, _ = index_row(wg, G, n_xcd)
                    if b >= rows:  # padding: nothing to do
                        push(now, "done", wg)
                        continue
                    group_of[wg] = b
                else:
                    group_of[wg] = wg // G
                push(now + work[0] * speed[x], "exchange", wg)

    start_ready(0.0)
    while events:
        now, _, kind, wg = heapq.heappop(events)
        if kind == "exchange":
            g = group_of[wg]
            members = arrived.setdefault(g, [])
            members.append(wg)
            size = G if rows is not None and not ticket else min(G, n_wg - g * G)
            if len(members) == size:
                for m in members:
                    push(now + work[1] * speed[m % n_xcd], "done", m)
        else:
            free[wg % n_xcd] += 1
            finished += 1
            start_ready(now)
    return finished


def test_model_reproduces_the_stall_beyond_one_xcd():
    """64 members per row on a 4096-workgroup grid (B = 64, G = 64) with one
    1024-lane workgroup per compute unit (32 slots per XCD): once only the
    slowest XCD is still starting workgroups, a new group can only gather
    members there and its 32 slots cannot hold 64 of them."""
    speed = [1.0] * 7 + [3.0]
    done = simulate(64 * 64, 64, 8, 32, speed)
    assert done < 64 * 64
    # the same grid with members per row within one XCD's slots finishes
    assert simulate(128 * 32, 32, 8, 32, speed) == 128 * 32


@pytest.mark.parametrize("seed", range(4))
def test_model_progress_for_every_group_within_the_cap(seed):
    """Every G up to one XCD's slots finishes on ticketed grids of the sizes
    the heuristic produces, whatever the XCDs' relative speeds."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for slots in (32, 38):
        for G in (2, 3, 8, 17, slots):
            for B in (1, 5, 64, 130, 255):
                speed = list(rng.uniform(0.5, 4.0, size=8))
                n = B * G
                work = (float(rng.uniform(0.5, 2.0)), float(rng.uniform(0.5, 2.0)))
                assert simulate(n, G, 8, slots, speed, ticket=True, work=work) == n, (slots, G, B)


def test_model_index_groups_when_the_grid_fits():
    """Groups by index need the whole grid resident at once: a grid within the
    device's slots always finishes, and one beyond them can stall."""
    speed = [1.0] * 7 + [3.0]
    assert simulate(4 * 14, 14, 8, 32, speed, ticket=False) == 56
    assert simulate(8 * 32, 32, 8, 32, speed, ticket=False) == 256
    # groups by index on a grid beyond the slots: a row whose members need more
    # slots of one XCD than it has waits for members queued behind itself
    assert simulate(16 * 40, 40, 8, 4, speed, ticket=False) < 16 * 40


def test_index_rows_one_xcd_each():
    """The padded index grid gives every member of every row exactly one
    workgroup, all of a row's members on one XCD (workgroup i on XCD i % X),
    and only padding beyond the last row."""
    for n_xcd in (1, 8):
        for B in (1, 3, 4, 8, 9, 16):
            for G in (2, 14, 16, 32):
                grid = n_xcd * G * -(-B // n_xcd)
                seen = {}
                for wg in range(grid):
                    b, g = index_row(wg, G, n_xcd)
                    if b >= B:
                        continue
                    assert (b, g) not in seen
                    seen[(b, g)] = wg % n_xcd
                assert len(seen) == B * G
                for b in range(B):
                    assert {seen[(b, g)] for g in range(G)} == {b % n_xcd}


def test_model_index_rows_per_xcd_when_the_padded_grid_fits():
    """One XCD per row: a padded grid within the device's slots finishes
    whatever the XCDs' speeds, also where B is not a multiple of the XCDs."""
    rng = np.random.Generator(np.random.PCG64(9))
    for B, G in ((4, 14), (16, 16), (3, 32), (9, 8), (1, 16)):
        grid = 8 * G * -(-B // 8)
        assert grid <= 8 * 32
        speed = list(rng.uniform(0.5, 4.0, size=8))
        assert simulate(grid, G, 8, 32, speed, ticket=False, rows=B) == grid, (B, G)
