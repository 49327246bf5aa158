"""A host-only model of how the row-group kernel's workgroups reach the device,
to check the progress argument behind the library's caps on workgroups per row.

The model follows the dispatch measured on MI355X:
  * workgroup i is bound to XCD i % X;
  * each XCD deals its own workgroups in index order to its E shader engines
    in a fixed rotation, and waits, in order, for a free slot on the engine
    whose turn it is (the engine's compute units times the row-group
    workgroups one compute unit holds), even while other engines have free
    slots;
  * a dealt workgroup starts and, after a short delay that differs between
    workgroups, takes the next ticket (start order, ticketed grids; ticket // G
    is its row group), or, on grids that fit the device at once, its index
    names its row: the G workgroups of XCD x's s-th block of G are row
    x + X * (s // G) of the grid's rows, the grid padded to X * G * ceil(B / X)
    workgroups (padding finishes at once);
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
    row, as the kernel assigns them (rows counted from the grid's first)."""
    x, s = wg % n_xcd, wg // n_xcd
    return x + n_xcd * (s // G), s % G


def simulate(n_wg, G, n_xcd, slots, speed, ticket=True, work=(1.0, 1.0), rows=None,
             engines=4, jitter=None, delay=None):
    """Returns the number of workgroups that finished (n_wg = no stall).
    slots: row-group slots per XCD, split evenly over `engines`.
    ticket=False: grouped by index; with rows=B, one XCD per row on the
    padded grid n_wg = X * G * ceil(B / X), else row wg // G.  jitter scales
    each workgroup's work; delay is each workgroup's start-to-ticket time."""
    per_engine = slots // engines
    queues = [deque(range(x, n_wg, n_xcd)) for x in range(n_xcd)]
    free = [[per_engine] * engines for _ in range(n_xcd)]
    dealt = [0] * n_xcd
    engine_of = {}
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

    def scale(wg):
        return 1.0 if jitter is None else jitter[wg]

    def start_ready(now):
        for x in range(n_xcd):
            while queues[x]:
                e = dealt[x] % engines
                if free[x][e] == 0:
                    break  # in order: the engine whose turn it is has no slot
                wg = queues[x].popleft()
                dealt[x] += 1
                free[x][e] -= 1
                engine_of[wg] = e
                if ticket:
                    push(now + (0.0 if delay is None else delay[wg]), "ticket", wg)
                    continue
                if rows is not None:
                    b, _ = index_row(wg, G, n_xcd)
                    if b >= rows:  # padding: nothing to do
                        push(now, "done", wg)
                        continue
                    group_of[wg] = b
                else:
                    group_of[wg] = wg // G
                push(now + work[0] * speed[x] * scale(wg), "exchange", wg)

    start_ready(0.0)
    while events:
        now, _, kind, wg = heapq.heappop(events)
        if kind == "ticket":
            group_of[wg] = state["ticket"] // G
            state["ticket"] += 1
            push(now + work[0] * speed[wg % n_xcd] * scale(wg), "exchange", wg)
        elif kind == "exchange":
            g = group_of[wg]
            members = arrived.setdefault(g, [])
            members.append(wg)
            size = G if rows is not None and not ticket else min(G, n_wg - g * G)
            if len(members) == size:
                for m in members:
                    push(now + work[1] * speed[m % n_xcd] * scale(m), "done", m)
        else:
            free[wg % n_xcd][engine_of[wg]] += 1
            finished += 1
            start_ready(now)
    return finished


def _random_run(rng, n):
    speed = list(rng.uniform(0.5, 4.0, size=8))
    jitter = rng.uniform(0.3, 3.0, size=n)
    delay = rng.exponential(0.3, size=n)
    work = (float(rng.uniform(0.5, 2.0)), float(rng.uniform(0.5, 2.0)))
    return speed, jitter, delay, work


def test_model_reproduces_the_stall_beyond_one_xcd():
    """64 members per row on a 4096-workgroup grid (B = 64, G = 64) with one
    1024-lane workgroup per compute unit (32 slots per XCD): once only the
    slowest XCD is still starting workgroups, a new group can only gather
    members there and its 32 slots cannot hold 64 of them."""
    speed = [1.0] * 7 + [3.0]
    assert simulate(64 * 64, 64, 8, 32, speed) < 64 * 64


@pytest.mark.parametrize("seed", [12, 17, 25])
def test_model_reproduces_the_stall_beyond_one_engine(seed):
    """32 members per row on a ticketed grid of 2048 workgroups: tickets
    follow start order, which differs from the dealing order, so the newest
    group's waiting members can fill the engine whose turn it is on the last
    XCD still dealing (8 slots), and the XCD waits for them while they wait
    for members queued behind them.  These seeds stall in the model; on the
    GPU such grids ran into the bounded wait of the bounds exchange twice in
    about 100,000 random calls."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = 64 * 32
    speed, jitter, delay, work = _random_run(rng, n)
    assert simulate(n, 32, 8, 32, speed, work=work, jitter=jitter, delay=delay) < n


@pytest.mark.parametrize("seed", range(4))
def test_model_progress_for_every_ticketed_group_within_one_engine(seed):
    """Every G up to one engine's slots finishes on ticketed grids of the
    sizes the heuristic produces, whatever the XCDs' speeds and the order in
    which started workgroups take tickets: at most G - 1 members wait, so the
    engine whose turn it is always holds a slot that frees up."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for slots in (32, 64):
        for G in (2, 3, 5, slots // 4):
            for B in (1, 5, 64, 130, 255):
                n = B * G
                speed, jitter, delay, work = _random_run(rng, n)
                assert simulate(n, G, 8, slots, speed, work=work, jitter=jitter,
                                delay=delay) == n, (slots, G, B)


def test_model_index_groups_when_the_grid_fits():
    """Groups by index need the whole grid resident at once: a grid within the
    device's slots always finishes (no engine is dealt more than it holds),
    and one beyond them can stall."""
    speed = [1.0] * 7 + [3.0]
    assert simulate(4 * 14, 14, 8, 32, speed, ticket=False) == 56
    assert simulate(8 * 32, 32, 8, 32, speed, ticket=False) == 256
    # groups by index on a grid beyond the slots: a row whose members need more
    # slots of one XCD than it has waits for members queued behind itself
    assert simulate(16 * 40, 40, 8, 4, speed, ticket=False, engines=1) < 16 * 40


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


def row_blocks(B, G, n_xcd, slots_per_xcd):
    """The launches of a batch whose G is above one engine's slots and whose
    padded grid does not fit the device: (first row, rows) of each index grid,
    as many whole rows per XCD as fit (the library's launch plan)."""
    rows = n_xcd * max(1, slots_per_xcd // G)
    return [(b0, min(rows, B - b0)) for b0 in range(0, B, rows)]


def test_model_row_blocks_each_fit_and_finish():
    """Each launch of the plan is an index grid within the device's slots, the
    launches cover every row once, and each finishes whatever the speeds."""
    rng = np.random.Generator(np.random.PCG64(4))
    for G in (9, 12, 16, 17, 31, 32):
        for B in (17, 33, 64, 134, 255):
            blocks = row_blocks(B, G, 8, 32)
            assert sum(r for _, r in blocks) == B
            assert [b0 for b0, _ in blocks] == list(range(0, B, blocks[0][1]))
            for _, r in blocks:
                grid = 8 * G * -(-r // 8)
                assert grid <= 8 * 32, (G, B, r)
                speed = list(rng.uniform(0.5, 4.0, size=8))
                assert simulate(grid, G, 8, 32, speed, ticket=False, rows=r) == grid, (G, B, r)
