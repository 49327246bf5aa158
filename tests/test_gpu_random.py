"""Randomised GPU parity: every entry point (the allocation-free paged call
included) on seeded random shapes, lengths, value distributions, page sizes,
windows and forced row splits, each compared with the oracle (bit-exact
sorted index sets and equal value multisets).

random_case(seed) draws one valid call from its seed alone, so a failing case
is named by its seed.  The cases cover what the method has to handle exactly
(PR #37591 digest, Implementation breakdown: exact results for every
distribution, including clustered scores; its tests: variable windows and all
three entry points)."""
import contextlib
import os

import numpy as np
import pytest
import torch

import exact_top_selection_amd as ets
import oracle
import workloads
from workloads import Workload
from tests.gpu_helpers import POISON, assert_parity, dev

pytestmark = pytest.mark.gpu

_SPECIAL_BITS = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F800000, 0xFF800000,
                          0x7FC00000, 0xFFFFFFFF, 0x3F800000, 0xBF800000], dtype=np.uint32)


def _values(rng, n, dist):
    if dist == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if dist == "banded":
        return (rng.standard_normal(n) * 1e-3 + float(rng.integers(1, 5))).astype(np.float32)
    if dist == "few":
        m = int(rng.integers(1, 20))
        pool = rng.standard_normal(m).astype(np.float32)
        return pool[rng.integers(0, m, size=n)]
    if dist == "equal":
        return np.full(n, 1.0, dtype=np.float32)
    if dist == "special":
        bits = _SPECIAL_BITS[rng.integers(0, _SPECIAL_BITS.size, size=n)]
        mix = rng.random(n) < 0.5
        bits[mix] = rng.standard_normal(int(mix.sum())).astype(np.float32).view(np.uint32)
        return bits.view(np.float32)
    if dist == "subnormal":
        bits = rng.integers(1, 1 << 23, size=n, dtype=np.uint32) | (
            rng.integers(0, 2, size=n, dtype=np.uint32) << 31)
        return bits.astype(np.uint32).view(np.float32)
    # concentrated: most scores in a few adjacent values of one coarse bucket
    return workloads.concentrated_row(rng, n) if n >= 64 else rng.standard_normal(n).astype(np.float32)


def _lengths(rng, B, L, k):
    kind = rng.integers(0, 4)
    if kind == 0:
        return np.full(B, L, dtype=np.int32)
    if kind == 1:
        return rng.integers(0, L + 1, size=B).astype(np.int32)
    if kind == 2:
        return np.clip(rng.integers(k - 2, k + 3, size=B), 0, None).astype(np.int32)
    out = rng.integers(-5, L + 6, size=B).astype(np.int32)  # clamped to [0, L]
    return out


def random_case(seed):
    """(workload, env overrides, window starts or None) for one seed."""
    rng = np.random.Generator(np.random.PCG64(seed))
    api = ["raw", "paged", "ragged", "window"][int(rng.integers(0, 4))]
    B = int(np.exp(rng.uniform(0, np.log(300))))
    L = int(np.exp(rng.uniform(0, np.log(300000))))
    while B * L > 8_000_000:
        L //= 2
    L = max(L, 1)
    k = int(min(2048, max(1, np.exp(rng.uniform(0, np.log(2048))))))
    dist = ["normal", "banded", "few", "equal", "special", "subnormal", "concentrated"][
        int(rng.integers(0, 7))]
    env = {}
    r = rng.random()
    if r < 0.3:
        env["ETS_ROW_SPLIT"] = str(int(rng.integers(2, 33)))
    if rng.random() < 0.25:
        env["ETS_MIN_CHUNK"] = str(int(rng.choice([4, 100, 1000, 4096, 20000])))
    name = "seed%d-%s-B%d-L%d-k%d-%s" % (seed, api, B, L, k, dist)
    if api == "ragged":
        lengths = rng.integers(0, L + 1, size=B).astype(np.int32)
        if rng.random() < 0.2:
            lengths[int(rng.integers(0, B))] = -3
        gaps = rng.integers(0, 8, size=B)
        starts = np.zeros(B, dtype=np.int64)
        pos = 0
        for b in range(B):
            pos += int(gaps[b])
            starts[b] = pos
            pos += max(int(lengths[b]), 0)
        packed = _values(rng, pos + 1, dist)
        w = Workload(name, "ragged", k, B, packed, row_starts=starts.astype(np.int32),
                     lengths=lengths)
        return w, env, None
    x = np.stack([_values(rng, L, dist) for _ in range(B)]) if B * L else np.zeros((B, L), np.float32)
    lens = _lengths(rng, B, L, k)
    if api == "raw":
        return Workload(name, "raw", k, B, x, L=L, lens=lens), env, None
    ps = int(rng.choice([1, 3, 16, 64, 100, 128]))
    P = -(-L // ps)
    pt = np.stack([rng.permutation(P) + int(rng.integers(0, 1000)) for _ in range(B)]).astype(np.int32)
    w = Workload(name, "paged", k, B, x, L=L, lens=lens, page_table=pt, page_size=ps)
    wins = rng.integers(-5, L + 6, size=B).astype(np.int32) if api == "window" else None
    if wins is None and rng.random() < 0.3:
        w.extra["noalloc"] = True  # through ets_topk_paged_noalloc
    return w, env, wins


@contextlib.contextmanager
def _env(env):
    saved = {v: os.environ.get(v) for v in ("ETS_ROW_SPLIT", "ETS_MIN_CHUNK")}
    for v in saved:
        os.environ.pop(v, None)
    os.environ.update(env)
    try:
        yield
    finally:
        for v, old in saved.items():
            if old is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = old


def _oracle(w, wins):
    if w.api == "raw":
        return oracle.topk_raw(w.scores, w.k, w.lens, threads=8)
    if w.api == "ragged":
        return oracle.topk_ragged(w.scores, w.row_starts, w.lengths, w.k, threads=8)
    if wins is None:
        return oracle.topk_paged(w.scores, w.lens, w.page_table, w.page_size, w.k, threads=8)
    # a window [w_b, n_b) is the ragged call over the rows' flat buffer, the
    # positions shifted back to row positions and mapped through the table
    B, L = w.scores.shape
    n = np.clip(w.lens.astype(np.int64), 0, L)
    lo = np.clip(wins.astype(np.int64), 0, n)
    starts = (np.arange(B) * L + lo).astype(np.int32)
    flat = oracle.topk_ragged(np.ascontiguousarray(w.scores.reshape(-1)), starts,
                              (n - lo).astype(np.int32), w.k, threads=8)
    out = np.full((B, w.k), -1, np.int32)
    ps = w.page_size
    for b in range(B):
        v = flat[b][flat[b] != -1].astype(np.int64) - b * L
        out[b, :v.size] = w.page_table[b, v // ps] * ps + v % ps
    return out


def run_case(seed):
    """Runs one random case on the GPU and checks it against the oracle."""
    w, env, wins = random_case(seed)
    cap = ets.group_cap(*ets.device_limits())
    if "ETS_ROW_SPLIT" in env and int(env["ETS_ROW_SPLIT"]) > cap:
        env["ETS_ROW_SPLIT"] = str(cap)
    print("case", w.name, env, "noalloc" if w.extra.get("noalloc") else "", flush=True)
    d = dev()
    out = torch.full((w.B, w.k), POISON, dtype=torch.int32, device=d)
    s = torch.from_numpy(w.scores).to(d)
    with _env(env):
        if w.api == "raw":
            ets.topk_raw(s, w.k, torch.from_numpy(w.lens).to(d), out=out)
        elif w.api == "ragged":
            ets.topk_ragged(s, torch.from_numpy(w.row_starts).to(d),
                            torch.from_numpy(w.lengths).to(d), w.k, max_len=max(w.max_len, 0),
                            out=out)
        elif w.extra.get("noalloc"):
            flag = torch.full((1,), -1, dtype=torch.int32, device=d)
            try:
                ets.topk_paged_noalloc(s, torch.from_numpy(w.lens).to(d),
                                       torch.from_numpy(w.page_table).to(d), out, w.page_size,
                                       error_flag=flag)
            except ets.EtsError as e:
                # only a split call whose workspace exceeds the static scratch
                need = ets.workspace_size(w.B, w.L, w.k)
                assert e.status == 6 and need > ets.NOALLOC_SCRATCH_BYTES, (e.status, need)
                return
            torch.cuda.synchronize(d)
            e = int(flag.item())
            assert e == 0, "a row group stopped waiting (error word %d)" % e
        else:
            ets.topk_paged(s, torch.from_numpy(w.lens).to(d), torch.from_numpy(w.page_table).to(d),
                           out, w.page_size,
                           window_starts=None if wins is None else torch.from_numpy(wins).to(d))
        torch.cuda.synchronize(d)
    for ws in ets._ws_cache.values():
        e = ets.workspace_error(ws)
        assert e == 0, "a row group stopped waiting (error word %d)" % e
    got = out.cpu().numpy()
    want = _oracle(w, wins)
    if wins is None:
        assert_parity(w, got, want)
    else:
        np.testing.assert_array_equal(np.sort(got, axis=1), np.sort(want, axis=1))


@pytest.mark.parametrize("seed", range(40))
def test_random_case(seed):
    run_case(10_000 + seed)
