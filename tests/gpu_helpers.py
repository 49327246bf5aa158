"""Shared helpers for the GPU parity tests: run a workload through the C ABI
(via the thin binding) and through the CPU oracle, and compare."""
from __future__ import annotations

import numpy as np
import torch

import exact_top_selection_amd as ets
import oracle
from tests.checkers import recall

POISON = 0x7EEEEEEE


def dev():
    return torch.device("cuda:0")


# Workspace layout of the row-group path (u32 words): a 64-word header, then
# per row a 192-word record (counters, then one u64 slot per member), three
# 4096-bin tables and a 4096-entry u64 tie list.
WS_HDR = 64
WS_ROW = 192 + 3 * 4096 + 2 * 4096
WS_KEPT_ZERO = WS_ROW  # record, member slots, tables and tie list: back at zero after every call


def workspace_dirty(ws: torch.Tensor) -> int:
    """Non-zero words of a workspace: header, records, tables and tie lists."""
    torch.cuda.synchronize()
    w = ws.view(torch.int32)
    B = (w.numel() - WS_HDR) // WS_ROW
    assert WS_HDR + B * WS_ROW == w.numel(), "not a row-group workspace"
    rows = w[WS_HDR:].view(B, WS_ROW)[:, :WS_KEPT_ZERO]
    return int(torch.count_nonzero(w[:WS_HDR]).item() + torch.count_nonzero(rows).item())


def run_gpu(w, out_fill: int = POISON, scores=None):
    """Run workload ``w`` on the GPU; returns the int32 [B, k] output (numpy)."""
    d = dev()
    s = torch.from_numpy(w.scores if scores is None else scores).to(d)
    out = torch.full((w.B, w.k), out_fill, dtype=torch.int32, device=d)
    if w.api == "raw":
        lens = None if w.lens is None else torch.from_numpy(w.lens).to(d)
        ets.topk_raw(s, w.k, lens, out=out)
    elif w.api == "paged":
        ets.topk_paged(s, torch.from_numpy(w.lens).to(d), torch.from_numpy(w.page_table).to(d),
                       out, w.page_size)
    else:
        ets.topk_ragged(s, torch.from_numpy(w.row_starts).to(d), torch.from_numpy(w.lengths).to(d),
                        w.k, max_len=w.max_len, out=out)
    torch.cuda.synchronize(d)
    return out.cpu().numpy()


def run_oracle(w, threads: int = 8):
    if w.api == "raw":
        return oracle.topk_raw(w.scores, w.k, w.lens, threads=threads)
    if w.api == "paged":
        return oracle.topk_paged(w.scores, w.lens, w.page_table, w.page_size, w.k, threads=threads)
    return oracle.topk_ragged(w.scores, w.row_starts, w.lengths, w.k, threads=threads)


def raw_positions(w, out_row: np.ndarray, b: int) -> np.ndarray:
    """Row-local positions of the valid entries of one output row."""
    v = out_row[out_row != -1].astype(np.int64)
    if w.api == "paged":
        ps = w.page_size
        inv = {int(pg): i for i, pg in enumerate(w.page_table[b])}
        return np.array([inv[int(x) // ps] * ps + int(x) % ps for x in v], dtype=np.int64)
    if w.api == "ragged":
        return v - int(w.row_starts[b])
    return v


def row_values(w, b: int) -> np.ndarray:
    n = int(w.row_lengths[b])
    if w.api == "ragged":
        s = int(w.row_starts[b])
        return w.scores[s:s + n]
    return w.scores[b, :n]


def assert_parity(w, got: np.ndarray, want: np.ndarray, check_values: bool = True) -> None:
    """Bit-exact sorted index sets per row (including the -1 count), and equal
    value multisets (by bit pattern) over the selected positions."""
    assert got.shape == want.shape
    gs = np.sort(got, axis=1)
    ws = np.sort(want, axis=1)
    bad = np.nonzero((gs != ws).any(axis=1))[0]
    if bad.size:
        b = int(bad[0])
        raise AssertionError(
            "%s: %d of %d rows differ; first row %d (n=%d) recall %.4f; got %s... want %s..."
            % (w.name, bad.size, w.B, b, int(w.row_lengths[b]), recall(got[b], want[b]),
               gs[b][:8].tolist(), ws[b][:8].tolist()))
    if check_values:
        for b in range(w.B):
            vals = row_values(w, b).view(np.uint32)
            pg = raw_positions(w, got[b], b)
            pw = raw_positions(w, want[b], b)
            np.testing.assert_array_equal(np.sort(vals[pg]), np.sort(vals[pw]))
