"""Exact per-row top-k selection for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/ets_topk.h`` (library
``libets_topk.so``, built from ``csrc/ets_topk.hip``).  This module only
checks and marshals arguments: every step of the selection runs in the HIP
kernels.  PyTorch provides device memory and the current stream.

Entry points (same names as the C ABI without the ``ets_`` prefix):

* :func:`topk_raw`    -- dense rows, row-local positions;
* :func:`topk_paged`  -- dense rows, paged KV slots through a page table
  (argument order of the pages' fused transform: scores, seq_lens,
  page_table, output, page_size);
* :func:`topk_ragged` -- packed ragged rows, packed-buffer positions.

Each output row holds min(k, n) selected entries in unspecified order followed
by -1 padding.  Scores are ranked by their order-preserving 32-bit key; among
equal bit patterns the lowest positions win.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

__all__ = ["topk_raw", "topk_paged", "topk_ragged", "topk_paged_noalloc", "workspace_size", "row_split", "floor_read",
           "floor_launch", "device_limits", "group_cap", "ticket_cap",
           "new_workspace", "workspace_init", "workspace_error", "workspace_error_async",
           "library_path", "MAX_K", "NOALLOC_SCRATCH_BYTES", "ERROR_BITS", "EtsError"]

MAX_K = 2048
NOALLOC_SCRATCH_BYTES = 4 << 20  # ETS_NOALLOC_SCRATCH_BYTES: topk_paged_noalloc's static scratch
# bits of a workspace's error word (workspace_error): which wait ran out
ERROR_BITS = {1: "bounds exchange", 2: "stale ticket", 4: "coarse histogram", 8: "round barrier",
              16: "tie list"}
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libets_topk.so")
_lock = threading.Lock()
_lib = None


class EtsError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, _status_text(status), status))


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    "libets_topk.so is not built (expected at %s); run "
                    "`python -c 'import __graft_entry__ as g; g.build()'` first" % _LIB_PATH)
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            lib.ets_topk_raw.argtypes = [vp, i64, i32, i32, vp, i32, vp, i64, vp, sz, vp]
            lib.ets_topk_paged.argtypes = [vp, i64, i32, i32, vp, vp, i64, i32, i32, vp, i64,
                                           vp, sz, vp]
            lib.ets_topk_ragged.argtypes = [vp, vp, vp, i32, i64, i32, vp, i64, vp, sz, vp]
            lib.ets_topk_paged_noalloc.argtypes = [vp, i64, i32, i32, vp, vp, i64, i32, i32, vp,
                                                   i64, vp, vp]
            lib.ets_topk_paged_window.argtypes = [vp, i64, i32, i32, vp, vp, vp, i64, i32, i32, vp,
                                                  i64, vp, sz, vp]
            lib.ets_workspace_size.argtypes = [i32, i64, i32, i32, ctypes.POINTER(sz)]
            lib.ets_row_split.argtypes = [i32, i64, i32, i32, i32]
            lib.ets_workspace_init.argtypes = [vp, sz, vp]
            lib.ets_workspace_error.argtypes = [vp, sz, vp, vp]
            pi32 = ctypes.POINTER(i32)
            lib.ets_device_limits.argtypes = [i32, pi32, pi32, pi32]
            lib.ets_group_cap.argtypes = [i32, i32, i32]
            lib.ets_ticket_cap.argtypes = [i32, i32, i32]
            lib.ets_status_string.argtypes = [i32]
            lib.ets_floor_read.argtypes = [vp, i64, i32, i32, vp, vp, i64, vp, i64, vp]
            lib.ets_floor_launch.argtypes = [i32, i64, vp]
            for fn in (lib.ets_topk_raw, lib.ets_topk_paged, lib.ets_topk_ragged,
                       lib.ets_topk_paged_noalloc, lib.ets_topk_paged_window,
                       lib.ets_workspace_size, lib.ets_row_split, lib.ets_workspace_init,
                       lib.ets_workspace_error, lib.ets_device_limits, lib.ets_group_cap,
                       lib.ets_ticket_cap, lib.ets_floor_read, lib.ets_floor_launch):
                fn.restype = ctypes.c_int32
            lib.ets_status_string.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def _status_text(status: int) -> str:
    try:
        return _load().ets_status_string(status).decode()
    except Exception:  # pragma: no cover - library unavailable
        return "status %d" % status


def _check(status: int, what: str) -> None:
    if status != 0:
        raise EtsError(status, what)


# The per-call checks below use only cheap tensor attributes (a decode step
# makes tens of calls, and an eager call's host time is all overhead).

def _require(t: torch.Tensor, name: str, dtype: torch.dtype, dim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype is not dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.ndim != dim:
        raise ValueError("%s must be %d-D, got shape %s" % (name, dim, tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must be on a HIP device, got %s" % (name, t.device))


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a 2-D tensor whose rows are contiguous."""
    rows, cols = t.shape
    st0, st1 = t.stride()
    if cols > 1 and st1 != 1:
        raise ValueError("%s rows must be contiguous (stride(1) == 1)" % name)
    return st0 if rows > 1 else max(cols, 1)


def _vec(t: torch.Tensor, name: str, n: int) -> None:
    _require(t, name, torch.int32, 1)
    if t.shape[0] != n:
        raise ValueError("%s must have %d entries, got %d" % (name, n, t.shape[0]))
    if n > 1 and t.stride(0) != 1:
        raise ValueError("%s must be contiguous" % name)


def _same_device(index: int, *named) -> None:
    for t, nm in named:
        if t is not None and t.get_device() != index:
            raise ValueError("%s must be on cuda:%d" % (nm, index))


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    """Handle of torch's current stream on a device (index or torch.device)."""
    index = device if isinstance(device, int) else device.index
    if index is None:
        index = torch.cuda.current_device()
    if _raw_stream is not None:
        return _raw_stream(index)
    return torch.cuda.current_stream(index).cuda_stream


def _on(index: int, fn, *args):
    """fn(*args) with device `index` current (the C calls act on the current
    device); switches only when another device is current."""
    if torch.cuda.current_device() == index:
        return fn(*args)
    with torch.cuda.device(index):
        return fn(*args)


def workspace_size(B: int, max_row_len: int, k: int, device: Optional[int] = None) -> int:
    """Bytes of workspace a call with these sizes needs on the device (0 if none).

    A workspace must be zero before its first use (``new_workspace`` or
    ``workspace_init``); every call returns the counters and tables it relies
    on to zero.  Calls that pass no workspace share one buffer per device and
    stream."""
    nbytes = ctypes.c_size_t(0)
    _check(_load().ets_workspace_size(B, max_row_len, k, -1 if device is None else device,
                                      ctypes.byref(nbytes)), "ets_workspace_size")
    return nbytes.value


def row_split(B: int, max_row_len: int, cu_count: int, xcd_count: int, groups_per_cu: int) -> int:
    """Workgroups per row chosen for (B, max_row_len) on a device of ``cu_count``
    CUs in ``xcd_count`` XCDs, each CU holding ``groups_per_cu`` row-group
    workgroups (0 = one per row, -1 = an ETS_ROW_SPLIT override above
    group_cap, which the calls reject)."""
    return int(_load().ets_row_split(B, max_row_len, cu_count, xcd_count, groups_per_cu))


def group_cap(cu_count: int, xcd_count: int, groups_per_cu: int) -> int:
    """Largest row group for a device of these sizes (pure host function)."""
    return int(_load().ets_group_cap(cu_count, xcd_count, groups_per_cu))


def ticket_cap(cu_count: int, xcd_count: int, groups_per_cu: int) -> int:
    """Largest row group one launch of a grid that does not fit the device at
    once takes: one shader engine's row-group slots (pure host function)."""
    return int(_load().ets_ticket_cap(cu_count, xcd_count, groups_per_cu))


def device_limits(device: Optional[int] = None):
    """(compute units, XCDs, row-group workgroups per compute unit) of a device
    (default: current): the inputs of row_split, group_cap and ticket_cap."""
    cu, xcd, occ = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_load().ets_device_limits(-1 if device is None else int(device), ctypes.byref(cu),
                                     ctypes.byref(xcd), ctypes.byref(occ)), "ets_device_limits")
    return cu.value, xcd.value, occ.value


# Workspace word set non-zero by a call that stopped waiting for the other
# workgroups of a row (its results are then undefined).
WORKSPACE_ERROR_WORD = 32

# Workspaces kept per (device, stream) for calls that pass none: zero-filled
# once, then every call returns what it relies on to zero, so one buffer
# serves all later calls on that stream.
_ws_cache = {}


def new_workspace(B: int, max_row_len: int, k: int,
                  device: Optional[torch.device] = None) -> Optional[torch.Tensor]:
    """A zero-filled workspace for calls with these sizes (None if none is needed)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    with torch.cuda.device(device):
        need = workspace_size(B, max_row_len, k)
    if need == 0:
        return None
    return torch.zeros(need, dtype=torch.uint8, device=device)


def workspace_init(workspace: torch.Tensor) -> None:
    """Zero-fills ``workspace`` on the current stream (needed once before its first use)."""
    _require(workspace, "workspace", torch.uint8, 1)
    with torch.cuda.device(workspace.device):
        _check(_load().ets_workspace_init(workspace.data_ptr(), workspace.numel(),
                                          _stream(workspace.device)), "ets_workspace_init")


def workspace_error_async(workspace: Optional[torch.Tensor], flag: torch.Tensor) -> None:
    """Enqueues a copy of the workspace's error word into ``flag`` (int32 [>=1] on
    the same device) and clears the word, on the current stream, without
    synchronising.  ``workspace`` None (a call that needed none) writes 0."""
    _require(flag, "flag", torch.int32, 1)
    if flag.numel() < 1:
        raise ValueError("flag needs one element")
    dev = flag.device
    if workspace is not None:
        _require(workspace, "workspace", torch.uint8, 1)
        if workspace.device != dev:
            raise ValueError("flag must be on the workspace's device")
    with torch.cuda.device(dev):
        _check(_load().ets_workspace_error(
            workspace.data_ptr() if workspace is not None else None,
            workspace.numel() if workspace is not None else 0, flag.data_ptr(), _stream(dev)),
            "ets_workspace_error")


def workspace_error(workspace: Optional[torch.Tensor]) -> int:
    """The workspace's error word, cleared afterwards (synchronises).  Non-zero
    means a call stopped waiting for its row group and its output is undefined."""
    dev = workspace.device if workspace is not None else torch.device("cuda", torch.cuda.current_device())
    flag = torch.full((1,), -1, dtype=torch.int32, device=dev)
    workspace_error_async(workspace, flag)
    return int(flag.item())


ETS_ERR_WORKSPACE = 3


def _select(what: str, fn, args: tuple, index: int, B: int, max_len: int, k: int,
            workspace: Optional[torch.Tensor]) -> None:
    """Runs one selection call fn(*args, workspace, workspace_bytes, stream) on
    device `index`.  The library reports a missing or short workspace before
    enqueueing anything (ETS_ERR_WORKSPACE), so the common call makes one C
    call: with the caller's workspace, or with the one kept for this device
    and stream (created, or grown, only when a call asks for it)."""
    stream = _stream(index)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
            raise TypeError("workspace must be a torch.Tensor on a HIP device")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        _same_device(index, (workspace, "workspace"))
        nbytes = workspace.numel() * workspace.element_size()
        st = _on(index, fn, *args, workspace.data_ptr(), nbytes, stream)
        if st == ETS_ERR_WORKSPACE:
            need = _on(index, workspace_size, B, max_len, k)
            raise ValueError("workspace must hold at least %d bytes, 16-byte aligned (got %d)"
                             % (need, nbytes))
        _check(st, what)
        return
    # a captured graph keeps a buffer's address for its replays, and the
    # shared buffer may be replaced by a larger one later: none under capture
    capturing = torch.cuda.is_current_stream_capturing()
    key = (index, stream)
    ws = None if capturing else _ws_cache.get(key)
    st = _on(index, fn, *args, ws.data_ptr() if ws is not None else None,
             ws.numel() if ws is not None else 0, stream)
    if st == ETS_ERR_WORKSPACE:
        need = _on(index, workspace_size, B, max_len, k)
        if capturing:
            raise ValueError("a call that needs a workspace (%d bytes) must be given one "
                             "while a graph is being captured: pass workspace=new_workspace(...)"
                             % need)
        with _lock:
            ws = _ws_cache.get(key)
            if ws is None or ws.numel() < need:
                ws = torch.zeros(need, dtype=torch.uint8, device=torch.device("cuda", index))
                _ws_cache[key] = ws
        st = _on(index, fn, *args, ws.data_ptr(), ws.numel(), stream)
    _check(st, what)


def _out(out: Optional[torch.Tensor], B: int, k: int, index: int) -> torch.Tensor:
    if out is None:
        return torch.empty((B, k), dtype=torch.int32, device=torch.device("cuda", index))
    _require(out, "out", torch.int32, 2)
    rows, cols = out.shape
    if rows != B or cols < k or out.get_device() != index:
        raise ValueError("out must be int32 [B, >=k] on cuda:%d" % index)
    if k > 1 and out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    return out


def _out_stride(out: torch.Tensor, B: int, k: int) -> int:
    return out.stride(0) if B > 1 else k


def topk_raw(scores: torch.Tensor, k: int, lens: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact top-k positions of each row of fp32 ``scores`` [B, L]; int32 [B, k]."""
    _require(scores, "scores", torch.float32, 2)
    B, L = scores.shape
    index = scores.get_device()
    if lens is not None:
        _vec(lens, "lens", B)
        _same_device(index, (lens, "lens"))
    out = _out(out, B, k, index)
    args = (scores.data_ptr(), _rows(scores, "scores"), B, L,
            lens.data_ptr() if lens is not None else None, k, out.data_ptr(),
            _out_stride(out, B, k))
    _select("ets_topk_raw", _load().ets_topk_raw, args, index, B, L, k, workspace)
    return out


def topk_paged(scores: torch.Tensor, seq_lens: torch.Tensor, page_table: torch.Tensor,
               page_indices: torch.Tensor, page_size: int,
               workspace: Optional[torch.Tensor] = None,
               window_starts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fills ``page_indices`` int32 [B, k] with the paged slots of each row's top-k.

    Slot of position i of row b: page_table[b, i // page_size] * page_size +
    i % page_size.  ``k`` is ``page_indices.shape[1]``.  With ``window_starts``
    (int32 [B]) row b selects among positions [window_starts[b], seq_lens[b])
    only (ets_topk_paged_window).
    """
    index, B, L, k = _paged_checks(scores, seq_lens, page_table, page_indices, page_size)
    lib = _load()
    if window_starts is None:
        args = (scores.data_ptr(), _rows(scores, "scores"), B, L, seq_lens.data_ptr(),
                page_table.data_ptr(), _rows(page_table, "page_table"), page_size, k,
                page_indices.data_ptr(), _out_stride(page_indices, B, k))
        _select("ets_topk_paged", lib.ets_topk_paged, args, index, B, L, k, workspace)
    else:
        _vec(window_starts, "window_starts", B)
        _same_device(index, (window_starts, "window_starts"))
        args = (scores.data_ptr(), _rows(scores, "scores"), B, L, window_starts.data_ptr(),
                seq_lens.data_ptr(), page_table.data_ptr(), _rows(page_table, "page_table"),
                page_size, k, page_indices.data_ptr(), _out_stride(page_indices, B, k))
        _select("ets_topk_paged_window", lib.ets_topk_paged_window, args, index, B, L, k,
                workspace)
    return page_indices


def _paged_checks(scores, seq_lens, page_table, page_indices, page_size):
    """Checks shared by the paged calls; returns (device index, B, L, k)."""
    _require(scores, "scores", torch.float32, 2)
    B, L = scores.shape
    index = scores.get_device()
    _vec(seq_lens, "seq_lens", B)
    _require(page_table, "page_table", torch.int32, 2)
    pt_rows, pt_pages = page_table.shape
    if pt_rows != B:
        raise ValueError("page_table must have B rows")
    _require(page_indices, "page_indices", torch.int32, 2)
    k = page_indices.shape[1]
    _out(page_indices, B, k, index)
    _same_device(index, (seq_lens, "seq_lens"), (page_table, "page_table"))
    if page_size < 1:
        raise ValueError("page_size must be >= 1")
    if pt_pages * page_size < L:
        raise ValueError("page_table has %d pages of %d, fewer than L = %d positions"
                         % (pt_pages, page_size, L))
    return index, B, L, k


def topk_paged_noalloc(scores: torch.Tensor, seq_lens: torch.Tensor, page_table: torch.Tensor,
                       page_indices: torch.Tensor, page_size: int,
                       error_flag: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``topk_paged`` without a workspace: split rows use the library's static
    per-device scratch (4 MiB), so the call allocates nothing, here or in the
    library.  Calls that may overlap on one device race.  ``error_flag``
    (int32 [>=1], optional) receives the scratch's error word."""
    index, B, L, k = _paged_checks(scores, seq_lens, page_table, page_indices, page_size)
    if error_flag is not None:
        _require(error_flag, "error_flag", torch.int32, 1)
        if error_flag.get_device() != index or error_flag.numel() < 1:
            raise ValueError("error_flag must be int32 [>=1] on cuda:%d" % index)
    st = _on(index, _load().ets_topk_paged_noalloc, scores.data_ptr(), _rows(scores, "scores"),
             B, L, seq_lens.data_ptr(), page_table.data_ptr(), _rows(page_table, "page_table"),
             page_size, k, page_indices.data_ptr(), _out_stride(page_indices, B, k),
             error_flag.data_ptr() if error_flag is not None else None, _stream(index))
    _check(st, "ets_topk_paged_noalloc")
    return page_indices


def topk_ragged(packed: torch.Tensor, row_starts: torch.Tensor, lengths: torch.Tensor, k: int,
                max_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact top-k of packed ragged rows; int32 [B, k] of packed-buffer positions.

    ``max_len`` bounds every length; if omitted it is read from ``lengths``,
    which synchronises the stream.
    """
    _require(packed, "packed", torch.float32, 1)
    index = packed.get_device()
    _require(row_starts, "row_starts", torch.int32, 1)
    B = row_starts.shape[0]
    _vec(row_starts, "row_starts", B)
    _vec(lengths, "lengths", B)
    _same_device(index, (row_starts, "row_starts"), (lengths, "lengths"))
    if packed.numel() > 1 and packed.stride(0) != 1:
        raise ValueError("packed must be contiguous")
    if max_len is None:
        max_len = int(lengths.max().item()) if B else 0
    out = _out(out, B, k, index)
    args = (packed.data_ptr(), row_starts.data_ptr(), lengths.data_ptr(), B, max_len, k,
            out.data_ptr(), _out_stride(out, B, k))
    _select("ets_topk_ragged", _load().ets_topk_ragged, args, index, B, max_len, k, workspace)
    return out


def floor_read(scores: torch.Tensor, lens: Optional[torch.Tensor] = None,
               row_starts: Optional[torch.Tensor] = None, max_len: Optional[int] = None,
               sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Measurement floor: reads what a selection call on the same rows reads,
    with its grid and loads, and returns each workgroup's largest key
    (int32 view of uint32 words, one per workgroup).

    Dense: ``scores`` [B, L] with optional ``lens``.  Ragged: ``scores`` is the
    packed 1-D buffer, ``lens`` the lengths and ``row_starts`` the offsets;
    ``max_len`` bounds the lengths.
    """
    dev = scores.device
    if row_starts is None:
        _require(scores, "scores", torch.float32, 2)
        B, L = scores.shape
        stride = _rows(scores, "scores")
        if lens is not None:
            _vec(lens, "lens", B)
        max_len = L
    else:
        _require(scores, "scores", torch.float32, 1)
        B = row_starts.shape[0]
        _vec(row_starts, "row_starts", B)
        if lens is None:
            raise ValueError("ragged rows need lens")
        _vec(lens, "lens", B)
        if max_len is None:
            raise ValueError("ragged rows need max_len")
        L, stride = 0, 0
    with torch.cuda.device(dev):
        limits = device_limits()
    words = B * max(1, row_split(B, max_len, *limits))
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=dev)
    _require(sink, "sink", torch.int32, 1)
    with torch.cuda.device(dev):
        st = _load().ets_floor_read(scores.data_ptr(), stride, B, L,
                                    lens.data_ptr() if lens is not None else None,
                                    row_starts.data_ptr() if row_starts is not None else None,
                                    max_len, sink.data_ptr(), sink.numel(), _stream(dev))
    _check(st, "ets_floor_read")
    return sink[:words]


def floor_launch(B: int, max_row_len: int, device: Optional[torch.device] = None) -> None:
    """Measurement floor: one empty launch of a selection call's grid."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.device(dev):
        st = _load().ets_floor_launch(B, max_row_len, _stream(dev))
    _check(st, "ets_floor_launch")
