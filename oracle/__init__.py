"""CPU oracle for exact per-row top-k selection (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The HIP library never links, loads
or calls it, and the two share no code.

The arithmetic lives in ``ets_oracle.c`` (plain C, full sort of each row on
the order-preserving key, ties to the lowest position); this module only
compiles it with gcc and marshals numpy arrays through ctypes.  Every function
cites the passage it follows in the C source:

* sglang PR #37591 digest, "Summary" (the DSA-indexer top-k is exact) and the
  ``order_key32`` excerpt (the order-preserving 32-bit key);
* sglang PR #36004 digest, "Implementation breakdown" item 4 and its test
  excerpt (paged slots through a page table, -1 pre-fill of the output);
* PR #37591 digest, the ``CoopParams`` excerpt (row_starts / lengths of packed
  ragged rows, the raw / paged / ragged output map).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ets_oracle.c")
_LIB = os.path.join(_HERE, "libets_oracle.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile ``ets_oracle.c`` into ``libets_oracle.so`` with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
               "-pthread", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i32p = ctypes.POINTER(ctypes.c_int32)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.ets_oracle_order_key.argtypes = [ctypes.c_uint32]
    lib.ets_oracle_order_key.restype = ctypes.c_uint32
    lib.ets_oracle_topk_raw.argtypes = [
        u32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i32p,
        ctypes.c_int32, i32p, ctypes.c_int64, ctypes.c_int]
    lib.ets_oracle_topk_raw.restype = ctypes.c_int
    lib.ets_oracle_topk_paged.argtypes = [
        u32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i32p, i32p,
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i32p, ctypes.c_int64,
        ctypes.c_int]
    lib.ets_oracle_topk_paged.restype = ctypes.c_int
    lib.ets_oracle_topk_ragged.argtypes = [
        u32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32, i32p, ctypes.c_int64,
        ctypes.c_int]
    lib.ets_oracle_topk_ragged.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            _lib = _bind(_LIB)
    return _lib


def _bits(a) -> np.ndarray:
    """fp32 array (or its raw uint32 bit patterns) as a C-contiguous uint32 view."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.uint32:
        return a
    raise TypeError("scores must be float32 (or their uint32 bit patterns)")


def _i32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


def _p32(a: np.ndarray, t=ctypes.c_int32):
    return a.ctypes.data_as(ctypes.POINTER(t))


def order_key(bits: int) -> int:
    """Order-preserving key of one fp32 bit pattern (ets_oracle.c, step 1)."""
    return int(_load().ets_oracle_order_key(ctypes.c_uint32(bits & 0xFFFFFFFF)))


def topk_raw(scores, k: int, lens=None, threads: int = 1) -> np.ndarray:
    """Exact top-k positions of each dense row; int32 [B, k], -1 padded.

    ``scores`` is float32 [B, L]; ``lens`` (int32 [B] or None for all L) is the
    valid prefix length of each row, clamped to [0, L].
    """
    s = _bits(scores)
    if s.ndim != 2:
        raise ValueError("scores must be 2-D [B, L]")
    B, L = s.shape
    out = np.empty((B, k), dtype=np.int32)
    lp = None
    if lens is not None:
        lens = _i32(lens)
        if lens.shape != (B,):
            raise ValueError("lens must be int32 [B]")
        lp = _p32(lens)
    rc = _load().ets_oracle_topk_raw(_p32(s, ctypes.c_uint32), L, B, L, lp, k,
                                     _p32(out), k, threads)
    if rc != 0:
        raise RuntimeError("oracle failed (code %d)" % rc)
    return out


def topk_paged(scores, seq_lens, page_table, page_size: int, k: int,
               threads: int = 1) -> np.ndarray:
    """Exact top-k of each dense row mapped to paged KV slots; int32 [B, k]."""
    s = _bits(scores)
    B, L = s.shape
    seq_lens = _i32(seq_lens)
    pt = _i32(page_table)
    if seq_lens.shape != (B,) or pt.ndim != 2 or pt.shape[0] != B:
        raise ValueError("seq_lens must be [B] and page_table [B, P]")
    if pt.shape[1] * page_size < min(L, int(seq_lens.max(initial=0))):
        raise ValueError("page_table too narrow for the row lengths")
    out = np.empty((B, k), dtype=np.int32)
    rc = _load().ets_oracle_topk_paged(_p32(s, ctypes.c_uint32), L, B, L, _p32(seq_lens),
                                       _p32(pt), pt.shape[1], page_size, k, _p32(out), k,
                                       threads)
    if rc != 0:
        raise RuntimeError("oracle failed (code %d)" % rc)
    return out


def topk_ragged(packed, row_starts, lengths, k: int, threads: int = 1) -> np.ndarray:
    """Exact top-k of packed ragged rows as packed-buffer positions; int32 [B, k]."""
    s = _bits(packed)
    if s.ndim != 1:
        raise ValueError("packed scores must be 1-D")
    row_starts = _i32(row_starts)
    lengths = _i32(lengths)
    B = row_starts.shape[0]
    if lengths.shape != (B,):
        raise ValueError("row_starts and lengths must both be [B]")
    ends = row_starts.astype(np.int64) + np.maximum(lengths, 0)
    if B and (row_starts.min() < 0 or ends.max() > s.shape[0]):
        raise ValueError("a ragged row lies outside the packed buffer")
    out = np.empty((B, k), dtype=np.int32)
    rc = _load().ets_oracle_topk_ragged(_p32(s, ctypes.c_uint32), _p32(row_starts),
                                        _p32(lengths), B, k, _p32(out), k, threads)
    if rc != 0:
        raise RuntimeError("oracle failed (code %d)" % rc)
    return out
