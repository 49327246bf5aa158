"""Seeded synthetic inputs for exact per-row top-k.

This module only draws numbers; it holds none of the selection arithmetic, so
both the oracle side and the HIP side can take their inputs from it.  All
draws come from ``numpy.random.Generator(PCG64(seed))``; floating-point recipes
are evaluated in float64 and rounded to float32 (round to nearest even) by
``astype``.

The five named workloads follow the shapes of the decode traffic described on
the pages (sglang PR #36004 digest, "Motivation" and the test excerpt: fp32
indexer scores, k = 1024, page size 64, c4_len up to 32768 for a 128k context;
PR #37591 digest, "Implementation breakdown" items 2-3: k = 2048, concentrated
"banded / narrow / subnormal" score distributions, ragged rows).  The real
model logits are not available, so these stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Workload", "make", "NAMES", "normal_dense", "concentrated_row"]


@dataclass
class Workload:
    """One batch of top-k inputs (host numpy arrays)."""

    name: str
    api: str                      # "raw" | "paged" | "ragged"
    k: int
    B: int
    scores: np.ndarray            # float32 [B, L] (dense) or [N] (ragged, packed)
    L: int = 0                    # dense row stride / capacity
    lens: Optional[np.ndarray] = None        # int32 [B] valid lengths (dense)
    page_table: Optional[np.ndarray] = None  # int32 [B, P]
    page_size: int = 0
    row_starts: Optional[np.ndarray] = None  # int32 [B] (ragged)
    lengths: Optional[np.ndarray] = None     # int32 [B] (ragged)
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def row_lengths(self) -> np.ndarray:
        """Valid length of every row (dense lengths clamped to [0, L])."""
        if self.api == "ragged":
            return np.maximum(self.lengths.astype(np.int64), 0)
        if self.lens is None:
            return np.full(self.B, self.L, dtype=np.int64)
        return np.clip(self.lens.astype(np.int64), 0, self.L)

    @property
    def max_len(self) -> int:
        rl = self.row_lengths
        return int(rl.max()) if rl.size else 0


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_dense(rng: np.random.Generator, B: int, L: int) -> np.ndarray:
    """float32 [B, L] with N(0, 1) entries."""
    return rng.standard_normal((B, L), dtype=np.float64).astype(np.float32)


def concentrated_row(rng: np.random.Generator, L: int) -> np.ndarray:
    """One row where 88% of entries sit in a single coarse bucket.

    Positions are split by a random permutation into floor(0.88 L) cluster
    entries float32(1 + U * 2^-20), floor(0.10 L) N(0, 1) entries and the rest
    special: half subnormal (random sign, mantissa U{1 .. 2^23 - 1}), half
    exact duplicates copied from random cluster / normal positions.
    """
    n_cluster = int(0.88 * L)
    n_normal = int(0.10 * L)
    n_special = L - n_cluster - n_normal
    n_sub = n_special // 2
    n_dup = n_special - n_sub
    perm = rng.permutation(L)
    row = np.empty(L, dtype=np.float32)
    pc = perm[:n_cluster]
    pn = perm[n_cluster:n_cluster + n_normal]
    ps = perm[n_cluster + n_normal:n_cluster + n_normal + n_sub]
    pd = perm[n_cluster + n_normal + n_sub:]
    row[pc] = (1.0 + rng.random(n_cluster) * 2.0 ** -20).astype(np.float32)
    row[pn] = rng.standard_normal(n_normal).astype(np.float32)
    sign = rng.integers(0, 2, size=n_sub, dtype=np.uint32) << np.uint32(31)
    mant = rng.integers(1, 1 << 23, size=n_sub, dtype=np.uint32)
    row[ps] = (sign | mant).view(np.float32)
    src = rng.choice(np.concatenate([pc, pn]), size=n_dup, replace=True)
    row[pd] = row[src]
    return row


def _c1(seed: int) -> Workload:
    rng = _rng(seed)
    B, L, ps = 1, 2048, 64
    scores = normal_dense(rng, B, L)
    lens = np.full(B, L, dtype=np.int32)
    pt = np.broadcast_to(np.arange(L // ps, dtype=np.int32), (B, L // ps)).copy()
    return Workload("C1", "paged", 1024, B, scores, L=L, lens=lens, page_table=pt,
                    page_size=ps, note="B=1 L=2048 k=1024 N(0,1), identity page table")


def _c2(seed: int) -> Workload:
    rng = _rng(seed)
    B, L, ps = 48, 8192, 64
    scores = normal_dense(rng, B, L)
    lens = np.full(B, L, dtype=np.int32)
    pt = np.broadcast_to(np.arange(L // ps, dtype=np.int32), (B, L // ps)).copy()
    return Workload("C2", "paged", 1024, B, scores, L=L, lens=lens, page_table=pt,
                    page_size=ps, note="B=48 L=8192 k=1024 N(0,1), identity page table")


def _c3(seed: int) -> Workload:
    rng = _rng(seed)
    B, L, ps = 64, 32768, 64
    scores = normal_dense(rng, B, L)
    lens = rng.integers(2048, 32768, size=B, endpoint=True).astype(np.int32)
    pt = np.stack([rng.permutation(L // ps) for _ in range(B)]).astype(np.int32)
    return Workload("C3", "paged", 1024, B, scores, L=L, lens=lens, page_table=pt,
                    page_size=ps,
                    note="B=64 L=32768 k=1024 N(0,1), seq_lens U[2048,32768], "
                         "per-row random permutation of 512 page ids")


def _c4(seed: int) -> Workload:
    rng = _rng(seed)
    B, L = 128, 32768
    scores = np.stack([concentrated_row(rng, L) for _ in range(B)])
    lens = np.full(B, L, dtype=np.int32)
    return Workload("C4", "raw", 2048, B, scores, L=L, lens=lens,
                    note="B=128 L=32768 k=2048 raw, 88% in one coarse bucket, "
                         "10% N(0,1), 2% subnormal / exact duplicates")


def _c5(seed: int) -> Workload:
    rng = _rng(seed)
    B = 4
    lengths = rng.integers(65536, 262144, size=B, endpoint=True).astype(np.int32)
    row_starts = np.zeros(B, dtype=np.int32)
    row_starts[1:] = np.cumsum(lengths[:-1], dtype=np.int64).astype(np.int32)
    parts = [(rng.standard_normal(int(n)) * 1e-3 + (b + 1)).astype(np.float32)
             for b, n in enumerate(lengths)]
    packed = np.concatenate(parts)
    return Workload("C5", "ragged", 2048, B, packed, row_starts=row_starts,
                    lengths=lengths,
                    note="B=4 ragged, lengths U[65536,262144], row b = N(0,1)*1e-3 + (b+1)")


_MAKERS = {"C1": _c1, "C2": _c2, "C3": _c3, "C4": _c4, "C5": _c5}
NAMES = tuple(_MAKERS)


def make(name: str, seed: int = 42) -> Workload:
    """Build one of the named workloads C1 .. C5 from ``seed``."""
    try:
        return _MAKERS[name](seed)
    except KeyError:
        raise KeyError("unknown workload %r (have %s)" % (name, ", ".join(NAMES))) from None
