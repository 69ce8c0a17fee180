"""CPU oracle for paged KV-cache block movement: copy, gather, scatter and
compaction of whole cache blocks.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the HIP library never
does, and this module imports nothing from it.

The Loom Kernels home page ("Next boundaries": KV-cache movement) names
scheduler-facing block copy, gather, scatter and compact work for prefix
reuse and preemption, without definitions. This module takes the plainest
reading, with a block the unit of movement (all block_size rows of all KV
heads, K and V alike) and a cache any array [num_blocks, ...]:

* copy: for each pair (src, dst), block dst becomes a copy of block src (the
  copy-on-write step of prefix reuse). No block is both a source and a
  destination, and no destination repeats.
* gather: out[i] = cache[ids[i]] (blocks leaving the pool on preemption).
* scatter: cache[ids[i]] = src[i] (blocks coming back); ids distinct.
* compact: with n live blocks, move every live block whose id is >= n into
  a free id < n, the k-th such block (in increasing id order) into the k-th
  free id (in increasing order), so the live blocks fill [0, n) with the
  fewest moves; block tables then map each moved id to its new one and keep
  every other entry. Sources (>= n) and destinations (< n) never meet, so
  the copy is a plain copy.

Moves are exact: bytes go unchanged, whatever the element type.

Parity status: pinned by ``tests/test_oracle_blocks.py`` (brute-force
loops, invariants: every sequence reads the same data after a compaction,
live blocks end in [0, n), the move count is the number of live blocks at or
above n, the remap is a bijection of the live ids onto [0, n)).
"""
from __future__ import annotations

import numpy as np


def copy_blocks(cache: np.ndarray, pairs) -> np.ndarray:
    """Cache after copying block src to block dst for every (src, dst) pair."""
    pairs = np.asarray(pairs, np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    nb = cache.shape[0]
    if np.any(pairs < 0) or np.any(pairs >= nb):
        raise ValueError("block id outside the pool")
    if len(np.unique(dst)) != len(dst):
        raise ValueError("a destination repeats")
    if np.intersect1d(src, dst).size:
        raise ValueError("a block is both a source and a destination")
    out = cache.copy()
    for s, d in zip(src, dst):
        out[d] = cache[s]
    return out


def gather_blocks(cache: np.ndarray, ids) -> np.ndarray:
    """out[i] = cache[ids[i]]."""
    ids = np.asarray(ids, np.int64)
    if np.any(ids < 0) or np.any(ids >= cache.shape[0]):
        raise ValueError("block id outside the pool")
    return np.stack([cache[i] for i in ids]) if len(ids) else cache[:0].copy()


def scatter_blocks(cache: np.ndarray, ids, src: np.ndarray) -> np.ndarray:
    """Cache after cache[ids[i]] = src[i]; ids distinct."""
    ids = np.asarray(ids, np.int64)
    if np.any(ids < 0) or np.any(ids >= cache.shape[0]):
        raise ValueError("block id outside the pool")
    if len(np.unique(ids)) != len(ids):
        raise ValueError("an id repeats")
    out = cache.copy()
    for i, b in enumerate(ids):
        out[b] = src[i]
    return out


def compact_plan(live):
    """(pairs [m, 2] int64, remap [num_blocks] int64, n_live) of the compaction:
    the k-th live block at or above n_live goes to the k-th free id below it;
    remap[b] is b's new id (b itself for blocks that stay or are free)."""
    live = np.asarray(live, bool)
    n = int(live.sum())
    holes = [b for b in range(n) if not live[b]]
    movers = [b for b in range(n, live.size) if live[b]]
    assert len(holes) == len(movers)
    remap = np.arange(live.size, dtype=np.int64)
    for s, d in zip(movers, holes):
        remap[s] = d
    pairs = np.array(list(zip(movers, holes)), np.int64).reshape(-1, 2)
    return pairs, remap, n


def remap_block_table(block_table: np.ndarray, remap: np.ndarray) -> np.ndarray:
    """Each entry e with 0 <= e < len(remap) becomes remap[e]; others stay."""
    bt = np.array(block_table, np.int64, copy=True)
    ok = (bt >= 0) & (bt < len(remap))
    bt[ok] = np.asarray(remap, np.int64)[bt[ok]]
    return bt.astype(block_table.dtype)
