"""Seeded synthetic inputs for paged KV-cache block movement (copy, gather,
scatter, compaction). Random numbers and layouts only.

Recipe (the pages give none): caches [num_blocks, block_size, Hkv, D] of
N(0, 1) draws rounded to the dtype (``normal_bits``, seeds ``seed`` for K
and ``seed + 1`` for V), at the decode geometry (Hkv 8, D 128, bf16, block
size 16) unless a case says otherwise; ids from one random permutation of
the pool (seed ``seed + 2``):

* copy: destinations are the first n ids of the permutation; each source is
  drawn, with repeats (one prefix block forked into several sequences), from
  the rest.
* gather / scatter: the first n ids of the permutation.
* compaction: each block is live with probability ``live_frac`` (seed
  ``seed + 3``); the live blocks are dealt, in a random order, to B
  sequences as their block tables (rows padded with -1).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import DTYPES, normal_bits


@dataclasses.dataclass
class BlockCase:
    name: str
    num_blocks: int
    block_size: int
    Hkv: int
    D: int
    dtype: str
    k_cache: np.ndarray  # uint16 [num_blocks, block_size, Hkv, D]
    v_cache: np.ndarray
    seed: int

    @property
    def block_bytes(self) -> int:
        return self.block_size * self.Hkv * self.D * 2

    def torch_caches(self):
        dt = DTYPES[self.dtype]
        return tuple(torch.from_numpy(a.view(np.int16)).view(dt) for a in (self.k_cache, self.v_cache))


def pool(num_blocks: int, *, block_size: int = 16, Hkv: int = 8, D: int = 128,
         dtype: str = "bf16", seed: int = 0) -> BlockCase:
    shape = (num_blocks, block_size, Hkv, D)
    return BlockCase(f"pool_NB{num_blocks}", num_blocks, block_size, Hkv, D, dtype,
                     normal_bits(shape, dtype, seed), normal_bits(shape, dtype, seed + 1), seed)


def _perm(n: int, seed: int) -> np.ndarray:
    return torch.randperm(n, generator=torch.Generator().manual_seed(int(seed))).numpy()


def copy_pairs(num_blocks: int, n: int, seed: int = 0) -> np.ndarray:
    """int32 [n, 2] (src, dst): distinct destinations, sources from the other
    blocks with repeats."""
    if 2 * n > num_blocks:
        raise ValueError("need num_blocks >= 2 n")
    p = _perm(num_blocks, seed + 2)
    g = torch.Generator().manual_seed(int(seed) + 5)
    rest = p[n:]
    src = rest[torch.randint(0, len(rest), (n,), generator=g).numpy()]
    return np.stack([src, p[:n]], axis=1).astype(np.int32)


def block_ids(num_blocks: int, n: int, seed: int = 0) -> np.ndarray:
    """int32 [n]: n distinct ids of the pool in random order."""
    return _perm(num_blocks, seed + 2)[:n].astype(np.int32)


def live_pool(num_blocks: int, B: int, live_frac: float = 0.5, seed: int = 0):
    """(live uint8 [num_blocks], block_table int32 [B, MB], n_per_seq int32 [B]):
    a random live set dealt to B sequences."""
    g = torch.Generator().manual_seed(int(seed) + 3)
    live = (torch.rand(num_blocks, generator=g) < live_frac).numpy()
    ids = np.flatnonzero(live)
    ids = ids[torch.randperm(len(ids), generator=g).numpy()]
    cuts = np.sort(torch.randint(0, len(ids) + 1, (B - 1,), generator=g).numpy())
    parts = np.split(ids, cuts)
    mb = max(1, max(len(x) for x in parts))
    bt = np.full((B, mb), -1, np.int32)
    for b, x in enumerate(parts):
        bt[b, :len(x)] = x
    return live.astype(np.uint8), bt, np.array([len(x) for x in parts], np.int32)
