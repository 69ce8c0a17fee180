"""Seeded synthetic inputs for RoPE + paged KV-cache write.

Random numbers and layouts only, none of the rotation arithmetic; the fp64
oracle and the HIP library both consume what this module produces.

The Loom Kernels benchmark page ("What the ratios mean") times the fused step
in BF16 at 1-512 tokens for a Qwen2.5-style model; here it runs at the decode
path's geometry (Hq/Hkv = 32/8, head dim 128) unless a case says otherwise.
Recipe:

* q, k and v come packed as one array [T, Hq + 2 Hkv, D] (the layout of a
  fused QKV projection), N(0, 1) float32 draws rounded to the dtype
  (``normal_bits``, seed ``seed``).
* The caches start with N(0, 1) contents as well (seeds ``seed + 3`` and
  ``seed + 4``), so slots the call must not touch can be checked bit for bit.
* ``scatter``: positions uniform over [0, max_position) and distinct slots
  drawn from a random permutation of the pool's slots (seed ``seed + 1``);
  with ``pad_every = n`` every n-th token is padding (slot -1).
* ``prefill``: ``nseq`` sequences, each a run of consecutive positions from
  a random start, their slots taken from per-sequence block tables dealt
  from a random permutation of the pool (as the decode workloads do).
* ``decode_step``: one new token per sequence of a decode case, at position
  context_len - 1, written where that sequence's block table puts it.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import DTYPES, normal_bits

QWEN_BASE = 1.0e6  # rope base of the Qwen2 family


@dataclasses.dataclass
class RopeCase:
    name: str
    T: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    block_size: int
    max_position: int
    base: float
    qkv: np.ndarray           # uint16 [T, Hq + 2 Hkv, D]
    positions: np.ndarray     # int32 [T]
    slot_mapping: np.ndarray  # int32 [T], -1 = padding
    k_cache: np.ndarray       # uint16 [num_blocks, block_size, Hkv, D], contents before the call
    v_cache: np.ndarray       # uint16 [num_blocks, block_size, Hkv, D]
    seed: int

    @property
    def q(self) -> np.ndarray:
        return self.qkv[:, : self.Hq]

    @property
    def k(self) -> np.ndarray:
        return self.qkv[:, self.Hq: self.Hq + self.Hkv]

    @property
    def v(self) -> np.ndarray:
        return self.qkv[:, self.Hq + self.Hkv:]

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    def algorithmic_bytes(self, cache_bytes: int = 2) -> int:
        """Bytes one call must move: q, k, v in; rotated q out; k and v rows of
        the written slots (``cache_bytes`` per element: 2, or 1 for an FP8
        cache); one cos/sin row per token; positions and slots."""
        es = 2
        live = int((self.slot_mapping >= 0).sum())
        qkv_in = self.T * (self.Hq + 2 * self.Hkv) * self.D * es
        q_out = self.T * self.Hq * self.D * es
        kv_out = 2 * live * self.Hkv * self.D * cache_bytes
        table = self.T * self.D * 4
        return qkv_in + q_out + kv_out + table + 8 * self.T

    def torch_qkv(self) -> torch.Tensor:
        return torch.from_numpy(self.qkv.view(np.int16)).view(DTYPES[self.dtype])

    def torch_caches(self):
        dt = DTYPES[self.dtype]
        return tuple(torch.from_numpy(a.view(np.int16)).view(dt) for a in (self.k_cache, self.v_cache))

    def describe(self) -> str:
        live = int((self.slot_mapping >= 0).sum())
        return (f"{self.name}: T={self.T} (live {live}) Hq={self.Hq} Hkv={self.Hkv} D={self.D} "
                f"{self.dtype} bs={self.block_size} pool={self.num_blocks} "
                f"max_pos={self.max_position} seed={self.seed}")


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def _make(name, T, positions, slots, num_blocks, *, Hq, Hkv, D, dtype, block_size,
          max_position, base, seed) -> RopeCase:
    qkv = normal_bits((T, Hq + 2 * Hkv, D), dtype, seed)
    kc = normal_bits((num_blocks, block_size, Hkv, D), dtype, seed + 3)
    vc = normal_bits((num_blocks, block_size, Hkv, D), dtype, seed + 4)
    return RopeCase(name, T, Hq, Hkv, D, dtype, block_size, max_position, float(base), qkv,
                    np.asarray(positions, np.int32), np.asarray(slots, np.int32), kc, vc, seed)


def scatter(T: int, *, Hq: int = 32, Hkv: int = 8, D: int = 128, dtype: str = "bf16",
            block_size: int = 16, max_position: int = 32768, base: float = QWEN_BASE,
            pool_slots: int | None = None, pad_every: int = 0, seed: int = 0) -> RopeCase:
    """T tokens at random positions written to distinct random slots."""
    need = max(2 * T, block_size)
    nslots = pool_slots if pool_slots is not None else need
    num_blocks = -(-nslots // block_size)
    g = _gen(seed + 1)
    positions = torch.randint(0, max_position, (T,), generator=g).numpy()
    slots = torch.randperm(num_blocks * block_size, generator=g)[:T].numpy()
    if pad_every > 0:
        slots = slots.copy()
        slots[pad_every - 1:: pad_every] = -1
    return _make(f"rope_scatter_T{T}", T, positions, slots, num_blocks, Hq=Hq, Hkv=Hkv, D=D,
                 dtype=dtype, block_size=block_size, max_position=max_position, base=base,
                 seed=seed)


def prefill(nseq: int, tokens: int, *, Hq: int = 32, Hkv: int = 8, D: int = 128,
            dtype: str = "bf16", block_size: int = 16, max_position: int = 32768,
            base: float = QWEN_BASE, seed: int = 0) -> RopeCase:
    """nseq sequences of `tokens` consecutive new tokens each, from random
    start positions, slots through per-sequence block tables."""
    g = _gen(seed + 1)
    starts = torch.randint(0, max_position - tokens + 1, (nseq,), generator=g).numpy()
    mb = -(-(max_position) // block_size)
    # blocks each sequence touches, dealt from one permutation of the pool
    first = starts // block_size
    last = (starts + tokens - 1) // block_size
    used = int((last - first + 1).sum())
    num_blocks = max(2 * used, 1)
    perm = torch.randperm(num_blocks, generator=g).numpy()
    positions, slots, k = [], [], 0
    for s, f, l in zip(starts, first, last):
        table = np.full(mb, -1, np.int64)
        n = int(l - f + 1)
        table[f: l + 1] = perm[k: k + n]
        k += n
        p = np.arange(s, s + tokens, dtype=np.int64)
        positions.append(p)
        slots.append(table[p // block_size] * block_size + p % block_size)
    T = nseq * tokens
    return _make(f"rope_prefill_{nseq}x{tokens}", T, np.concatenate(positions),
                 np.concatenate(slots), num_blocks, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                 block_size=block_size, max_position=max_position, base=base, seed=seed)


def decode_step(case, *, max_position: int | None = None, base: float = QWEN_BASE,
                seed: int = 0) -> RopeCase:
    """The write that feeds a decode case: sequence b's new token sits at
    position context_lens[b] - 1, in the slot its block table gives; a
    sequence with an empty context is padding. The caches are the decode
    case's own (copied)."""
    bs = case.block_size
    L = case.context_lens.astype(np.int64)
    pos = np.maximum(L - 1, 0)
    blk = case.block_table[np.arange(case.B), pos // bs].astype(np.int64)
    slots = np.where(L > 0, blk * bs + pos % bs, -1)
    maxp = max_position if max_position is not None else int(case.max_blocks_per_seq * bs)
    qkv = normal_bits((case.B, case.Hq + 2 * case.Hkv, case.D), case.dtype, seed)
    return RopeCase(f"rope_decode_{case.name}", case.B, case.Hq, case.Hkv, case.D, case.dtype,
                    bs, maxp, float(base), qkv, pos.astype(np.int32), slots.astype(np.int32),
                    case.k_cache.copy(), case.v_cache.copy(), seed)
