"""fp64 CPU oracle for rotary position embedding (RoPE) fused with the paged
KV-cache write.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the HIP library never
does, and this module imports nothing from it.

The operation is the one the Loom Kernels home page lists as "RoPE +
paged-KV write" (packed Q/K rotation and a write into the native cache; the
benchmark page, "What the ratios mean", times it at 1-512 tokens against two
separate calls): the step that fills the cache the paged decode reads. The
pages name it without formulas, so this module takes the rotary embedding of
RoFormer (Su et al., 2021, section 3.2): pair i of a head vector, i < D/2,
turns by the angle m * theta_i at position m, with theta_i = base^(-2i/D).
Pairs are (x[i], x[i + D/2]) (the rotate-half arrangement of GPT-NeoX and of
the Qwen2 family, the model family the pages' measurement names); the
rotation of a pair by angle a is

    x'[i]       = x[i] cos a - x[i + D/2] sin a
    x'[i + D/2] = x[i + D/2] cos a + x[i] sin a.

The angles are tabulated once as a float32 cos/sin table [max_position, D]
(cos of pair i in column i, its sin in column D/2 + i); the rotation uses the
table's float32 values widened exactly. Rotated keys, and values unchanged,
go to cache slot slot_mapping[t] (block slot // block_size, row slot %
block_size) of caches laid out [num_blocks, block_size, Hkv, D]; a negative
slot writes nothing (a padding token).

Parity status: pinned by ``tests/test_oracle_rope.py`` (identity at position
0, closed forms at D = 2 and D = 4, the complex-multiplication form of the
rotation, the relative-position property, a pure-Python brute force, and
round trips of the cache write through a block table).
"""
from __future__ import annotations

import numpy as np

from . import round_to_dtype, widen


def inv_frequencies(rotary_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D) for i < D/2, in fp64."""
    if rotary_dim < 2 or rotary_dim % 2:
        raise ValueError("rotary_dim must be even and >= 2")
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * i / rotary_dim)


def cos_sin_table(max_position: int, rotary_dim: int, base: float) -> np.ndarray:
    """Exact (fp64) table [max_position, D]: cos(m theta_i) in column i,
    sin(m theta_i) in column D/2 + i."""
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_frequencies(rotary_dim, base)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def cos_sin_table_f32(max_position: int, rotary_dim: int, base: float) -> np.ndarray:
    """The float32 table: each exact entry rounded to nearest-even."""
    return cos_sin_table(max_position, rotary_dim, base).astype(np.float32)


def rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE of x [..., D] (fp64) by per-pair cos/sin [..., D/2]."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def rope_kv_write(q, k, v, positions, slot_mapping, table, k_cache, v_cache, *, dtype: str):
    """The fused step in fp64.

    q: uint16 [T, Hq, D]; k, v: uint16 [T, Hkv, D] (bit patterns of dtype);
    positions, slot_mapping: int [T]; table: float32 [max_position, D];
    k_cache, v_cache: uint16 [num_blocks, block_size, Hkv, D], the contents
    before the call.

    Returns (q_rot, k_rot, k_cache_after, v_cache_after): q_rot fp64
    [T, Hq, D] and k_rot fp64 [T, Hkv, D] unrounded; the caches as bit
    patterns after the write, the rotated keys rounded to nearest-even and the
    values copied bit for bit. Raises ValueError on a position outside the
    table, a slot outside the pool, or two tokens writing one slot.
    """
    q = np.asarray(q, np.uint16)
    k = np.asarray(k, np.uint16)
    v = np.asarray(v, np.uint16)
    pos = np.asarray(positions, np.int64)
    slots = np.asarray(slot_mapping, np.int64)
    T, Hq, D = q.shape
    if k.shape[0] != T or v.shape != k.shape or k.shape[2] != D or table.shape[1] != D:
        raise ValueError("bad shape")
    if np.any(pos < 0) or np.any(pos >= table.shape[0]):
        raise ValueError("position outside the table")
    NB, bs, Hkv, Dc = k_cache.shape
    if Dc != D or k.shape[1] != Hkv or v_cache.shape != k_cache.shape:
        raise ValueError("bad cache shape")
    live = slots >= 0
    if np.any(slots[live] >= NB * bs):
        raise ValueError("slot outside the pool")
    if len(np.unique(slots[live])) != int(live.sum()):
        raise ValueError("two tokens write one slot")

    tab = table.astype(np.float64)[pos]          # [T, D], float32 values widened
    cos, sin = tab[:, None, : D // 2], tab[:, None, D // 2:]
    q_rot = rotate(widen(q, dtype), cos, sin)
    k_rot = rotate(widen(k, dtype), cos, sin)

    kc = np.array(k_cache, np.uint16, copy=True).reshape(NB * bs, Hkv, D)
    vc = np.array(v_cache, np.uint16, copy=True).reshape(NB * bs, Hkv, D)
    kc[slots[live]] = round_to_dtype(k_rot[live], dtype)
    vc[slots[live]] = v[live]
    return q_rot, k_rot, kc.reshape(k_cache.shape), vc.reshape(v_cache.shape)
