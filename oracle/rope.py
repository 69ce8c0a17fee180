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

The write into an FP8 cache (``rope_kv_write_fp8``; the home page's "Next
boundaries" name FP8 KV-cache compression) stores OCP E4M3FN codes with one
float32 scale per tensor, the format the FP8 decode reads: the code of a
value x is the E4M3FN value nearest to x times the float32 reciprocal of
the scale (ties to the even code), with magnitudes beyond the largest
finite 448 held at 448 rather than turned into NaN (readings: the pages give
no quantisation rule). A code is an integer decided by floating point, so
it is decided in the precision the kernel uses, float32, in a fixed order
of operations: for a key pair (x, y) with table entries (c, s), x' =
fl(fl(x c) - fl(y s)) and y' = fl(fl(y c) + fl(x s)), fl the float32
rounding; then fl(x' * r_k) is encoded, r_k = fl(1 / k_scale). A value is
widened exactly and fl(v * r_v) encoded, r_v = fl(1 / v_scale). The rotated
query stays 16-bit as in ``rope_kv_write``.

Parity status: pinned by ``tests/test_oracle_rope.py`` (identity at position
0, closed forms at D = 2 and D = 4, the complex-multiplication form of the
rotation, the relative-position property, a pure-Python brute force, and
round trips of the cache write through a block table; the E4M3FN encoder
against torch's CPU cast on every in-range input tried, on every code's own
value and on the midpoints between codes, and its saturation by closed form;
the float32 key rotation within its rounding bound of the fp64 one).
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


# ---------------------------------------------------------------------------
# FP8 (E4M3FN) cache write

def _e4m3_values() -> np.ndarray:
    """The values of the non-negative finite E4M3FN codes 0x00 .. 0x7E, in
    code order (which is value order): exponent field e (bias 7) and
    fraction f, value f/8 * 2^-6 for e = 0, (1 + f/8) * 2^(e-7) otherwise."""
    codes = np.arange(0x7F)
    e, f = codes >> 3, codes & 7
    return np.where(e == 0, f / 8.0 * 2.0 ** -6, (1.0 + f / 8.0) * 2.0 ** (e - 7.0))


def fp8_encode(x) -> np.ndarray:
    """float32 values -> E4M3FN codes (uint8): the nearest code value, ties
    to the even code, magnitudes above 448 held at 448 (0x7E), NaN to 0x7F
    with its sign; the sign bit is the input's (so -0.0 gives 0x80)."""
    x = np.asarray(x, np.float32)
    vals = _e4m3_values()
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, vals[-1]))
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # vals[hi] >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == vals[hi], hi, code)
    sign = np.signbit(x).astype(np.int64) << 7
    out = np.where(nan, 0x7F, code) | sign
    return out.astype(np.uint8)


def rotate_f32(x, y, c, s):
    """The float32 rotation of pairs (x, y) by (c, s), in the order the FP8
    write fixes: (fl(fl(x c) - fl(y s)), fl(fl(y c) + fl(x s)))."""
    x, y, c, s = (np.asarray(t, np.float32) for t in (x, y, c, s))
    return (np.float32(x * c) - np.float32(y * s)).astype(np.float32), \
           (np.float32(y * c) + np.float32(x * s)).astype(np.float32)


def rope_kv_write_fp8(q, k, v, positions, slot_mapping, table, k_cache, v_cache, *, dtype: str,
                      k_scale: float, v_scale: float):
    """The fused step with an FP8 cache.

    As ``rope_kv_write``, with k_cache, v_cache uint8 E4M3FN codes
    [num_blocks, block_size, Hkv, D] and float32 scales. Returns (q_rot,
    k_cache_after, v_cache_after): q_rot fp64 [T, Hq, D] unrounded; at each
    written slot the key codes encode fl(x' * fl(1 / k_scale)) for the
    float32 rotation x' of ``rotate_f32`` and the value codes fl(v * fl(1 /
    v_scale)); every other byte is unchanged.
    """
    ks, vs = np.float32(k_scale), np.float32(v_scale)
    if not (np.isfinite(ks) and ks > 0 and np.isfinite(vs) and vs > 0):
        raise ValueError("scales must be finite and positive")
    k_cache = np.asarray(k_cache, np.uint8)
    v_cache = np.asarray(v_cache, np.uint8)
    dummy = np.zeros(k_cache.shape, np.uint16)
    # shape, position and slot checks and the query rotation are the 16-bit step's
    q_rot, _, _, _ = rope_kv_write(q, k, v, positions, slot_mapping, table, dummy, dummy,
                                   dtype=dtype)
    pos = np.asarray(positions, np.int64)
    slots = np.asarray(slot_mapping, np.int64)
    live = slots >= 0
    D = q.shape[2]
    h = D // 2
    tab = np.asarray(table, np.float32)[pos][:, None, :]       # [T, 1, D]
    kw = widen(np.asarray(k, np.uint16), dtype).astype(np.float32)
    x1, x2 = rotate_f32(kw[..., :h], kw[..., h:], tab[..., :h], tab[..., h:])
    k_rot = np.concatenate([x1, x2], axis=-1)
    rk, rv = np.float32(1) / ks, np.float32(1) / vs      # float32 reciprocals
    k_codes = fp8_encode((k_rot * rk).astype(np.float32))
    v_codes = fp8_encode((widen(np.asarray(v, np.uint16), dtype).astype(np.float32) * rv)
                         .astype(np.float32))
    NB, bs, Hkv, _ = k_cache.shape
    kc = np.array(k_cache, copy=True).reshape(NB * bs, Hkv, D)
    vc = np.array(v_cache, copy=True).reshape(NB * bs, Hkv, D)
    kc[slots[live]] = k_codes[live]
    vc[slots[live]] = v_codes[live]
    return q_rot, kc.reshape(k_cache.shape), vc.reshape(v_cache.shape)
