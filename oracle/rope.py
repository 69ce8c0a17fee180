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
float32 scale per tensor, the format the FP8 decode reads. The pages give no
quantisation rule; the reading taken is the plain one: the code of an
element is the E4M3FN value nearest to its exact value divided by the
tensor's scale (ties to the even code), magnitudes beyond the largest finite
448 held at 448 rather than turned into NaN. For a key the exact value is
the fp64 rotation of the widened input by the table's float32 cos/sin
values. A kernel computes these values in float32, so its code may be the
neighbouring one exactly where the exact value lies within the float32
evaluation's error of a midpoint between two codes;
``fp8_write_error_bounds`` derives that error from the roundings a float32
evaluation makes and ``fp8_codes_within_rounding`` is the resulting
acceptance rule. ``rope_kv_write_fp8_f32_model`` is a float32 model of one
such evaluation (products, then their difference, then the product with
the float32 reciprocal of the scale, no fused multiply-add), kept as a
bit-exact regression check, not as the definition. The rotated query stays
16-bit as in ``rope_kv_write``.

Parity status: pinned by ``tests/test_oracle_rope.py`` (identity at position
0, closed forms at D = 2 and D = 4, the complex-multiplication form of the
rotation, the relative-position property, a pure-Python brute force, and
round trips of the cache write through a block table; the E4M3FN encoder
against torch's CPU cast on every in-range input tried, on every code's own
value and on the midpoints between codes, and its saturation by closed form;
the float32 key rotation within its rounding bound of the fp64 one; the FP8
write's error bound against float32 evaluations, including values placed on
code midpoints, and its acceptance rule against planted mistakes).
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


def _nearest_e4m3(x64: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """Codes of fp64 magnitudes-with-sign: the nearest finite E4M3FN value,
    ties to the even code, magnitudes above 448 held at 448 (0x7E), NaN to
    0x7F; the sign bit is `sign`."""
    vals = _e4m3_values()
    a = np.abs(x64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, vals[-1]))
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # vals[hi] >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == vals[hi], hi, code)
    out = np.where(nan, 0x7F, code) | (sign.astype(np.int64) << 7)
    return out.astype(np.uint8)


def fp8_encode(x) -> np.ndarray:
    """float32 values -> E4M3FN codes (uint8): the nearest code value, ties
    to the even code, magnitudes above 448 held at 448 (0x7E), NaN to 0x7F
    with its sign; the sign bit is the input's (so -0.0 gives 0x80)."""
    x = np.asarray(x, np.float32)
    return _nearest_e4m3(x.astype(np.float64), np.signbit(x))


def fp8_encode_exact(x) -> np.ndarray:
    """The same rule applied to fp64 values as they are (no float32 step)."""
    x = np.asarray(x, np.float64)
    return _nearest_e4m3(x, np.signbit(x))


def fp8_value(codes) -> np.ndarray:
    """E4M3FN codes -> fp64 values (NaN for 0x7F and 0xFF), from the format:
    exponent field e (bias 7), fraction f, f/8 * 2^-6 for e = 0."""
    c = np.asarray(codes, np.int64)
    mag = _e4m3_values()[np.minimum(c & 0x7F, 0x7E)]
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def _fp8_ordinal(codes) -> np.ndarray:
    """Position of a finite code in value order, -0 and +0 both 0."""
    c = np.asarray(codes, np.int64)
    m = c & 0x7F
    return np.where(c & 0x80, -m, m)


# float32 unit roundoff (round to nearest) and half the smallest subnormal
_U32 = 2.0 ** -24
_TINY32 = 2.0 ** -150


def rotate_f32(x, y, c, s):
    """The float32 rotation of pairs (x, y) by (c, s), in the order the FP8
    write fixes: (fl(fl(x c) - fl(y s)), fl(fl(y c) + fl(x s)))."""
    x, y, c, s = (np.asarray(t, np.float32) for t in (x, y, c, s))
    return (np.float32(x * c) - np.float32(y * s)).astype(np.float32), \
           (np.float32(y * c) + np.float32(x * s)).astype(np.float32)


def rope_kv_write_fp8(q, k, v, positions, slot_mapping, table, k_cache, v_cache, *, dtype: str,
                      k_scale: float, v_scale: float):
    """The fused step into an FP8 cache by its plain definition, in fp64.

    As ``rope_kv_write``, with k_cache, v_cache uint8 E4M3FN codes
    [num_blocks, block_size, Hkv, D] and float32 scales. The key at a
    written slot is the exact rotation of the widened key by the table's
    float32 cos/sin values (fp64, ``rotate``), divided by k_scale; the value
    is the widened value divided by v_scale; each is encoded to the nearest
    E4M3FN code (ties to even, held at 448; ``fp8_encode_exact``).

    Returns a dict: q_rot (fp64 [T, Hq, D], unrounded), k_cache and v_cache
    (the codes after the write; every other byte unchanged), and, for the
    live tokens in order (slot_mapping >= 0), slots, the exact scaled keys
    and values k_exact, v_exact [n, Hkv, D] and k_eps, v_eps: how far a
    float32 evaluation may land from them (``fp8_write_error_bounds``).
    """
    ks, vs = np.float32(k_scale), np.float32(v_scale)
    if not (np.isfinite(ks) and ks > 0 and np.isfinite(vs) and vs > 0):
        raise ValueError("scales must be finite and positive")
    k_cache = np.asarray(k_cache, np.uint8)
    v_cache = np.asarray(v_cache, np.uint8)
    dummy = np.zeros(k_cache.shape, np.uint16)
    # shape, position and slot checks and both rotations are the 16-bit step's
    q_rot, k_rot, _, _ = rope_kv_write(q, k, v, positions, slot_mapping, table, dummy, dummy,
                                       dtype=dtype)
    pos = np.asarray(positions, np.int64)
    slots = np.asarray(slot_mapping, np.int64)
    live = slots >= 0
    D = q.shape[2]
    h = D // 2
    k_exact = k_rot[live] / np.float64(ks)
    v_exact = widen(np.asarray(v, np.uint16), dtype)[live] / np.float64(vs)
    tab = np.asarray(table, np.float32).astype(np.float64)[pos[live]][:, None, :]
    kw = widen(np.asarray(k, np.uint16), dtype)[live]
    c, sn = tab[..., :h], tab[..., h:]
    x, y = kw[..., :h], kw[..., h:]
    mag = np.concatenate([np.abs(x * c) + np.abs(y * sn), np.abs(y * c) + np.abs(x * sn)], axis=-1)
    k_eps, v_eps = fp8_write_error_bounds(mag, np.abs(v_exact) * np.float64(vs), ks, vs)
    NB, bs, Hkv, _ = k_cache.shape
    kc = np.array(k_cache, copy=True).reshape(NB * bs, Hkv, D)
    vc = np.array(v_cache, copy=True).reshape(NB * bs, Hkv, D)
    kc[slots[live]] = fp8_encode_exact(k_exact)
    vc[slots[live]] = fp8_encode_exact(v_exact)
    return {"q_rot": q_rot, "k_cache": kc.reshape(k_cache.shape),
            "v_cache": vc.reshape(v_cache.shape), "slots": slots[live], "k_exact": k_exact,
            "v_exact": v_exact, "k_eps": k_eps, "v_eps": v_eps}


def fp8_write_error_bounds(key_terms, value_mag, k_scale, v_scale):
    """Bounds on |float32 result - exact scaled value| for the FP8 write.

    A float32 evaluation of a rotated key x c - y s (or y c + x s) divided
    by the scale may round each product, their sum and the reciprocal of
    the scale and the final product once: with u = 2^-24, A = |x c| + |y s|
    and d the rounded sum, |d - (x c - y s)| <= (2u + u^2) A, and the two
    further roundings scale by (1 + u)^2, so

        |result - exact| <= (2u + u^2) ((1 + u)^2 + 1) A / k_scale

    plus, for results in the float32 subnormal range, an absolute 2^-150 per
    rounding (three before the reciprocal product, one after, and one on the
    reciprocal). A value v takes two roundings (reciprocal and product):
    (2u + u^2) |v| / v_scale plus the same absolute terms. A relative 1e-15
    covers the fp64 evaluation of the exact values. key_terms: A per key
    element; value_mag: |v|. Returns (k_eps, v_eps)."""
    u, t = _U32, _TINY32
    ks, vs = np.float64(k_scale), np.float64(v_scale)
    A = np.asarray(key_terms, np.float64)
    vm = np.asarray(value_mag, np.float64)
    k_eps = ((2 * u + u * u) * ((1 + u) ** 2 + 1) + 1e-15) * A / ks \
        + 3 * t * (1 + u) ** 2 / ks + t + t * A * (1 + u) ** 2
    v_eps = ((2 * u + u * u) + 1e-15) * vm / vs + t + t * vm * (1 + u)
    return k_eps, v_eps


def fp8_codes_within_rounding(got, exact, eps):
    """The FP8 write's acceptance rule. A written code passes when it
    stands for the same value as the nearest code of the exact value, or
    for the adjacent value on the other side of a rounding midpoint m with
    |exact - m| <= eps (a float32 evaluation within eps of the exact value
    may land on either side of m). Returns (passes [bool array], number of
    adjacent-code passes)."""
    got = np.asarray(got, np.uint8)
    exact = np.asarray(exact, np.float64)
    ref = fp8_encode_exact(exact)
    gv, rv = fp8_value(got), fp8_value(ref)
    same = gv == rv
    adj = np.abs(_fp8_ordinal(got) - _fp8_ordinal(ref)) == 1
    near = np.abs(exact - 0.5 * (gv + rv)) <= eps
    ok = same | (adj & near)
    return ok, int(np.count_nonzero(adj & near & ~same))


def rope_kv_write_fp8_f32_model(q, k, v, positions, slot_mapping, table, k_cache, v_cache, *,
                                dtype: str, k_scale: float, v_scale: float):
    """A float32 model of the FP8 write: a bit-exact regression check, not
    the definition (that is ``rope_kv_write_fp8``).

    The codes encode fl(x' * fl(1 / k_scale)) for the float32 rotation x' of
    ``rotate_f32`` and fl(v * fl(1 / v_scale)), fl the float32 rounding, in
    that order with no fused multiply-add. Returns (q_rot, k_cache_after,
    v_cache_after).
    """
    ks, vs = np.float32(k_scale), np.float32(v_scale)
    if not (np.isfinite(ks) and ks > 0 and np.isfinite(vs) and vs > 0):
        raise ValueError("scales must be finite and positive")
    k_cache = np.asarray(k_cache, np.uint8)
    v_cache = np.asarray(v_cache, np.uint8)
    dummy = np.zeros(k_cache.shape, np.uint16)
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
