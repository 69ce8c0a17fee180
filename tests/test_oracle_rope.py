"""Pins of the RoPE + paged-KV-write oracle (oracle/rope.py) against what the
rotary embedding's definition fixes (RoFormer, section 3.2; rotate-half
pairing), independent of the oracle's own formulas: closed forms at D = 2 and
D = 4, the complex-multiplication form, the relative-position property, a
pure-Python brute force and cache round trips through block tables."""
import cmath
import math

import numpy as np
import pytest

import oracle
from oracle import rope
import workloads
from workloads import rope as wrope


def test_table_row_zero_is_identity():
    t = rope.cos_sin_table(4, 128, 1e6)
    assert np.all(t[0, :64] == 1.0) and np.all(t[0, 64:] == 0.0)


def test_d2_closed_form():
    # D = 2: one pair, theta_0 = 1 whatever the base; (1, 0) at position m
    # turns to (cos m, sin m): counter-clockwise, as R(m theta) of RoFormer
    for m in (1, 2, 7):
        tab = rope.cos_sin_table(m + 1, 2, 10000.0)
        out = rope.rotate(np.array([1.0, 0.0]), tab[m, :1], tab[m, 1:])
        assert out[0] == pytest.approx(math.cos(m), abs=1e-15)
        assert out[1] == pytest.approx(math.sin(m), abs=1e-15)
        # and (0, 1) turns to (-sin m, cos m)
        out = rope.rotate(np.array([0.0, 1.0]), tab[m, :1], tab[m, 1:])
        assert out[0] == pytest.approx(-math.sin(m), abs=1e-15)
        assert out[1] == pytest.approx(math.cos(m), abs=1e-15)


def test_d4_frequency_and_pairing():
    # D = 4, base 100: theta = (1, 100^-1/2 = 0.1). Dimension 1 pairs with
    # dimension 3 (rotate-half), and turns by 10 * 0.1 = 1 rad at position 10.
    tab = rope.cos_sin_table(11, 4, 100.0)
    x = np.array([0.0, 1.0, 0.0, 0.0])
    out = rope.rotate(x, tab[10, :2], tab[10, 2:])
    assert out == pytest.approx([0.0, math.cos(1.0), 0.0, math.sin(1.0)], abs=1e-14)
    # dimension 0 turns by 10 rad, into dimension 2
    out = rope.rotate(np.array([1.0, 0.0, 0.0, 0.0]), tab[10, :2], tab[10, 2:])
    assert out == pytest.approx([math.cos(10.0), 0.0, math.sin(10.0), 0.0], abs=1e-14)


def test_inv_frequencies_closed_form():
    th = rope.inv_frequencies(128, 1e6)
    assert th[0] == 1.0
    assert th[32] == pytest.approx(1e6 ** -0.5, rel=1e-15)
    assert th[63] == pytest.approx(1e6 ** (-126 / 128), rel=1e-14)
    assert np.all(np.diff(th) < 0)


def test_complex_form():
    # pair i as the complex number x[i] + j x[i + D/2], times exp(j m theta_i)
    rng = np.random.default_rng(5)
    D, base = 128, 1e6
    x = rng.standard_normal(D)
    th = [base ** (-2 * i / D) for i in range(D // 2)]
    for m in (0, 1, 37, 4095, 31999):
        tab = rope.cos_sin_table(m + 1, D, base)
        out = rope.rotate(x, tab[m, : D // 2], tab[m, D // 2:])
        for i in range(D // 2):
            z = complex(x[i], x[i + D // 2]) * cmath.exp(1j * m * th[i])
            assert out[i] == pytest.approx(z.real, abs=1e-11)
            assert out[i + D // 2] == pytest.approx(z.imag, abs=1e-11)


def test_relative_position_and_norm():
    # <R(m) q, R(n) k> depends on m - n only; each pair keeps its length
    rng = np.random.default_rng(6)
    D, base = 64, 10000.0
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    tab = rope.cos_sin_table(200, D, base)
    h = D // 2

    def R(x, m):
        return rope.rotate(x, tab[m, :h], tab[m, h:])

    for m, n, s in ((5, 3, 40), (100, 17, 60), (9, 9, 150)):
        assert np.dot(R(q, m), R(k, n)) == pytest.approx(np.dot(R(q, m + s), R(k, n + s)), abs=1e-10)
        assert np.dot(R(q, m), R(k, n)) == pytest.approx(np.dot(R(q, m - n), k), abs=1e-10)
        r = R(q, m)
        assert np.hypot(r[:h], r[h:]) == pytest.approx(np.hypot(q[:h], q[h:]), abs=1e-12)


def test_table_f32_is_rounded_exact_table():
    t64 = rope.cos_sin_table(300, 128, 1e6)
    t32 = rope.cos_sin_table_f32(300, 128, 1e6)
    assert t32.dtype == np.float32
    # every float32 entry is the nearest float32 to the exact value
    up = np.nextafter(t32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(t32, np.float32(-np.inf)).astype(np.float64)
    e = np.abs(t32.astype(np.float64) - t64)
    assert np.all(e <= np.abs(up - t64)) and np.all(e <= np.abs(dn - t64))
    assert np.allclose(t64[:, :64] ** 2 + t64[:, 64:] ** 2, 1.0, atol=1e-15)


def _brute(case, table):
    """Pure-Python loops, scalar math, for a tiny case."""
    T, Hq, Hkv, D = case.T, case.Hq, case.Hkv, case.D
    h2 = D // 2
    qv = oracle.widen(case.q, case.dtype)
    kv = oracle.widen(case.k, case.dtype)
    qo = np.zeros((T, Hq, D))
    ko = np.zeros((T, Hkv, D))
    for t in range(T):
        p = int(case.positions[t])
        for src, dst, H in ((qv, qo, Hq), (kv, ko, Hkv)):
            for h in range(H):
                for i in range(h2):
                    c, s = float(table[p, i]), float(table[p, h2 + i])
                    a, b = float(src[t, h, i]), float(src[t, h, i + h2])
                    dst[t, h, i] = a * c - b * s
                    dst[t, h, i + h2] = b * c + a * s
    return qo, ko


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_brute_force_tiny(dtype):
    case = wrope.scatter(5, Hq=8, Hkv=2, D=64, dtype=dtype, max_position=1000, pad_every=3, seed=2)
    table = rope.cos_sin_table_f32(case.max_position, case.D, case.base)
    q_rot, k_rot, kc, vc = rope.rope_kv_write(case.q, case.k, case.v, case.positions,
                                              case.slot_mapping, table, case.k_cache,
                                              case.v_cache, dtype=dtype)
    qb, kb = _brute(case, table)
    assert np.allclose(q_rot, qb, rtol=0, atol=1e-12)
    assert np.allclose(k_rot, kb, rtol=0, atol=1e-12)
    # slot s sits at block s // bs, row s % bs; padding tokens write nothing
    bs = case.block_size
    touched = np.zeros(case.k_cache.shape[:2], bool)
    for t in range(case.T):
        s = int(case.slot_mapping[t])
        if s < 0:
            continue
        touched[s // bs, s % bs] = True
        assert np.array_equal(kc[s // bs, s % bs], oracle.round_to_dtype(kb[t], dtype))
        assert np.array_equal(vc[s // bs, s % bs], case.v[t])
    assert np.array_equal(kc[~touched], case.k_cache[~touched])
    assert np.array_equal(vc[~touched], case.v_cache[~touched])
    assert int((case.slot_mapping < 0).sum()) == 1


def test_position_zero_writes_keys_unchanged():
    case = wrope.scatter(4, Hq=4, Hkv=1, D=128, max_position=1, seed=3)
    assert np.all(case.positions == 0)
    table = rope.cos_sin_table_f32(1, 128, case.base)
    q_rot, k_rot, kc, _ = rope.rope_kv_write(case.q, case.k, case.v, case.positions,
                                             case.slot_mapping, table, case.k_cache,
                                             case.v_cache, dtype="bf16")
    assert np.array_equal(q_rot, oracle.widen(case.q, "bf16"))
    flat = kc.reshape(-1, 1, 128)
    for t in range(4):
        assert np.array_equal(flat[case.slot_mapping[t]], case.k[t])


@pytest.mark.parametrize("bs", [16, 32])
def test_decode_step_round_trip(bs):
    # the new token of each sequence lands where the decode reads position L-1
    dec = workloads.make_case("rt", 6, [1, 17, 33, 64, 5, 40], dtype="bf16", block_size=bs,
                              Hq=8, Hkv=2, D=128, seed=4)
    case = wrope.decode_step(dec, seed=9)
    table = rope.cos_sin_table_f32(case.max_position, 128, case.base)
    _, k_rot, kc, vc = rope.rope_kv_write(case.q, case.k, case.v, case.positions,
                                          case.slot_mapping, table, case.k_cache,
                                          case.v_cache, dtype="bf16")
    for b in range(dec.B):
        L = int(dec.context_lens[b])
        blk = dec.block_table[b, (L - 1) // bs]
        assert np.array_equal(kc[blk, (L - 1) % bs], oracle.round_to_dtype(k_rot[b], "bf16"))
        assert np.array_equal(vc[blk, (L - 1) % bs], case.v[b])
        assert case.positions[b] == L - 1


def test_prefill_slots_follow_block_tables():
    case = wrope.prefill(3, 40, Hq=4, Hkv=1, D=64, block_size=16, max_position=500, seed=1)
    assert case.T == 120
    s = case.slot_mapping.astype(np.int64)
    assert len(np.unique(s)) == 120 and np.all(s >= 0)
    for q in range(3):
        p = case.positions[q * 40:(q + 1) * 40].astype(np.int64)
        assert np.all(np.diff(p) == 1)
        sl = s[q * 40:(q + 1) * 40]
        # consecutive positions in one block occupy consecutive rows
        same = (p[1:] // 16) == (p[:-1] // 16)
        assert np.all((sl[1:] - sl[:-1])[same] == 1)
        assert np.all(sl % 16 == p % 16)


def test_oracle_rejects_bad_inputs():
    case = wrope.scatter(3, Hq=4, Hkv=1, D=64, max_position=10, seed=0)
    table = rope.cos_sin_table_f32(10, 64, case.base)
    args = (case.q, case.k, case.v)
    with pytest.raises(ValueError):
        rope.rope_kv_write(*args, np.array([0, 1, 10]), case.slot_mapping, table,
                           case.k_cache, case.v_cache, dtype="bf16")
    with pytest.raises(ValueError):
        rope.rope_kv_write(*args, case.positions, np.array([0, 0, 1]), table,
                           case.k_cache, case.v_cache, dtype="bf16")
    with pytest.raises(ValueError):
        rope.rope_kv_write(*args, case.positions, np.array([0, 1, case.num_blocks * 16]), table,
                           case.k_cache, case.v_cache, dtype="bf16")


# ---------------------------------------------------------------------------
# the FP8 (E4M3FN) cache write


def torch_e4m3(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_encode_gives_every_code_back():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = oracle.widen_fp8(codes).astype(np.float32)
    assert np.array_equal(rope.fp8_encode(vals), codes)


def test_fp8_encode_matches_torch_inside_the_range():
    # torch's CPU cast rounds to nearest-even; checked on log-uniform values
    # over the whole range (subnormals included), every code's midpoint with
    # its neighbour, and one float32 step either side of each midpoint
    rng = np.random.default_rng(0)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 200000)).astype(np.float32)
    x = mag * np.where(rng.random(mag.size) < 0.5, -1, 1).astype(np.float32)
    vals = oracle.widen_fp8(np.arange(0x7F, dtype=np.uint8))
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)      # exact in float32
    near = np.concatenate([mid, np.nextafter(mid, np.float32(0)),
                           np.nextafter(mid, np.float32(1000))])
    x = np.concatenate([x, near, -near]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(rope.fp8_encode(x), torch_e4m3(x))


def test_fp8_encode_ties_go_to_the_even_code():
    vals = oracle.widen_fp8(np.arange(0x7F, dtype=np.uint8))
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    got = rope.fp8_encode(mid).astype(int)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))


def test_fp8_encode_holds_large_magnitudes_at_448():
    x = np.array([448.0, 450.0, 464.0, 464.03125, 480.0, 1e6, 3e38, np.inf], np.float32)
    assert np.all(rope.fp8_encode(x) == 0x7E)
    assert np.all(rope.fp8_encode(-x) == 0xFE)
    assert rope.fp8_encode(np.float32(np.nan)) & 0x7F == 0x7F
    assert rope.fp8_encode(np.float32(-0.0)) == 0x80 and rope.fp8_encode(np.float32(0.0)) == 0


def test_float32_key_rotation_is_within_its_rounding_of_the_exact_one():
    rng = np.random.default_rng(1)
    x, y = (rng.standard_normal(100000).astype(np.float32) for _ in range(2))
    a = rng.uniform(0, 2 * np.pi, 100000)
    c, s = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
    x1, y1 = rope.rotate_f32(x, y, c, s)
    X, Y, C, S = (t.astype(np.float64) for t in (x, y, c, s))
    u = 2.0 ** -24
    # three roundings: of each product and of the sum
    assert np.all(np.abs(x1 - (X * C - Y * S)) <= u * (np.abs(X * C) + np.abs(Y * S)) * 2.01 + 1e-45)
    assert np.all(np.abs(y1 - (Y * C + X * S)) <= u * (np.abs(Y * C) + np.abs(X * S)) * 2.01 + 1e-45)
    # and the order is the stated one: products rounded first
    assert np.array_equal(x1, (np.float32(x * c) - np.float32(y * s)).astype(np.float32))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_write_codes_stand_for_the_scaled_16bit_write(dtype):
    case = wrope.scatter(24, Hq=4, Hkv=2, D=64, dtype=dtype, block_size=16, seed=5,
                         pad_every=5, max_position=4096)
    tab = rope.cos_sin_table_f32(case.max_position, case.D, case.base)
    ks, vs = 0.0125, 0.0078125
    kc0 = np.full(case.k_cache.shape, 0x11, np.uint8)
    vc0 = np.full(case.v_cache.shape, 0x22, np.uint8)
    r = rope.rope_kv_write_fp8(case.q, case.k, case.v, case.positions, case.slot_mapping, tab,
                               kc0, vc0, dtype=dtype, k_scale=ks, v_scale=vs)
    kc, vc = r["k_cache"], r["v_cache"]
    q_rot, k_rot, _, _ = rope.rope_kv_write(case.q, case.k, case.v, case.positions,
                                            case.slot_mapping, tab, case.k_cache,
                                            case.v_cache, dtype=dtype)
    assert np.array_equal(r["q_rot"], q_rot)
    live = case.slot_mapping >= 0
    s = case.slot_mapping[live].astype(np.int64)
    assert np.array_equal(r["slots"], s)
    kf = kc.reshape(-1, case.Hkv, case.D)
    vf = vc.reshape(-1, case.Hkv, case.D)
    # each code is the nearest E4M3FN value to the exact key/value over the
    # scale: within half a code step (2^-4 relative, or 2^-10 absolute below
    # 2^-6; exact division and exact rotation, so no slack)
    kd = oracle.widen_fp8(kf[s]) * ks
    vd = oracle.widen_fp8(vf[s]) * vs
    kr, vr = k_rot[live], oracle.widen(case.v, dtype)[live]
    assert np.all(np.abs(kd - kr) <= 2.0 ** -4 * np.abs(kr) + 2.0 ** -10 * ks)
    assert np.all(np.abs(vd - vr) <= 2.0 ** -4 * np.abs(vr) + 2.0 ** -10 * vs)
    # nothing else was touched
    untouched = np.ones(kf.shape[0], bool)
    untouched[s] = False
    assert np.all(kf[untouched] == 0x11) and np.all(vf[untouched] == 0x22)


# ---------------------------------------------------------------------------
# the FP8 write's error bound and acceptance rule (oracle/rope.py): a float32
# evaluation of x c - y s (or a value) times the float32 reciprocal of the
# scale stays within fp8_write_error_bounds of the exact quotient, and a
# code the rule accepts is the nearest one or its neighbour across a
# midpoint that the bound reaches

def f32_keys(x, y, c, sn, ks):
    """A float32 evaluation in another legitimate order than the model's:
    fused products (x*c exact in fp64, rounded once with y*s) then the
    reciprocal product."""
    X, Y, C, S = (np.asarray(t, np.float64) for t in (x, y, c, sn))
    d = (X * C - Y * S).astype(np.float32)
    return (d * (np.float32(1) / np.float32(ks))).astype(np.float32)


def keys_on_midpoints(rng, n, ks):
    """Key pairs (x, y) and angles whose exact rotated value over ks lands
    within a few float32 roundings of a midpoint between two E4M3FN codes."""
    vals = rope.fp8_value(np.arange(0x7E, dtype=np.uint8))
    mids = 0.5 * (vals[:-1] + vals[1:])
    m = rng.choice(mids, size=n) * rng.choice([-1.0, 1.0], size=n)
    a = rng.uniform(0, 2 * np.pi, n)
    c, sn = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
    # x c - y s = m ks with y drawn, x solved and rounded to bf16
    y = (rng.standard_normal(n) * 0.5).astype(np.float32)
    x = ((m * ks + y.astype(np.float64) * sn) / np.where(np.abs(c) < 1e-3, 1e-3, c))
    xb = oracle.widen(oracle.round_to_dtype(x, "bf16"), "bf16")
    yb = oracle.widen(oracle.round_to_dtype(y, "bf16"), "bf16")
    return xb, yb, c, sn


@pytest.mark.parametrize("ks", [0.01, 0.0125, 0.003, 1.0 / 3.0, 7.5e-4])
def test_fp8_key_error_bound_covers_float32_evaluations(ks):
    rng = np.random.default_rng(int(ks * 1e6))
    x, y, c, sn = keys_on_midpoints(rng, 200000, ks)
    X, Y, C, S = (np.asarray(t, np.float64) for t in (x, y, c, sn))
    exact = (X * C - Y * S) / np.float64(np.float32(ks))
    A = np.abs(X * C) + np.abs(Y * S)
    eps, _ = rope.fp8_write_error_bounds(A, np.zeros(1), np.float32(ks), np.float32(1))
    x1, _ = rope.rotate_f32(x.astype(np.float32), y.astype(np.float32), c, sn)
    model = (x1 * (np.float32(1) / np.float32(ks))).astype(np.float32).astype(np.float64)
    other = f32_keys(x, y, c, sn, ks).astype(np.float64)
    for v in (model, other):
        err = np.abs(v - exact)
        assert np.all(err <= eps)
        # and the bound is not vacuous: some evaluation comes within 10x of it
        assert (err / eps).max() > 0.1


@pytest.mark.parametrize("vs", [0.01, 0.02, 0.003, 1.0 / 3.0])
def test_fp8_value_error_bound_covers_float32_evaluations(vs):
    rng = np.random.default_rng(int(vs * 1e6) + 1)
    v = oracle.widen(oracle.round_to_dtype(rng.standard_normal(500000), "bf16"), "bf16")
    exact = v / np.float64(np.float32(vs))
    _, eps = rope.fp8_write_error_bounds(np.zeros(1), np.abs(v), np.float32(1), np.float32(vs))
    model = (v.astype(np.float32) * (np.float32(1) / np.float32(vs))).astype(np.float32)
    err = np.abs(model.astype(np.float64) - exact)
    assert np.all(err <= eps) and (err / eps).max() > 0.1


def test_fp8_acceptance_rule_takes_the_float32_model_and_counts_midpoint_cases():
    case = wrope.scatter(64, Hq=32, Hkv=8, D=128, dtype="bf16", block_size=16, seed=3,
                         pad_every=0, max_position=32768)
    tab = rope.cos_sin_table_f32(case.max_position, case.D, case.base)
    zeros = np.zeros(case.k_cache.shape, np.uint8)
    r = rope.rope_kv_write_fp8(case.q, case.k, case.v, case.positions, case.slot_mapping, tab,
                               zeros, zeros, dtype="bf16", k_scale=0.01, v_scale=0.01)
    _, km, vm = rope.rope_kv_write_fp8_f32_model(case.q, case.k, case.v, case.positions,
                                                 case.slot_mapping, tab, zeros, zeros,
                                                 dtype="bf16", k_scale=0.01, v_scale=0.01)
    s = r["slots"]
    ok_k, n_k = rope.fp8_codes_within_rounding(km.reshape(-1, 8, 128)[s], r["k_exact"],
                                               r["k_eps"])
    ok_v, n_v = rope.fp8_codes_within_rounding(vm.reshape(-1, 8, 128)[s], r["v_exact"],
                                               r["v_eps"])
    assert ok_k.all() and ok_v.all()
    # 1/0.01 is not a float32: bf16 values times fl(1/0.01) sit on either
    # side of the codes' midpoints where the exact quotient does not
    assert n_v > 0
    assert n_k + n_v < 0.02 * (ok_k.size + ok_v.size)


def test_fp8_acceptance_rule_rejects_planted_mistakes():
    vals = rope.fp8_value(np.arange(0x7F, dtype=np.uint8))
    exact = np.array([1.0, 1.0, 0.3, 101.0, -2.0, 448.0, 0.0])
    eps = np.full(exact.shape, 1e-6)
    ref = rope.fp8_encode_exact(exact)
    assert rope.fp8_codes_within_rounding(ref, exact, eps)[0].all()
    # one code too high, away from any midpoint
    ok, _ = rope.fp8_codes_within_rounding(ref + 1, exact[:5].tolist() + [440.0, 0.01], eps)
    assert not ok[:5].any()
    # two codes off, the sign flipped, a NaN code
    assert not rope.fp8_codes_within_rounding(ref[:1] + 2, exact[:1], eps[:1])[0].any()
    assert not rope.fp8_codes_within_rounding(ref[4:5] ^ 0x80, exact[4:5], eps[4:5])[0].any()
    assert not rope.fp8_codes_within_rounding(np.array([0x7F], np.uint8), exact[:1],
                                              eps[:1])[0].any()
    # a neighbour is taken only within eps of the midpoint between the two
    mid = 0.5 * (vals[40] + vals[41])
    for delta, want in ((0.5e-6, True), (2e-6, False)):
        x = np.array([mid - delta])  # exact just below the midpoint: nearest is code 40
        assert rope.fp8_encode_exact(x)[0] == 40
        ok, n = rope.fp8_codes_within_rounding(np.array([41], np.uint8), x, np.array([1e-6]))
        assert bool(ok[0]) == want and n == int(want)
    # a rotation with the sign of the sine flipped fails the rule
    case = wrope.scatter(8, Hq=4, Hkv=2, D=64, dtype="bf16", block_size=16, seed=4,
                         pad_every=0, max_position=4096)
    tab = rope.cos_sin_table_f32(case.max_position, case.D, case.base)
    zeros = np.zeros(case.k_cache.shape, np.uint8)
    r = rope.rope_kv_write_fp8(case.q, case.k, case.v, case.positions, case.slot_mapping, tab,
                               zeros, zeros, dtype="bf16", k_scale=0.01, v_scale=0.01)
    bad = tab.copy()
    bad[:, 32:] *= -1
    rb = rope.rope_kv_write_fp8(case.q, case.k, case.v, case.positions, case.slot_mapping, bad,
                                zeros, zeros, dtype="bf16", k_scale=0.01, v_scale=0.01)
    s = r["slots"]
    ok, _ = rope.fp8_codes_within_rounding(rb["k_cache"].reshape(-1, 2, 64)[s], r["k_exact"],
                                           r["k_eps"])
    assert ok.mean() < 0.5
