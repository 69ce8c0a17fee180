"""Pins of the fp64 oracle against facts it cannot produce by itself.

Each test fixes the oracle to a closed form, an invariant of softmax
attention, an identity of the split-K/LSE regrouping (Loom Kernels home page,
"Supported now": paged MQA/GQA decode with GQA packing and local split-K/LSE),
or an exact library conversion. The tests are chosen so that a plausible
mistake in the oracle (a dropped scale, a wrong sign, a swapped block/slot or
head index, an off-by-one on the context, a wrong merge weight, a rounding
slip) fails at least one of them. No GPU is involved.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

RNG = np.random.default_rng(1234)
TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def bits(x, dtype):
    """float values -> 16-bit patterns (torch CPU cast, RNE)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(TDT[dtype])
    return t.view(torch.int16).numpy().view(np.uint16)


def vals(b, dtype):
    return oracle.widen(b, dtype)


def small_case(B=3, Hq=8, Hkv=2, D=16, bs=4, ctx=(5, 9, 1), dtype="bf16", seed=0,
               q_sigma=1.0, extra_pool=3):
    g = np.random.default_rng(seed)
    ctx = np.asarray(ctx, np.int32)
    need = [-(-int(L) // bs) for L in ctx]
    MB = max(1, max(need))
    pool = sum(need) + extra_pool
    perm = g.permutation(pool).astype(np.int32)
    bt = np.zeros((B, MB), np.int32)
    pos = 0
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
        bt[b, need[b]:] = perm[-1]
    q = bits(g.standard_normal((B, Hq, D)) * q_sigma, dtype)
    k = bits(g.standard_normal((pool, bs, Hkv, D)), dtype)
    v = bits(g.standard_normal((pool, bs, Hkv, D)), dtype)
    return dict(q=q, k_cache=k, v_cache=v, block_table=bt, context_lens=ctx), dtype


def run(c, dtype, scale=0.25, **kw):
    return oracle.attention(c["q"], c["k_cache"], c["v_cache"], c["block_table"],
                            c["context_lens"], scale=scale, dtype=dtype, **kw)


def gather(c, dtype, b, g):
    """Valid K and V rows of (sequence b, kv head g), by logical token."""
    L = int(c["context_lens"][b])
    bs = c["k_cache"].shape[1]
    t = np.arange(L)
    ids = c["block_table"][b, t // bs]
    K = vals(c["k_cache"][ids, t % bs, g, :], dtype)
    V = vals(c["v_cache"][ids, t % bs, g, :], dtype)
    return K, V


# --------------------------------------------------------------------------
# 16-bit conversions

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_widen_is_exact_for_every_pattern(dtype):
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(allb, dtype)
    if dtype == "bf16":
        ref = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    else:
        ref = allb.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_round_bf16_matches_torch_on_float32_inputs():
    # random float32 patterns across the whole range, plus exact halfway points
    r = RNG.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    half = (RNG.integers(0, 1 << 16, size=20000).astype(np.uint32) << 16) | 0x8000
    x32 = np.concatenate([r, half]).view(np.float32)
    x32 = x32[~np.isnan(x32)]
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_to_dtype(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def test_round_f16_matches_numpy_on_float64_inputs():
    e = RNG.uniform(-30, 18, size=200000)
    x = RNG.choice([-1.0, 1.0], size=e.size) * RNG.uniform(1, 2, size=e.size) * 2.0 ** e
    # exact f16 halfway points (ties to even) and neighbours
    b = RNG.integers(0, 0x7bff, size=20000).astype(np.uint16)
    lo = b.view(np.float16).astype(np.float64)
    hi = (b + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (lo + hi) / 2
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -25, 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.round_to_dtype(x, "f16")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_round_inverts_widen(dtype):
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    w = oracle.widen(allb, dtype)
    keep = ~np.isnan(w)
    assert np.array_equal(oracle.round_to_dtype(w[keep], dtype), allb[keep])


# --------------------------------------------------------------------------
# closed forms

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_token_context_returns_v_exactly(dtype):
    c, dt = small_case(ctx=(1, 1, 1), dtype=dtype, seed=3)
    out, lse = run(c, dt)
    G = 8 // 2
    for b in range(3):
        blk = c["block_table"][b, 0]
        for h in range(8):
            assert np.array_equal(out[b, h], vals(c["v_cache"][blk, 0, h // G], dt))


def test_constant_v_returns_the_constant():
    c, dt = small_case(ctx=(7, 13, 2), seed=4)
    row = bits(RNG.standard_normal(16), dt)
    c["v_cache"][:] = row  # every slot, every head
    out, _ = run(c, dt)
    ref = vals(row, dt)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("which", ["q", "k"])
def test_zero_q_or_k_gives_the_mean_of_exactly_the_valid_tokens(which):
    c, dt = small_case(ctx=(5, 9, 1), seed=5)
    c[which if which == "q" else "k_cache"][:] = 0
    out, lse = run(c, dt)
    for b in range(3):
        L = int(c["context_lens"][b])
        for h in range(8):
            _, V = gather(c, dt, b, h // 4)
            assert V.shape[0] == L
            assert np.max(np.abs(out[b, h] - V.mean(axis=0))) <= 1e-12
            assert lse[b, h] == pytest.approx(math.log(L), abs=1e-14)


def test_two_token_closed_form_pins_scale_and_sign():
    c, dt = small_case(B=1, ctx=(2,), seed=6)
    scale = float(np.float32(0.3))   # the scale argument is a float32
    out, lse = run(c, dt, scale=scale)
    qv = vals(c["q"], dt)
    for h in range(8):
        K, V = gather(c, dt, 0, h // 4)
        s0, s1 = scale * float(qv[0, h] @ K[0]), scale * float(qv[0, h] @ K[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        assert np.max(np.abs(out[0, h] - (w0 * V[0] + w1 * V[1]))) <= 1e-12
        hi, lo = max(s0, s1), min(s0, s1)
        assert lse[0, h] == pytest.approx(hi + math.log1p(math.exp(lo - hi)), abs=1e-12)


@pytest.mark.parametrize("pos", ["first", "block_edge", "last"])
def test_needle_picks_exactly_one_token(pos):
    B, Hq, Hkv, D, bs = 1, 8, 2, 16, 4
    L = 11
    c, dt = small_case(B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, ctx=(L,), seed=7)
    tstar = {"first": 0, "block_edge": bs - 1, "last": L - 1}[pos]
    c["k_cache"][:] = 0
    qrow = bits(np.ones(D), dt)
    c["q"][:] = qrow
    blk = c["block_table"][0, tstar // bs]
    c["k_cache"][blk, tstar % bs, :, :] = bits(np.full(D, 8.0), dt)  # score gap 8*16*scale
    out, _ = run(c, dt, scale=1.0)  # gap = 128 >> 40
    for h in range(Hq):
        vstar = vals(c["v_cache"][blk, tstar % bs, h // 4], dt)
        assert np.max(np.abs(out[0, h] - vstar)) <= 1e-15 * max(1.0, np.max(np.abs(vstar)))


def test_gqa_head_mapping_is_consecutive_groups():
    c, dt = small_case(ctx=(6, 3, 8), seed=8)
    for g in range(2):
        c["v_cache"][:, :, g, :] = bits(np.full(16, g + 1.0), dt)
    out, _ = run(c, dt)
    for h in range(8):
        assert np.all(out[:, h] == (h // 4) + 1.0)


# --------------------------------------------------------------------------
# invariants

def test_block_permutation_with_consistent_table_is_bitwise_invariant():
    c, dt = small_case(ctx=(5, 9, 12), seed=9, extra_pool=5)
    out, lse = run(c, dt)
    pool = c["k_cache"].shape[0]
    perm = RNG.permutation(pool)            # new physical position of old block i
    k2 = np.empty_like(c["k_cache"]); v2 = np.empty_like(c["v_cache"])
    k2[perm] = c["k_cache"]; v2[perm] = c["v_cache"]
    c2 = dict(c, k_cache=k2, v_cache=v2, block_table=perm[c["block_table"]].astype(np.int32))
    out2, lse2 = run(c2, dt)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_output_lies_in_the_convex_hull_of_valid_values():
    c, dt = small_case(ctx=(5, 9, 12), seed=10, q_sigma=3.0)
    out, _ = run(c, dt, scale=1.0)
    for b in range(3):
        for h in range(8):
            _, V = gather(c, dt, b, h // 4)
            assert np.all(out[b, h] >= V.min(0) - 1e-12) and np.all(out[b, h] <= V.max(0) + 1e-12)


def test_linearity_in_v():
    c, dt = small_case(ctx=(5, 9, 12), seed=11)
    # V on a coarse grid so that 2V and V + 1 are exact in bf16
    grid = RNG.integers(-8, 8, size=c["v_cache"].shape) / 4.0
    c["v_cache"] = bits(grid, dt)
    out, _ = run(c, dt)
    out2, _ = run(dict(c, v_cache=bits(2 * grid, dt)), dt)
    out3, _ = run(dict(c, v_cache=bits(grid + 1.0, dt)), dt)
    assert np.array_equal(out2, 2 * out)
    assert np.max(np.abs(out3 - (out + 1.0))) <= 1e-12


def test_doubling_q_and_halving_scale_is_bitwise_invariant():
    c, dt = small_case(ctx=(5, 9, 12), seed=12)
    out, lse = run(c, dt, scale=0.5)
    q2 = bits(2 * vals(c["q"], dt), dt)
    out2, lse2 = run(dict(c, q=q2), dt, scale=0.25)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_equal_query_heads_in_a_group_give_equal_outputs():
    c, dt = small_case(ctx=(5, 9, 12), seed=13)
    c["q"][:, 1] = c["q"][:, 0]
    c["q"][:, 6] = c["q"][:, 5]
    out, _ = run(c, dt)
    assert np.array_equal(out[:, 1], out[:, 0]) and np.array_equal(out[:, 6], out[:, 5])
    assert not np.array_equal(out[:, 4], out[:, 0])


def test_poison_outside_the_valid_tokens_is_never_read():
    c, dt = small_case(ctx=(5, 9, 2), seed=14, extra_pool=4)
    out, lse = run(c, dt)
    bs = c["k_cache"].shape[1]
    nanb = bits(np.full(16, np.nan), dt)
    live = set()
    for b in range(3):
        L = int(c["context_lens"][b])
        n = -(-L // bs)
        live.update(int(x) for x in c["block_table"][b, :n])
        last = c["block_table"][b, n - 1]
        for off in range(L - (n - 1) * bs, bs):   # slots past L in the last block
            c["k_cache"][last, off] = nanb
            c["v_cache"][last, off] = nanb
        c["block_table"][b, n:] = -1              # padding entries
    for i in range(c["k_cache"].shape[0]):
        if i not in live:
            c["k_cache"][i] = nanb
            c["v_cache"][i] = nanb
    out2, lse2 = run(c, dt)
    assert np.all(np.isfinite(out2))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_empty_context_gives_zero_and_minus_infinity():
    c, dt = small_case(ctx=(0, 4, 0), seed=15)
    out, lse = run(c, dt)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(lse[1]))


def test_thread_count_does_not_change_the_bits():
    c, dt = small_case(B=4, ctx=(5, 9, 12, 3), seed=16)
    a = run(c, dt, nthreads=1)
    b = run(c, dt, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_live_block_id_outside_the_pool_is_an_error():
    c, dt = small_case(ctx=(5, 9, 12), seed=17)
    c["block_table"][1, 0] = c["k_cache"].shape[0]
    with pytest.raises(oracle.OracleError):
        run(c, dt)


def test_context_longer_than_the_table_is_an_error():
    c, dt = small_case(ctx=(5, 9, 12), seed=18)
    c["context_lens"][0] = c["block_table"].shape[1] * c["k_cache"].shape[1] + 1
    with pytest.raises(oracle.OracleError):
        run(c, dt)


# --------------------------------------------------------------------------
# split-K / LSE regrouping

@pytest.mark.parametrize("bs", [4, 8])
def test_split_merge_equals_single_pass_for_every_partition_size(bs):
    ctx = (1, 5, 16, 17, 31, 64)
    c, dt = small_case(B=len(ctx), bs=bs, ctx=ctx, seed=19)
    out, lse = run(c, dt)
    for P in range(bs, 64 + bs, bs):
        S = -(-64 // P)
        o_p, l_p = oracle.partials(c["q"], c["k_cache"], c["v_cache"], c["block_table"],
                                   c["context_lens"], scale=0.25, dtype=dt,
                                   partition_tokens=P, num_splits=S)
        merged = oracle.merge(o_p, l_p, c["context_lens"], partition_tokens=P)
        assert np.max(np.abs(merged - out)) <= 1e-12, P
        # the lse of the whole sequence is the log-sum-exp of the partition lses
        for b, L in enumerate(ctx):
            n = -(-L // P)
            assert np.all(np.isneginf(l_p[b, :, n:]))
            lp = l_p[b, :, :n]
            M = lp.max(axis=1)
            tot = M + np.log(np.exp(lp - M[:, None]).sum(axis=1))
            assert np.max(np.abs(tot - lse[b])) <= 1e-12


def test_one_partition_is_the_single_pass_bitwise():
    c, dt = small_case(ctx=(5, 9, 12), seed=20)
    out, lse = run(c, dt)
    o_p, l_p = oracle.partials(c["q"], c["k_cache"], c["v_cache"], c["block_table"],
                               c["context_lens"], scale=0.25, dtype=dt,
                               partition_tokens=12, num_splits=1)
    assert np.array_equal(o_p[:, :, 0], out) and np.array_equal(l_p[:, :, 0], lse)


# --------------------------------------------------------------------------
# a second, dense formulation (numpy gather + two-pass softmax)

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_matches_a_dense_numpy_formulation(dtype):
    c, dt = small_case(B=4, Hq=12, Hkv=3, D=32, bs=8, ctx=(1, 8, 9, 30), dtype=dtype, seed=21)
    scale = float(np.float32(0.17))
    out, lse = run(c, dt, scale=scale)
    q = vals(c["q"], dt)
    for b in range(4):
        for h in range(12):
            K, V = gather(c, dt, b, h // 4)
            s = scale * (K @ q[b, h])
            w = np.exp(s - s.max())
            ref = (w[:, None] * V).sum(0) / w.sum()
            assert np.max(np.abs(out[b, h] - ref)) <= 1e-12
            assert abs(lse[b, h] - (s.max() + np.log(w.sum()))) <= 1e-12


@pytest.mark.parametrize("Hq,Hkv,D", [(14, 2, 64), (32, 1, 64), (8, 8, 16), (20, 1, 32),
                                     (6, 2, 128), (32, 1, 128), (64, 1, 64), (128, 1, 32)])
def test_matches_the_dense_formulation_at_other_geometries(Hq, Hkv, D):
    # odd group sizes (G = 7, 20, 3), MQA (G = 32, 64, 128), MHA (G = 1), D = 16..128:
    # query head h reads KV head h // G
    G = Hq // Hkv
    c, dt = small_case(B=3, Hq=Hq, Hkv=Hkv, D=D, bs=8, ctx=(1, 9, 23), dtype="bf16", seed=G + D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = run(c, dt, scale=scale)
    q = vals(c["q"], dt)
    for b in range(3):
        for h in range(Hq):
            K, V = gather(c, dt, b, h // G)
            s_ = scale * (K @ q[b, h])
            w = np.exp(s_ - s_.max())
            ref = (w[:, None] * V).sum(0) / w.sum()
            assert np.max(np.abs(out[b, h] - ref)) <= 1e-12
            assert abs(lse[b, h] - (s_.max() + np.log(w.sum()))) <= 1e-12


# --------------------------------------------------------------------------
# regression fixture for the tiny workload (written by tests/golden/make_golden.py,
# which calls only oracle/ and workloads/)

def test_tiny_workload_matches_its_golden_fixture():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_seed0.json")
    with open(path) as f:
        gold = json.load(f)
    c = workloads.tiny(gold["seed"])
    assert c.block_table.tolist() == gold["block_table"]
    out, lse = oracle.attention_case(c)
    ref = np.array([float.fromhex(x) for x in gold["out_hex"]]).reshape(out.shape)
    assert np.max(np.abs(out - ref)) <= 1e-13
    rounded = oracle.round_to_dtype(out, "bf16")
    assert rounded.reshape(-1).tolist() == gold["out_bf16_bits"]


def test_large_logits_stay_finite_in_single_pass_and_merge():
    # scores of several hundred: exp without subtracting the running maximum
    # (in the softmax or in the partition merge) overflows fp64
    ctx = (5, 16, 29)
    c, dt = small_case(B=3, bs=4, ctx=ctx, seed=22)
    scale = 128.0
    out, lse = run(c, dt, scale=scale)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert np.max(lse) > 800.0
    q = vals(c["q"], dt)
    for b in range(3):
        for h in range(8):
            K, V = gather(c, dt, b, h // 4)
            s = scale * (K @ q[b, h])
            w = np.exp(s - s.max())
            assert np.max(np.abs(out[b, h] - (w[:, None] * V).sum(0) / w.sum())) <= 1e-12
    o_p, l_p = oracle.partials(c["q"], c["k_cache"], c["v_cache"], c["block_table"],
                               c["context_lens"], scale=scale, dtype=dt,
                               partition_tokens=8, num_splits=4)
    merged = oracle.merge(o_p, l_p, c["context_lens"], partition_tokens=8)
    assert np.max(np.abs(merged - out)) <= 1e-12


# --------------------------------------------------------------------------
# FP8 (E4M3FN) cache

def fp8_codes(x):
    """float values -> E4M3FN byte codes (torch CPU cast, RNE)."""
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def small_fp8_case(k_scale, v_scale, dtype="bf16", seed=3, **kw):
    c, _ = small_case(dtype=dtype, seed=seed, **kw)
    g = np.random.default_rng(seed + 100)
    shape = c["k_cache"].shape
    c["k_cache"] = fp8_codes(g.standard_normal(shape) * 40)
    c["v_cache"] = fp8_codes(g.standard_normal(shape) * 40)
    return c


def run_fp8(c, dtype, k_scale, v_scale, scale=0.25, **kw):
    return oracle.attention_fp8(c["q"], c["k_cache"], c["v_cache"], c["block_table"],
                                c["context_lens"], scale=scale, dtype=dtype, k_scale=k_scale,
                                v_scale=v_scale, **kw)


def test_fp8_widen_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.widen_fp8(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.nonzero(nan)[0].tolist() == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # the format's landmarks: largest finite, smallest normal and subnormal, one
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_cache_equals_the_16bit_oracle_on_the_same_values(dtype):
    # power-of-two scales keep code * scale exact in the 16-bit dtype, so the
    # FP8 path must give the 16-bit oracle's fp64 result on those values
    ks, vs = 2.0 ** -5, 2.0 ** -6
    c = small_fp8_case(ks, vs, dtype=dtype)
    c16 = dict(c)
    c16["k_cache"] = bits(oracle.widen_fp8(c["k_cache"]) * ks, dtype)
    c16["v_cache"] = bits(oracle.widen_fp8(c["v_cache"]) * vs, dtype)
    assert np.array_equal(vals(c16["k_cache"], dtype), oracle.widen_fp8(c["k_cache"]) * ks)
    assert np.array_equal(vals(c16["v_cache"], dtype), oracle.widen_fp8(c["v_cache"]) * vs)
    o8, l8 = run_fp8(c, dtype, ks, vs)
    o16, l16 = run(c16, dtype)
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)


def test_fp8_one_token_returns_its_scaled_v_exactly():
    ks, vs = 0.0123, 0.0371  # not powers of two
    c = small_fp8_case(ks, vs, ctx=(1, 1, 1))
    o, lse = run_fp8(c, "bf16", ks, vs)
    for b in range(3):
        blk = c["block_table"][b, 0]
        for h in range(8):
            v = oracle.widen_fp8(c["v_cache"][blk, 0, h // 4]) * float(np.float32(vs))
            assert np.array_equal(o[b, h], v)


def test_fp8_scales_enter_where_the_definition_puts_them():
    # two tokens: out = sigma(s0 - s1) v0 + sigma(s1 - s0) v1 with
    # s_i = scale * q . (k_i * k_scale) and v_i * v_scale
    ks, vs, scale = 0.05, 0.02, 0.3
    c = small_fp8_case(ks, vs, ctx=(2, 2, 2))
    o, _ = run_fp8(c, "bf16", ks, vs, scale=scale)
    ksf, vsf, sf = (float(np.float32(x)) for x in (ks, vs, scale))
    for b in range(3):
        blk = c["block_table"][b, 0]
        for h in range(8):
            g = h // 4
            q = vals(c["q"][b, h], "bf16")
            k = oracle.widen_fp8(c["k_cache"][blk, :2, g]) * ksf
            v = oracle.widen_fp8(c["v_cache"][blk, :2, g]) * vsf
            s = sf * (k @ q)
            w1 = 1.0 / (1.0 + math.exp(s[0] - s[1]))
            want = (1.0 - w1) * v[0] + w1 * v[1]
            assert np.allclose(o[b, h], want, rtol=1e-12, atol=1e-15)
    # swapping the two scales must change the result
    o2, _ = run_fp8(c, "bf16", vs, ks, scale=scale)
    assert not np.allclose(o, o2)


def test_fp8_nan_codes_outside_the_valid_tokens_are_never_read():
    ks, vs = 0.01, 0.01
    c = small_fp8_case(ks, vs, ctx=(5, 9, 1), extra_pool=2)
    clean, _ = run_fp8(c, "bf16", ks, vs)
    bs = c["k_cache"].shape[1]
    live = set()
    for b, L in enumerate(c["context_lens"]):
        n = -(-int(L) // bs)
        live.update(int(x) for x in c["block_table"][b, :n])
        last = c["block_table"][b, n - 1]
        c["k_cache"][last, int(L) - (n - 1) * bs:] = 0x7F
        c["v_cache"][last, int(L) - (n - 1) * bs:] = 0xFF
    for i in range(c["k_cache"].shape[0]):
        if i not in live:
            c["k_cache"][i] = 0x7F
            c["v_cache"][i] = 0xFF
    got, _ = run_fp8(c, "bf16", ks, vs)
    assert np.all(np.isfinite(got)) and np.array_equal(got, clean)


def test_fp8_split_merge_equals_single_pass():
    ks, vs = 0.013, 0.021
    c = small_fp8_case(ks, vs, ctx=(13, 20, 7))
    ref, lse = run_fp8(c, "bf16", ks, vs)
    for P in (4, 8, 12):
        S = -(-20 // P)
        o, l = oracle.partials_fp8(c["q"], c["k_cache"], c["v_cache"], c["block_table"],
                                   c["context_lens"], scale=0.25, dtype="bf16", k_scale=ks,
                                   v_scale=vs, partition_tokens=P, num_splits=S)
        got = oracle.merge(o, l, c["context_lens"], partition_tokens=P)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_fp8_workload_codes_stand_for_scaled_normal_draws():
    c = workloads.splitk(2, 256, seed=5, kv_dtype="fp8")
    for codes, scale in ((c.k_cache, c.k_scale), (c.v_cache, c.v_scale)):
        x = oracle.widen_fp8(codes) * scale
        assert np.isfinite(x).all()
        assert abs(float(np.abs(x).max()) / scale - 448.0) < 1e-9   # amax maps to the top code
        assert abs(float(x.std()) - 1.0) < 0.01
