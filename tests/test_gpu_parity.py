"""GPU parity: the HIP library against the fp64 oracle on every workload.

Workloads are the pages' sweeps (Loom Kernels benchmark page, "Reproduce":
the paged-decode backend sweep and the split-K sweep; "What the ratios mean":
short-context route and D128 long-context split-K/LSE path) plus the ragged
and bandwidth-bound cases, all at Hq/Hkv 32/8, D 128. Each call goes through
the C ABI via the ctypes binding; the tolerance gates are in helpers.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_case, compare, device_case, out_bits, run_library

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


def test_tiny():
    c = workloads.tiny(0)
    note(c.describe())
    check_case(c)


@pytest.mark.parametrize("case", list(workloads.short_cases(0)), ids=lambda c: c.name)
def test_short_context_sweep(case):
    note(case.describe())
    check_case(case)


SPLITK = list(workloads.splitk_cases(0))


@pytest.mark.parametrize("case", SPLITK, ids=lambda c: c.name)
def test_split_k_sweep_planned(case):
    import paged_gqa_decode_02_amd as pd
    S, P = pd.paged_decode_plan(case.B, 32, 8, 128, case.max_blocks_per_seq, 16, torch.bfloat16)
    note(f"{case.describe()} plan S={S} P={P}")
    check_case(case)


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 5, 8, 13, 16, 64])
@pytest.mark.parametrize("B,L", [(1, 1024), (2, 256), (8, 128), (4, 512)])
def test_split_k_forced_split_counts(B, L, splits):
    c = workloads.splitk(B, L, seed=7)
    note(f"{c.describe()} forced S={splits}")
    check_case(c, num_splits=splits, what=f"{c.name} S={splits}")


def test_ragged_batch():
    c = workloads.ragged(0)
    note(c.describe())
    check_case(c)


@pytest.mark.parametrize("splits", [1, 3, 8, 32])
def test_ragged_batch_forced_splits(splits):
    c = workloads.ragged(1)
    note(f"{c.describe()} S={splits}")
    check_case(c, num_splits=splits, what=f"ragged S={splits}")


def test_large_bandwidth_bound_full_size():
    c = workloads.large(0)
    note(c.describe())
    check_case(c)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bs", [16, 32])
def test_odd_lengths_every_tail(dtype, bs):
    # contexts hitting every residue of the block size and of the 8-token step
    lens = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 300]
    c = workloads.make_case(f"tails_{dtype}_bs{bs}", len(lens), lens, dtype=dtype,
                            block_size=bs, seed=11)
    note(c.describe())
    for s in (None, 1, 2, 5):
        check_case(c, num_splits=s, what=f"{c.name} S={s}")


def test_empty_contexts_give_zero_rows():
    lens = [0, 5, 0, 300, 0]
    c = workloads.make_case("empty_mix", len(lens), lens, dtype="bf16", block_size=16, seed=12,
                            max_blocks_per_seq=32)
    note(c.describe())
    for s in (None, 1, 4):
        out = run_library(c, num_splits=s)
        b = out_bits(out)
        assert np.all(b[[0, 2, 4]] == 0)
        ref, _ = oracle.attention_case(c)
        compare(b, ref, "bf16", what=f"empty_mix S={s}")


# ---------------------------------------------------------------------------
# invariants the oracle is pinned to, now held bitwise by the GPU


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_token_context_returns_v_bitwise(dtype):
    c = workloads.make_case("one_token", 8, 1, dtype=dtype, block_size=16, seed=13,
                            max_blocks_per_seq=4)
    out = out_bits(run_library(c))
    for b in range(8):
        blk = c.block_table[b, 0]
        for h in range(32):
            assert np.array_equal(out[b, h], c.v_cache[blk, 0, h // 4])


def test_constant_v_returns_the_constant_bitwise():
    c = workloads.make_case("const_v", 4, [17, 64, 200, 1000], dtype="bf16", block_size=16,
                            seed=14)
    row = c.v_cache[0, 0, 0].copy()
    c.v_cache[:] = row
    for s in (None, 1, 7):
        out = out_bits(run_library(c, num_splits=s))
        assert np.all(out == row[None, None, :]), s


def test_block_permutation_is_bitwise_invariant():
    c = workloads.make_case("perm", 6, [40, 129, 1, 77, 256, 33], dtype="bf16", block_size=16,
                            seed=15)
    base = out_bits(run_library(c))
    rng = np.random.default_rng(0)
    perm = rng.permutation(c.num_blocks)
    c.k_cache[perm] = c.k_cache.copy()
    c.v_cache[perm] = c.v_cache.copy()
    c.block_table[:] = perm[c.block_table]
    assert np.array_equal(out_bits(run_library(c)), base)


def test_repeated_calls_are_bitwise_identical():
    c = workloads.ragged(2)
    dev = device_case(c)
    import paged_gqa_decode_02_amd as pd
    outs = []
    for _ in range(5):
        outs.append(out_bits(pd.paged_decode_attention(*dev, scale=c.scale)))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_poison_outside_the_valid_tokens_is_never_read():
    lens = [5, 16, 17, 100, 1]
    c = workloads.make_case("poison", len(lens), lens, dtype="bf16", block_size=16, seed=16,
                            max_blocks_per_seq=10)
    clean = out_bits(run_library(c))
    nan = np.uint16(0x7FC0)
    live = set()
    for b, L in enumerate(lens):
        n = -(-L // 16)
        live.update(int(x) for x in c.block_table[b, :n])
        last = c.block_table[b, n - 1]
        c.k_cache[last, L - (n - 1) * 16:] = nan
        c.v_cache[last, L - (n - 1) * 16:] = nan
    dead = [i for i in range(c.num_blocks) if i not in live]
    assert dead
    for i in dead:
        c.k_cache[i] = nan
        c.v_cache[i] = nan
    for b, L in enumerate(lens):   # padding entries point at a NaN block (a valid id)
        c.block_table[b, -(-L // 16):] = dead[0]
    for s in (None, 1, 3):
        got = out_bits(run_library(c, num_splits=s))
        ref, _ = oracle.attention_case(c)
        compare(got, ref, "bf16", what=f"poison S={s}")
        if s is None:
            assert np.array_equal(got, clean)


@pytest.mark.parametrize("where", ["first", "block_last", "block_first", "partition_edge", "last"])
def test_needle(where):
    L, bs = 1000, 16
    c = workloads.make_case("needle", 2, L, dtype="bf16", block_size=bs, seed=17)
    S, P = 4, None
    import paged_gqa_decode_02_amd as pd
    S, P = pd.paged_decode_plan(2, 32, 8, 128, c.max_blocks_per_seq, bs, torch.bfloat16,
                                num_splits=4)
    t = {"first": 0, "block_last": 5 * bs - 1, "block_first": 7 * bs, "partition_edge": P - 1,
         "last": L - 1}[where]
    c.k_cache[:] = 0
    one = np.uint16(0x3F80)  # 1.0 in bf16
    c.q[:] = one
    for b in range(2):
        blk = c.block_table[b, t // bs]
        c.k_cache[blk, t % bs] = np.uint16(0x4100)  # 8.0: score 8*128*scale = 90.5
    for s in (None, 1, 4, 7):
        out = out_bits(run_library(c, num_splits=s))
        for b in range(2):
            blk = c.block_table[b, t // bs]
            for h in range(32):
                assert np.array_equal(out[b, h], c.v_cache[blk, t % bs, h // 4]), (where, s, b, h)


RAMPS = {0.02: [1000, 777, 16, 1024], 0.05: [1000, 777, 16, 1024],
         0.6: [300, 77, 16, 64], -0.03: [1000, 777, 16, 1024]}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("slope", sorted(RAMPS))
def test_scores_that_rise_or_fall_through_the_context(dtype, slope):
    # All query heads of a sequence share q0 and token t's key is a multiple
    # of q0, so every score is close to slope * t - c (plus a little noise,
    # c the largest slope * t): the maximum then keeps rising by less than a
    # tile's worth, or by much more (0.6 per token, about 14 in log2 units
    # per tile), or falls. The kernel's softmax reference lags the running
    # maximum, its weights grow up to their bound between moves; the result
    # must not depend on that. The shift keeps the scores that carry weight
    # near 0: scores of 60 and more carry the fp32 rounding of their dot
    # products (about 1e-5 of a score) past the 1-ulp gate on outputs that
    # cancel to near zero, in any fp32 evaluation.
    lens = RAMPS[slope]
    c = workloads.make_case(f"ramp_{dtype}_{slope}", len(lens), lens, dtype=dtype,
                            block_size=16, seed=21)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    widen = lambda bits: torch.from_numpy(bits.view(np.int16)).view(tdt).float()
    pack = lambda x: x.to(tdt).view(torch.int16).numpy().view(np.uint16)
    rng = np.random.default_rng(5)
    for b, L in enumerate(lens):
        q0 = widen(c.q[b, 0])
        c.q[b] = c.q[b, 0][None, :]
        unit = q0 / (float(c.scale) * float((q0 * q0).sum()))
        top = max(slope * t for t in range(L))
        for t in range(L):
            blk, off = c.block_table[b, t // 16], t % 16
            for g in range(c.Hkv):
                noise = torch.from_numpy(rng.normal(0, 0.01, c.D).astype(np.float32))
                c.k_cache[blk, off, g] = pack((slope * t - top) * unit + noise)
    for s in (None, 1, 3):
        check_case(c, num_splits=s, what=f"{c.name} S={s}")
