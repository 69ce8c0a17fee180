"""Invariants of the split planner, checked on its internal plan fields.

The planner source is compiled on its own with g++ into a small host driver
(tests/plan_probe.cpp), so these checks see the slices and virtual heads the
C ABI does not return. No GPU."""
import itertools
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_gqa_decode_02_amd", "csrc")
MAX_WAVE_BLOCKS, MAX_WAVES = 256, 8

GEOMS = [(32, 8, 128), (32, 8, 64), (14, 2, 64), (32, 1, 128), (32, 1, 64), (8, 8, 128),
         (20, 1, 128), (64, 4, 64), (21, 1, 128), (17, 1, 64), (48, 2, 128), (64, 8, 128),
         (28, 4, 128), (40, 8, 128), (64, 1, 128), (128, 1, 64), (96, 2, 128), (40, 1, 128)]
BATCHES = (1, 2, 3, 8, 16, 32, 64, 256)
CONTEXTS = (16, 48, 1000, 1024, 4096, 9306, 20001, 65536, 131072)


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_probe")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "plan_probe.cpp"),
                    os.path.join(CSRC, "pd_plan.cpp"), "-o", exe], check=True)

    def run(rows):
        text = "".join(" ".join(str(x) for x in r) + "\n" for r in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        lines = out.stdout.split("\n")[:len(rows)]
        return [tuple(int(x) for x in ln.split()) for ln in lines]
    return run


def shapes(requests=(0,)):
    for (Hq, Hkv, D), B, L, bs, req in itertools.product(GEOMS, BATCHES, CONTEXTS, (16, 32),
                                                        requests):
        yield B, Hq, Hkv, D, -(-L // bs), bs, 1, req


def test_every_plan_tiles_the_context_within_the_kernel_limits(probe):
    rows = list(shapes(requests=(0, 1, 2, 3, 7, 64)))
    for r, (st, S, P, NH, NT, Pw, HS) in zip(rows, probe([r + (0,) for r in rows])):
        B, Hq, Hkv, D, MB, bs, _, req = r
        assert st == 0, r
        cap = MB * bs
        G = Hq // Hkv
        # virtual heads: the fewest equal parts of at most 16 query heads
        assert G % HS == 0 and G // HS <= 16, r
        assert all(G % h or G // h > 16 for h in range(1, HS)), r
        # partitions cover the context, block aligned, none empty
        assert P % bs == 0 and S * P >= cap > (S - 1) * P, r
        # slices cover a partition, block aligned, none empty, within one wave's reach
        assert Pw % bs == 0 and Pw <= MAX_WAVE_BLOCKS * bs, r
        assert NT * Pw >= P > (NT - 1) * Pw, r
        assert NH in (1, 2, 4, 8) and (Hkv * HS) % NH == 0 and NH * NT <= MAX_WAVES, r
        if req:
            # a forced S fixes P, unless the waves' reach (whole slices of 256
            # blocks) caps the partition
            want = -(-(-(-cap // req)) // bs) * bs
            assert P == want or (P < want and P % (MAX_WAVE_BLOCKS * bs) == 0), r


def test_fp8_plans_keep_the_partitions_of_the_16_bit_plan(probe):
    # the plan and workspace queries do not know the cache format: an FP8 call
    # must use the same S and P (it may cut a partition into more slices)
    rows = [r for r in shapes(requests=(0, 1, 3)) if r[3] == 128]
    a = probe([r + (0,) for r in rows])
    b = probe([r + (1,) for r in rows])
    for r, x, y in zip(rows, a, b):
        assert x[:3] == y[:3], (r, x, y)
        assert y[4] >= x[4], (r, x, y)


def test_the_planner_rejects_what_the_kernels_are_not_built_for(probe):
    rows = [(1, 32, 8, 96, 4, 16, 1, 0, 0), (1, 129, 1, 128, 4, 16, 1, 0, 0),
            (1, 32, 8, 128, 4, 8, 1, 0, 0), (1, 32, 8, 128, 4, 16, 2, 0, 0),
            (1, 30, 8, 128, 4, 16, 1, 0, 0), (65536, 32, 8, 128, 4, 16, 1, 0, 0)]
    st = [x[0] for x in probe(rows)]
    assert st == [7, 7, 7, 3, 2, 2]


def test_the_fill_target_is_one_wave_per_simd_of_a_whole_mi355x(probe):
    # the heuristic assumes 256 CUs x 4 SIMDs and does not query the device:
    # 32 sequences x 8 KV heads x 4 slices = 1,024 waves fill it, one
    # sequence fewer leaves SIMDs idle and splits the context
    rows = [(B, 32, 8, 128, 64, 16, 1, 0, 0) for B in (31, 32)]
    (st31, S31, *_), (st32, S32, *_) = probe(rows)
    assert st31 == st32 == 0
    assert S31 > 1 and S32 == 1
    # in 4-wave workgroups: B x 8 KV heads x 4 slices x S reaches 1,024
    B = 4
    (_, S, _, NH, NT, _, _), = probe([(B, 32, 8, 128, 64, 16, 1, 0, 0)])
    assert NH * NT == 4 and B * 8 * NT * S // NH >= 1024


def test_many_query_heads_per_kv_head_split_to_fill_the_gpu(probe):
    # MQA 32/1 at batch 8: 16 virtual heads in pairs fill 1,024 waves with
    # 32 partitions; 32/8 at batch 8 takes 4
    (st, S, P, NH, NT, Pw, HS), = probe([(8, 32, 1, 128, 256, 16, 1, 0, 0)])
    assert st == 0 and HS == 2 and NH == 2 and S * NT * 8 * HS // NH >= 1024 // 2
    (st, S, P, NH, NT, Pw, HS), = probe([(8, 32, 8, 128, 64, 16, 1, 0, 0)])
    assert st == 0 and S == 4


def test_unsplit_fp8_plans_with_one_kv_head_per_workgroup_take_eight_slices(probe):
    # an FP8 cache's tiles carry more work per byte: an unsplit plan with
    # one KV head per workgroup puts two waves on each SIMD (eight slices);
    # the 16-bit plan of the same shape keeps four, and a split FP8 plan
    # keeps four as well
    ragged = (32, 32, 8, 128, 32, 32, 1, 0)        # contexts up to 1,024, block 32
    uniform = (32, 32, 8, 128, 64, 16, 1, 0)       # B32 ctx1024
    split = (8, 32, 8, 128, 64, 16, 1, 0)          # B8 ctx1024: S = 4
    short = (1, 32, 8, 128, 4, 16, 1, 0)           # 64 tokens: four blocks
    rows = probe([r + (fp8,) for r in (ragged, uniform, split, short) for fp8 in (0, 1)])
    (r16, r8), (u16, u8), (s16, s8), (t16, t8) = zip(rows[::2], rows[1::2])
    for a, b in ((r16, r8), (u16, u8)):
        assert a[1] == b[1] == 1 and a[2] == b[2], (a, b)   # same S and P
        assert a[3] == b[3] == 1 and a[4] == 4 and b[4] == 8, (a, b)
        assert b[5] * b[4] == b[2], b                       # eight equal slices
    assert s16[1] == s8[1] > 1 and s16[4] == s8[4] == 4, (s16, s8)
    assert t8[4] == t16[4] == 4, (t16, t8)                  # a slice is at least a block


def test_split_plans_keep_the_merge_grid_within_int32(probe):
    # the merge kernel takes one workgroup per (sequence, query head): a
    # split whose B x Hq passes INT32_MAX is refused (PD_ERR_SHAPE), the
    # unsplit plan of the same shape is not
    big = (65535, 4096 * 16, 4096, 128, 4, 16, 1)
    (st1, S1, *_), (st2, *_), (st3, S3, *_) = probe(
        [big + (0, 0), big + (2, 0), (65535, 8, 1, 128, 4, 16, 1, 2, 0)])
    assert st1 == 0 and S1 == 1
    assert st2 == 2
    assert st3 == 0 and S3 == 2


def test_small_split_batches_spread_over_more_cus(probe):
    # B1 ctx1024: 8 KV heads x 4 slices would stop at S = 8 (two tiles per
    # wave), 64 workgroups; two-wave workgroups reach S = 16, 128
    # workgroups, the same 256 waves on twice the CUs. B1 ctx2048 keeps its
    # 16 partitions (more would take a second merge batch) and B4 ctx1024
    # already has a workgroup per CU.
    rows = probe([(1, 32, 8, 128, 64, 16, 1, 0, 0), (1, 32, 8, 128, 128, 16, 1, 0, 0),
                  (4, 32, 8, 128, 64, 16, 1, 0, 0), (2, 32, 8, 128, 32, 16, 1, 0, 0)])
    (st1, S1, P1, NH1, NT1, *_), (st2, S2, _, NH2, NT2, *_), (st3, S3, _, NH3, NT3, *_), \
        (st4, S4, _, NH4, NT4, *_) = rows
    assert st1 == st2 == st3 == st4 == 0
    assert (S1, NH1, NT1) == (16, 1, 2) and P1 == 64
    assert (S2, NH2, NT2) == (16, 1, 4)
    assert (S3, NH3, NT3) == (8, 1, 4)
    assert (S4, NH4, NT4) == (8, 1, 2)      # B2 ctx512: 64 -> 128 workgroups
