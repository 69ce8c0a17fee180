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
