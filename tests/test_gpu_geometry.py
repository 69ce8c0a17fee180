"""GPU parity at other head geometries.

First, other KV-head counts with four query heads per KV head: KV heads pair
up in a workgroup only when Hkv is even, and the planner's choices change
with B * Hkv (one, two, three, four and sixteen KV heads). Then other group
sizes and head dims: the Qwen2.5-style 14/2 at D 64, MQA 32/1 (two virtual
KV heads of 16), MHA (G = 1), G = 2, 3, 5, 8, 16, 20, up to 128 (eight
virtual KV heads) and D 64 at 32/8. All
with ragged (and empty) contexts that leave partial tiles, both dtypes and
block sizes, the planned split count and forced ones.
"""
import pytest
import torch

import workloads
from helpers import check_case

pytestmark = pytest.mark.gpu


GEOMETRIES = [(1, "bf16", 16), (2, "f16", 32), (3, "bf16", 32), (4, "f16", 16), (16, "bf16", 16)]


@pytest.mark.parametrize("hkv,dtype,bs", GEOMETRIES)
@pytest.mark.parametrize("splits", [None, 1, 3])
def test_kv_head_counts(hkv, dtype, bs, splits):
    lens = [1, 37, 700, 1024, 513]
    c = workloads.make_case(f"heads_{4 * hkv}x{hkv}_{dtype}_bs{bs}", len(lens), lens, dtype=dtype,
                            block_size=bs, Hq=4 * hkv, Hkv=hkv, seed=60 + hkv)
    print(f"{c.describe()} S={splits}", flush=True)
    check_case(c, num_splits=splits, what=f"{c.name} S={splits}")


@pytest.mark.parametrize("hkv", [2, 16])
def test_many_sequences_pair_kv_heads(hkv):
    # enough sequences that the planner pairs KV heads (B * Hkv >= 512)
    B = 512 // hkv
    c = workloads.make_case(f"pairs_{hkv}", B, 160, dtype="bf16", block_size=16, Hq=4 * hkv,
                            Hkv=hkv, seed=70 + hkv)
    import paged_gqa_decode_02_amd as pd
    S, P = pd.paged_decode_plan(B, 4 * hkv, hkv, 128, c.max_blocks_per_seq, 16, torch.bfloat16)
    print(f"{c.describe()} plan S={S} P={P}", flush=True)
    check_case(c)


def test_f16_block32_long_contexts():
    c = workloads.make_case("f16_bs32_long", 16, [4096, 3000, 1, 2048] * 4, dtype="f16",
                            block_size=32, seed=80)
    print(c.describe(), flush=True)
    check_case(c)


# ---------------------------------------------------------------------------
# other geometries: head dim 64, odd group sizes (14/2 -> 7), MQA (32/1), MHA

import numpy as np

OTHER = [
    # Hq, Hkv, D, dtype, bs
    (14, 2, 64, "bf16", 16),    # the pages' 14/2 D64 route
    (14, 2, 128, "f16", 32),
    (32, 1, 128, "bf16", 16),   # MQA
    (32, 1, 64, "f16", 16),
    (8, 8, 128, "bf16", 32),    # MHA, G = 1
    (16, 8, 64, "bf16", 16),    # G = 2
    (24, 8, 128, "f16", 16),    # G = 3
    (40, 8, 128, "bf16", 16),   # G = 5
    (64, 8, 128, "bf16", 32),   # G = 8
    (32, 2, 64, "f16", 32),     # G = 16
    (20, 1, 128, "bf16", 16),   # G = 20: two virtual KV heads of 10
    (32, 8, 64, "bf16", 16),    # D = 64 at the 32/8 grouping
    (21, 1, 128, "f16", 16),    # G = 21: three virtual KV heads of 7 (odd split)
    (17, 1, 64, "bf16", 32),    # G = 17 (prime): 17 virtual KV heads of 1
    (48, 2, 128, "bf16", 16),   # G = 24: two virtual KV heads of 12, two KV heads
    (64, 1, 128, "bf16", 16),   # G = 64: four virtual KV heads of 16
    (128, 1, 64, "f16", 32),    # G = 128: eight virtual KV heads of 16
    (96, 2, 128, "bf16", 16),   # G = 48: three virtual KV heads of 16, two KV heads
    (40, 1, 128, "f16", 16),    # G = 40: four virtual KV heads of 10
    (12, 2, 128, "bf16", 16),   # G = 6
    (72, 8, 128, "bf16", 32),   # G = 9
    (11, 1, 128, "bf16", 16),   # G = 11 (prime, one wave of 11 heads)
    (30, 2, 64, "f16", 16),     # G = 15
    (33, 1, 64, "bf16", 16),    # G = 33: three virtual KV heads of 11
    (100, 1, 128, "f16", 16),   # G = 100: ten virtual KV heads of 10
]


def other_case(Hq, Hkv, D, dtype, bs, lens, seed, name="geom"):
    return workloads.make_case(f"{name}_{Hq}x{Hkv}_D{D}_{dtype}_bs{bs}", len(lens), lens,
                               dtype=dtype, block_size=bs, Hq=Hq, Hkv=Hkv, D=D, seed=seed,
                               scale=float(np.float32(1.0 / np.sqrt(D))))


@pytest.mark.parametrize("Hq,Hkv,D,dtype,bs", OTHER)
@pytest.mark.parametrize("splits", [None, 1, 3])
def test_other_geometries(Hq, Hkv, D, dtype, bs, splits):
    lens = [1, 37, 700, 1024, 513, 0, 16]
    c = other_case(Hq, Hkv, D, dtype, bs, lens, seed=Hq + 3 * Hkv + D)
    print(f"{c.describe()} S={splits}", flush=True)
    check_case(c, num_splits=splits, what=f"{c.name} S={splits}")


@pytest.mark.parametrize("Hq,Hkv,D,B,L", [(14, 2, 64, 32, 1024), (32, 1, 128, 8, 4096),
                                          (32, 1, 64, 64, 512), (14, 2, 64, 1, 4096),
                                          (64, 8, 128, 16, 2048)])
def test_other_geometries_planned_long(Hq, Hkv, D, B, L):
    c = other_case(Hq, Hkv, D, "bf16", 16, [L] * B, seed=B + L, name="long")
    import paged_gqa_decode_02_amd as pd
    S, P = pd.paged_decode_plan(B, Hq, Hkv, D, c.max_blocks_per_seq, 16, torch.bfloat16)
    print(f"{c.describe()} plan S={S} P={P}", flush=True)
    check_case(c)


@pytest.mark.parametrize("Hq,Hkv,D", [(14, 2, 64), (32, 1, 128)])
def test_bench_geometry_workloads_full_size(Hq, Hkv, D):
    # the bench's B64 x 4,096-token geometry workloads, at the planned split
    # count the bench times, every output against the oracle
    c = workloads.geometry(Hq, Hkv, D, 64, 4096, seed=0)
    print(c.describe(), flush=True)
    check_case(c)


@pytest.mark.parametrize("lens,dtype,bs,kv", [([32768, 20001], "bf16", 16, ""),
                                            ([65536], "f16", 32, ""),
                                            ([40000, 1, 12345], "bf16", 16, ""),
                                            ([32768, 7000], "bf16", 16, "fp8")])
@pytest.mark.parametrize("splits", [None, 1])
def test_long_contexts(lens, dtype, bs, kv, splits):
    # contexts past what one workgroup's slices cover (8 waves x 256 blocks):
    # the plan adds partitions even when one is asked for
    c = workloads.make_case(f"long_{max(lens)}_{dtype}_bs{bs}{'_' + kv if kv else ''}", len(lens),
                            lens, dtype=dtype, block_size=bs, seed=len(lens) + bs, kv_dtype=kv)
    import paged_gqa_decode_02_amd as pd
    S, P = pd.paged_decode_plan(c.B, c.Hq, c.Hkv, c.D, c.max_blocks_per_seq, bs,
                                workloads.DTYPES[dtype], splits)
    print(f"{c.describe()} S={S} P={P}", flush=True)
    assert S * P >= max(lens)
    check_case(c, num_splits=splits, what=f"{c.name} S={splits}")
