"""GPU parity at other KV-head counts with four query heads per KV head.

The kernel serves any Hkv with Hq = 4 * Hkv and D = 128: KV heads pair up in
a workgroup only when Hkv is even, and the planner's choices change with
B * Hkv. These cases cover one, two, three, four and sixteen KV heads, with
ragged contexts that leave partial tiles, both dtypes and block sizes, the
planned split count and forced ones.
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
