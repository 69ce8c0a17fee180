"""Small split batches against the fp64 oracle: batches of 1 to 4 sequences,
whose plans run two-wave workgroups and up to 16 partitions (a split that
would leave CUs without a workgroup spreads its waves over more of them),
at 32/8, 14/2 D64 and 32/2 (16 query heads per KV head), block sizes 16 and
32, 16-bit and FP8 caches, with ragged lengths that leave some partitions
empty and some sequences empty. Each case prints its description and plan
before it runs."""
import math

import numpy as np
import pytest
import torch

import paged_gqa_decode_02_amd as pd
import workloads
from helpers import check_case

pytestmark = pytest.mark.gpu

GEOMS = [(32, 8, 128), (14, 2, 64), (32, 2, 128)]


@pytest.mark.parametrize("kv", ["", "fp8"])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: f"{g[0]}x{g[1]}_D{g[2]}")
@pytest.mark.parametrize("B,cap", [(1, 512), (1, 1024), (2, 512), (2, 1024), (3, 2048), (4, 512)])
def test_small_split_batch_matches_the_oracle(B, cap, geom, bs, kv):
    Hq, Hkv, D = geom
    rng = np.random.default_rng(B * 7919 + cap + bs + Hq)
    lens = rng.integers(1, cap + 1, size=B)
    lens[0] = cap                                  # one full row
    if B > 2:
        lens[-1] = 0                               # and an empty one
    case = workloads.make_case(f"small_B{B}_cap{cap}_{Hq}x{Hkv}_D{D}_bs{bs}{'_' + kv if kv else ''}",
                               B, lens.astype(np.int32), Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                               block_size=bs, seed=B + cap + bs, max_blocks_per_seq=cap // bs,
                               scale=float(np.float32(1.0 / math.sqrt(D))), kv_dtype=kv)
    S, P = pd.paged_decode_plan(B, Hq, Hkv, D, cap // bs, bs, torch.bfloat16)
    print(case.describe(), "plan S", S, "P", P, flush=True)
    check_case(case)
