"""A seeded sweep of random valid shapes against the fp64 oracle: batch,
head geometry (GQA, odd groups, MQA-like groups up to 64 query heads per KV
head), head dim 64 or 128, block size 16 or 32, f16 or bf16, 16-bit or FP8
cache, ragged context lengths that include empty sequences and full rows,
spare block-table capacity, and the planned or a forced split count. Each
case prints its description before it runs. Sizes stay small enough for the
oracle to finish each case in well under a second."""
import math

import numpy as np
import pytest

import workloads
from helpers import check_case

pytestmark = pytest.mark.gpu

GEOMETRIES = [(32, 8), (14, 2), (8, 8), (28, 4), (40, 2), (32, 1), (64, 1), (12, 3), (6, 1),
              (48, 16)]


def random_case(i):
    rng = np.random.default_rng(1000 + i)
    Hq, Hkv = GEOMETRIES[rng.integers(len(GEOMETRIES))]
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    B = int(rng.integers(1, 13))
    cap_blocks = int(rng.integers(1, 65))            # up to 2,048 tokens at block size 32
    MB = cap_blocks + int(rng.integers(0, 4))         # spare table capacity
    cap = cap_blocks * bs
    kind = rng.integers(4)
    if kind == 0:
        lens = np.full(B, cap)
    elif kind == 1:
        lens = rng.integers(0, cap + 1, size=B)
    else:
        lens = rng.integers(1, cap + 1, size=B)
        lens[rng.integers(B)] = 0 if kind == 2 else cap
    dtype = str(rng.choice(["bf16", "f16"]))
    kv = "fp8" if rng.random() < 0.3 else ""
    splits = None if rng.random() < 0.5 else int(rng.integers(1, 40))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    case = workloads.make_case(f"rand{i}", B, lens.astype(np.int32), Hq=Hq, Hkv=Hkv, D=D,
                               dtype=dtype, block_size=bs, seed=2000 + i, max_blocks_per_seq=MB,
                               scale=scale, kv_dtype=kv)
    return case, splits


@pytest.mark.parametrize("i", range(48))
def test_random_shape_matches_the_oracle(i):
    case, splits = random_case(i)
    print(case.describe(), "splits", splits, flush=True)
    check_case(case, num_splits=splits)
