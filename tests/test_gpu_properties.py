"""GPU checks against closed forms and invariants that need no oracle.

Attention with all scores equal (K = 0, or q = 0) is the plain mean of
exactly the valid tokens' values, so a masking, tail or partition error
shows at once (an extra or missing token moves the mean); query heads of
one KV head with equal q must give bitwise-equal outputs (GQA packing, the
column copies of a wave and the virtual KV heads of a large group); and every
output lies between the smallest and largest valid value of its dim (a
convex combination). Ragged contexts with partial tiles and an empty one,
planned and forced split counts, 16-bit and FP8 caches, several geometries.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import compare, out_bits, run_library

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 100, 255, 256, 1000, 0, 33]

GEOMS = [(32, 8, 128, "bf16", 16, ""), (32, 8, 128, "f16", 32, ""), (14, 2, 64, "bf16", 16, ""),
         (32, 1, 128, "f16", 16, ""), (21, 1, 128, "bf16", 32, ""), (17, 1, 64, "bf16", 16, ""),
         (32, 8, 128, "bf16", 16, "fp8"), (32, 1, 128, "f16", 32, "fp8"),
         (64, 1, 128, "bf16", 16, ""), (128, 1, 64, "f16", 16, "fp8")]


def make(Hq, Hkv, D, dtype, bs, kv, seed, lens=LENS):
    return workloads.make_case(f"prop_{Hq}x{Hkv}_D{D}_{dtype}_bs{bs}{'_' + kv if kv else ''}",
                               len(lens), lens, dtype=dtype, block_size=bs, Hq=Hq, Hkv=Hkv, D=D,
                               seed=seed, scale=float(np.float32(1.0 / np.sqrt(D))), kv_dtype=kv)


def values(c):
    """The cache's V values in fp64 (FP8 codes times v_scale)."""
    if c.fp8:
        return oracle.widen_fp8(c.v_cache) * float(c.v_scale)
    return oracle.widen(c.v_cache, c.dtype)


def valid_rows(c, V, b, g):
    L = int(c.context_lens[b])
    t = np.arange(L)
    return V[c.block_table[b, t // c.block_size], t % c.block_size, g]


def geom_id(x):
    Hq, Hkv, D, dtype, bs, kv = x
    return f"{Hq}x{Hkv}_D{D}_{dtype}_bs{bs}{'_' + kv if kv else ''}"


@pytest.mark.parametrize("zero", ["k", "q"])
@pytest.mark.parametrize("splits", [None, 1, 3])
@pytest.mark.parametrize("geom", GEOMS, ids=geom_id)
def test_equal_scores_give_the_mean_of_exactly_the_valid_tokens(geom, splits, zero):
    c = make(*geom, seed=31)
    if zero == "k":
        c.k_cache[:] = 0
    else:
        c.q[:] = 0
    V = values(c)
    G = c.Hq // c.Hkv
    mean = np.zeros((c.B, c.Hq, c.D))
    for b in range(c.B):
        if c.context_lens[b] == 0:
            continue  # an empty context gives a zero row
        for h in range(c.Hq):
            mean[b, h] = valid_rows(c, V, b, h // G).mean(axis=0)
    got = out_bits(run_library(c, num_splits=splits))
    compare(got, mean, c.dtype, what=f"{c.name} zero {zero} S={splits}")


@pytest.mark.parametrize("splits", [None, 1, 4])
@pytest.mark.parametrize("geom", GEOMS, ids=geom_id)
def test_equal_query_heads_of_a_kv_head_give_bitwise_equal_outputs(geom, splits):
    c = make(*geom, seed=32)
    G = c.Hq // c.Hkv
    for g in range(c.Hkv):
        c.q[:, g * G:(g + 1) * G] = c.q[:, g * G:g * G + 1]
    got = out_bits(run_library(c, num_splits=splits))
    for g in range(c.Hkv):
        block = got[:, g * G:(g + 1) * G]
        assert np.array_equal(block, np.broadcast_to(block[:, :1], block.shape)), (g, splits)


@pytest.mark.parametrize("splits", [None, 1, 5])
@pytest.mark.parametrize("geom", GEOMS, ids=geom_id)
def test_outputs_lie_within_the_range_of_the_valid_values(geom, splits):
    c = make(*geom, seed=33)
    V = values(c)
    G = c.Hq // c.Hkv
    got = out_bits(run_library(c, num_splits=splits))
    g_val = oracle.widen(got, c.dtype)
    ulp = 2.0 ** -7 if c.dtype == "bf16" else 2.0 ** -10
    for b in range(c.B):
        if c.context_lens[b] == 0:
            assert np.all(got[b] == 0)
            continue
        for g in range(c.Hkv):
            rows = valid_rows(c, V, b, g)
            lo, hi = rows.min(axis=0), rows.max(axis=0)
            # one rounding to the dtype may step past the range by half an ulp
            slack = ulp * np.maximum(np.abs(lo), np.abs(hi)) + 1e-30
            x = g_val[b, g * G:(g + 1) * G]
            assert np.all(x >= lo - slack) and np.all(x <= hi + slack), (b, g, splits)


@pytest.mark.parametrize("splits", [None, 1, 3])
@pytest.mark.parametrize("geom", [GEOMS[0], GEOMS[3], GEOMS[6]], ids=geom_id)
def test_lengths_outside_the_row_count_as_its_bounds(geom, splits):
    # a length above the row's capacity (max_blocks_per_seq * block_size) is
    # taken as the capacity and a negative one as 0: the outputs equal those
    # of the lengths at the bounds, and nothing of the call lingers in the
    # split workspace (the same workspace then gives the in-range call's bits
    # again)
    import torch
    import paged_gqa_decode_02_amd as pd
    Hq, Hkv, D, dtype, bs, kv = geom
    MB = 6
    cap = MB * bs
    c = workloads.make_case(f"bounds_{Hq}x{Hkv}_{dtype}_bs{bs}{'_' + kv if kv else ''}", 5,
                            [cap, cap, 7, 0, cap - 1], dtype=dtype, block_size=bs, Hq=Hq,
                            Hkv=Hkv, D=D, seed=91, max_blocks_per_seq=MB,
                            scale=float(np.float32(1.0 / np.sqrt(D))), kv_dtype=kv)
    print(f"{c.describe()} S={splits}", flush=True)
    from helpers import device_case
    q, k, v, bt, cl = device_case(c)
    ws = pd.alloc_workspace(q, k, bt, splits)

    def call(lens):
        out = torch.full_like(q, float("nan"))
        if kv:
            pd.paged_decode_attention_fp8(q, k, v, bt, lens, out, k_scale=c.k_scale,
                                          v_scale=c.v_scale, scale=c.scale, workspace=ws,
                                          num_splits=splits)
        else:
            pd.paged_decode_attention(q, k, v, bt, lens, out, scale=c.scale, workspace=ws,
                                      num_splits=splits)
        torch.cuda.synchronize()
        return out_bits(out)

    base = call(cl)
    ref, _ = oracle.attention_case(c)
    compare(base, ref, c.dtype, what=c.name)
    wild = torch.tensor([cap + 17, 2**31 - 1, 7, -7, cap - 1], dtype=torch.int32, device="cuda")
    assert np.array_equal(call(wild), base)
    assert np.array_equal(call(cl), base)
