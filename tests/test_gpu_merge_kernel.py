"""The LSE merge kernel that every split call queues after the decode
kernel, against the fp64 oracle: planned MQA shapes (many query heads per KV
head, many partitions), forced partition counts up to 64 over a ragged
batch, ragged and empty contexts, an FP8 cache, lengths outside the row, and
a HIP graph holding both kernels replayed with the context lengths
rewritten between replays."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_02_amd as pd
import workloads
from helpers import check_case, compare, device_case, out_bits, run_library

pytestmark = pytest.mark.gpu


def planned_splits(case, splits=None):
    """The partition count S the call will use (S > 1: the merge kernel runs)."""
    S, _ = pd.paged_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.max_blocks_per_seq,
                                case.block_size, workloads.DTYPES[case.dtype], splits)
    return S


@pytest.mark.parametrize("Hq,Hkv,D,B,L", [(32, 1, 128, 8, 4096), (32, 1, 64, 4, 2048),
                                          (64, 1, 128, 2, 1024), (40, 2, 128, 3, 3000)])
def test_planned_mqa_splits_through_the_merge_kernel(Hq, Hkv, D, B, L):
    case = workloads.geometry(Hq, Hkv, D, B, L, seed=Hq + D + B)
    S = planned_splits(case)
    print(case.describe(), "S", S, flush=True)
    assert S > 1
    check_case(case)


@pytest.mark.parametrize("splits", [9, 16, 17, 40, 64])
def test_forced_splits_over_a_ragged_batch(splits):
    # 32/8, contexts from empty to full: most sequences leave partitions empty
    case = workloads.make_case("mk_ragged", 5, [1024, 1, 333, 0, 1000], dtype="bf16",
                               block_size=16, seed=splits, max_blocks_per_seq=64)
    print(case.describe(), "splits", splits, flush=True)
    check_case(case, num_splits=splits)


def test_fp8_cache_through_the_merge_kernel():
    case = workloads.geometry(32, 1, 128, 4, 2048, seed=77, kv_dtype="fp8")
    S = planned_splits(case)
    print(case.describe(), "S", S, flush=True)
    assert S > 1
    check_case(case)


def test_lengths_outside_the_row_are_clamped_by_the_merge_kernel():
    # the merge kernel takes a length above the row's capacity as the
    # capacity and a negative one as 0, like the decode kernel
    case = workloads.geometry(32, 1, 128, 3, 1024, seed=78)
    q, k, v, bt, cl = device_case(case)
    cap = case.max_blocks_per_seq * case.block_size
    cl.copy_(torch.tensor([cap + 5000, -3, 2 ** 31 - 1], dtype=torch.int32))
    out = pd.paged_decode_attention(q, k, v, bt, cl, scale=case.scale, num_splits=32)
    torch.cuda.synchronize()
    case.context_lens[:] = [cap, 0, cap]
    ref, _ = oracle.attention_case(case)
    compare(out_bits(out), ref, case.dtype, what="clamped lengths")


def test_graph_with_both_kernels_reads_lengths_at_replay():
    case = workloads.make_case("mk_graph", 4, [4000, 2500, 4096, 1], Hq=32, Hkv=1, D=128,
                               dtype="bf16", block_size=16, seed=79, max_blocks_per_seq=256,
                               scale=float(np.float32(1 / math.sqrt(128))))
    S = planned_splits(case)
    print(case.describe(), "S", S, flush=True)
    assert S > 1
    q, k, v, bt, cl = device_case(case)
    out = torch.empty_like(q)
    ws = pd.alloc_workspace(q, k, bt)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pd.paged_decode_attention(q, k, v, bt, cl, out, scale=case.scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pd.paged_decode_attention(q, k, v, bt, cl, out, scale=case.scale, workspace=ws)
    rng = np.random.default_rng(6)
    for rep in range(5):
        lens = rng.integers(0 if rep == 2 else 1, 4097, size=4).astype(np.int32)
        cl.copy_(torch.from_numpy(lens))
        g.replay()
        torch.cuda.synchronize()
        got = out_bits(out)
        eager = out_bits(pd.paged_decode_attention(q, k, v, bt, cl, scale=case.scale,
                                                   workspace=pd.alloc_workspace(q, k, bt)))
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), rep
        case.context_lens[:] = lens
        ref, _ = oracle.attention_case(case)
        compare(got, ref, "bf16", what=f"merge-kernel graph replay {rep}")


def test_merge_kernel_results_are_bitwise_stable():
    case = workloads.geometry(32, 1, 128, 8, 4096, seed=80)
    dev = device_case(case)
    a = out_bits(run_library(case, dev=dev))
    for _ in range(3):
        assert np.array_equal(out_bits(run_library(case, dev=dev)), a)


@pytest.mark.parametrize("splits", [2, 3, 4, 5, 8, 9, 16, 17, 33])
@pytest.mark.parametrize("kv", ["", "fp8"])
def test_every_merge_batch_ignores_what_empty_partitions_hold(splits, kv):
    # the merge kernel loads its first batch over all S rows before it knows
    # the length, and drops the rows of empty partitions by selects: with
    # the workspace filled with NaN bytes before every call, batches of 4,
    # 8 and 16 (and a second batch past 16) must still give the oracle's
    # rows, for contexts that leave most partitions empty
    lens = [1024, 1, 333, 0, 1000, 17, 512, 64]
    case = workloads.make_case(f"mk_nan_S{splits}{'_' + kv if kv else ''}", len(lens), lens,
                               dtype="bf16", block_size=16, seed=100 + splits,
                               max_blocks_per_seq=64, kv_dtype=kv)
    q, k, v, bt, cl = device_case(case)
    S, _ = pd.paged_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.max_blocks_per_seq,
                                case.block_size, torch.bfloat16, splits)
    print(case.describe(), "splits", splits, "S", S, flush=True)
    assert S > 1
    need = pd.paged_decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D,
                                           case.max_blocks_per_seq, case.block_size,
                                           torch.bfloat16, splits)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref, _ = oracle.attention_case(case)
    for rep in range(2):
        ws.fill_(0xFF)
        if kv:
            out = pd.paged_decode_attention_fp8(q, k, v, bt, cl, k_scale=case.k_scale,
                                                v_scale=case.v_scale, scale=case.scale,
                                                workspace=ws, num_splits=splits)
        else:
            out = pd.paged_decode_attention(q, k, v, bt, cl, scale=case.scale, workspace=ws,
                                            num_splits=splits)
        torch.cuda.synchronize()
        compare(out_bits(out), ref, "bf16", what=f"{case.name} rep {rep}")
